"""C-ABI checks that need no GPU: the library loads, exports every entry point
declared in include/simsd.h, and rejects bad arguments on the host before any
launch. Every call below returns before touching the HIP runtime: a case that
must pass a check stops at a later one (a missing workspace, a misaligned
pointer), so no call with these fake pointers ever reaches a launch."""
import ctypes
import os
import re

import pytest

from masked_attention_simsd_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "simsd.h")

FAKE = ctypes.c_void_p(0x100000)  # aligned, never dereferenced on these paths
MISALIGNED = ctypes.c_void_p(0x100008)


@pytest.fixture(autouse=True)
def no_launch_attempted():
    """Fails a test in which any call got as far as a kernel launch (on a
    machine without a GPU the launch fails and records its HIP error)."""
    ok = os.path.exists(binding.LIB_PATH)
    before = binding.load_library().simsd_last_hip_error() if ok else 0
    yield
    if ok:
        assert binding.load_library().simsd_last_hip_error() == before == 0, "a call reached a kernel launch"


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:int|size_t|const char\*)\s+(simsd_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        pytest.skip("libsimsd.so not built")
    return binding.load_library()


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert set(names) == set(binding.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code in range(12):
        assert lib.simsd_status_string(code)
    assert lib.simsd_status_string(0) == b"ok"


def _attn(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, kp=FAKE, vp=FAKE, off=FAKE, tau=FAKE, out=FAKE, lse=None,
             b=2, B=4, Hq=8, Hkv=2, d=128, maxp=100, scale=0.0, flags=0, status=None,
             ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return lib.simsd_verify_attention(a["q"], a["k"], a["v"], a["kp"], a["vp"], a["off"], a["tau"],
                                      a["out"], a["lse"], a["b"], a["B"], a["Hq"], a["Hkv"], a["d"],
                                      a["maxp"], a["scale"], a["flags"], a["status"], a["ws"],
                                      a["wsb"], None)


def test_attention_host_errors(lib):
    assert _attn(lib, q=None) == 1
    assert _attn(lib, kp=None) == 1
    assert _attn(lib, kp=None, vp=None, maxp=0, ws=None) == 6  # empty prefix needs no cache
    assert _attn(lib, b=0) == 2
    assert _attn(lib, B=65) == 2
    assert _attn(lib, B=0) == 2
    assert _attn(lib, maxp=-1) == 2
    assert _attn(lib, maxp=(1 << 30) + 1) == 2
    assert _attn(lib, Hq=6, Hkv=4) == 3
    assert _attn(lib, d=96) == 4
    assert _attn(lib, flags=3) == 5
    assert _attn(lib, flags=64) == 5
    # the paired K/V layout needs v_pre == k_pre + d elements
    assert _attn(lib, flags=binding.SIMSD_KV_PAIRED) == 5
    assert _attn(lib, flags=binding.SIMSD_KV_PAIRED, vp=ctypes.c_void_p(FAKE.value + 2 * 128), ws=None) == 6
    assert _attn(lib, scale=float("nan")) == 9
    assert _attn(lib, out=MISALIGNED) == 7
    assert _attn(lib, ws=None) == 6
    assert _attn(lib, ws=MISALIGNED) == 6
    need = lib.simsd_verify_attention_workspace(2, 4, 8, 2, 128, 100)
    assert need > 0
    assert _attn(lib, wsb=need - 1) == 6


def _attn_rope(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, kp=FAKE, vp=FAKE, off=FAKE, tau=FAKE, sp=FAKE, base=10000.0,
             rflags=0, krot=None, out=FAKE, lse=None, b=2, B=4, Hq=8, Hkv=2, d=128, maxp=100,
             scale=0.0, flags=0, status=None, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return lib.simsd_verify_attention_rope(a["q"], a["k"], a["v"], a["kp"], a["vp"], a["off"], a["tau"],
                                           a["sp"], a["base"], a["rflags"], a["krot"], a["out"], a["lse"],
                                           a["b"], a["B"], a["Hq"], a["Hkv"], a["d"], a["maxp"], a["scale"],
                                           a["flags"], a["status"], a["ws"], a["wsb"], None)


def test_fused_rope_attention_host_errors(lib):
    assert _attn_rope(lib, sp=None) == 1
    assert _attn_rope(lib, q=None) == 1
    assert _attn_rope(lib, rflags=8) == 5
    assert _attn_rope(lib, rflags=6) == 5  # explicit positions exclude the no-copy ablation
    assert _attn_rope(lib, rflags=4, ws=None) == 6  # accepted: stops at the workspace, the last check
    assert _attn_rope(lib, flags=3) == 5
    assert _attn_rope(lib, base=0.0) == 9
    assert _attn_rope(lib, base=float("nan")) == 9
    assert _attn_rope(lib, krot=MISALIGNED) == 7
    # the cos/sin table: (NO_COPY ? 2B : B) * d <= 8192
    assert _attn_rope(lib, B=33, rflags=2) == 2
    assert _attn_rope(lib, B=64, rflags=2, d=64, Hq=8, Hkv=2, ws=None) == 6
    # k_rot overlapping k_blk: [b][2B][Hkv][d] bf16 = 2*8*2*128*2 bytes
    assert _attn_rope(lib, krot=ctypes.c_void_p(0x100000 + 4096)) == 10
    assert _attn_rope(lib, krot=ctypes.c_void_p(0x100000 + 8192), ws=None) == 6
    assert lib.simsd_status_string(10)


def test_noalloc_attention_host_errors(lib):
    # the same argument checks as simsd_verify_attention, before any HIP call;
    # sizes whose workspace exceeds the fixed scratch buffer are refused
    f = lambda **kw: lib.simsd_verify_attention_noalloc(
        kw.get("q", FAKE), FAKE, FAKE, kw.get("kp", FAKE), FAKE, FAKE, FAKE, kw.get("out", FAKE), None,
        kw.get("b", 2), kw.get("B", 4), kw.get("Hq", 8), kw.get("Hkv", 2), kw.get("d", 128),
        kw.get("maxp", 100), 0.0, kw.get("flags", 0), None, None)
    assert f(q=None) == 1
    assert f(out=None) == 1
    assert f(b=0) == 2
    assert f(Hq=9) == 3
    assert f(d=96) == 4
    assert f(flags=3) == 5
    assert f(q=MISALIGNED) == 7
    # the split plan keeps partials near one workgroup per CU (16.5 MiB at
    # most for 8 sequences, B = 16, 32/8 heads); forcing 4096 workgroups asks
    # for far more than the fixed buffer
    big = dict(b=8, B=16, Hq=32, Hkv=8, maxp=16384)
    assert lib.simsd_verify_attention_workspace(8, 16, 32, 8, 128, 16384) <= binding.NOALLOC_SCRATCH_BYTES
    with binding.tuning(attn_target_wg=4096):
        assert lib.simsd_verify_attention_workspace(8, 16, 32, 8, 128, 16384) > binding.NOALLOC_SCRATCH_BYTES
        assert f(**big) == binding.SIMSD_ERR_SCRATCH
    assert lib.simsd_status_string(binding.SIMSD_ERR_SCRATCH) != b"unknown status"


def test_workspace_sizes(lib):
    assert lib.simsd_verify_attention_workspace(0, 4, 8, 2, 128, 100) == 0
    assert lib.simsd_verify_attention_workspace(1, 4, 8, 3, 128, 100) == 0
    assert lib.simsd_verify_attention_workspace(1, 4, 8, 2, 100, 100) == 0
    assert lib.simsd_verify_attention_workspace(1, 4, 8, 2, 128, -1) == 0
    assert lib.simsd_verify_attention_workspace(1, 4, 8, 2, 128, (1 << 30) + 1) == 0
    assert lib.simsd_verify_attention_workspace(1, 4, 8, 2, 128, 1 << 30) > 0
    for cfg in [(16, 8, 32, 8, 128, 4096), (8, 16, 32, 8, 128, 16384), (64, 8, 32, 8, 128, 8192),
                (1, 4, 1, 1, 64, 32), (1, 64, 32, 8, 128, 100)]:
        n = lib.simsd_verify_attention_workspace(*cfg)
        assert n % 256 == 0 and 0 < n < (1 << 31)
    n = lib.simsd_accept_workspace(16, 8, 32768)
    assert n >= 262144 + 16 * 8 * 8 and n % 256 == 0
    assert lib.simsd_accept_workspace(0, 8, 32768) == 0
    assert lib.simsd_accept_workspace(1, 65, 32768) == 0
    assert lib.simsd_accept_workspace(1, 8, 0) == 0


def test_tuning_is_explicit_and_changes_only_what_it_names(lib):
    # unknown keys and values below -1 are refused
    assert lib.simsd_set_tuning(-1, 0) == 2
    assert lib.simsd_set_tuning(9, 0) == 2
    assert lib.simsd_set_tuning(0, -2) == 2
    cfg = (16, 8, 32, 8, 128, 4096)
    base = lib.simsd_verify_attention_workspace(*cfg)
    # the environment is never read: setting a variable of the old tuning
    # scheme changes nothing
    os.environ["SIMSD_ATTN_TARGET_WG"] = "4096"
    try:
        assert lib.simsd_verify_attention_workspace(*cfg) == base
    finally:
        os.environ.pop("SIMSD_ATTN_TARGET_WG", None)
    # an explicit override does (more splits, more partials), and -1 restores it
    with binding.tuning(attn_target_wg=4096):
        assert lib.simsd_verify_attention_workspace(*cfg) > base
    assert lib.simsd_verify_attention_workspace(*cfg) == base


def test_rope_host_errors(lib):
    f = lambda **kw: lib.simsd_rope_copy(kw.get("q", FAKE), kw.get("k", FAKE), kw.get("sp", FAKE),
                                         kw.get("b", 1), kw.get("B", 4), kw.get("Hq", 8),
                                         kw.get("Hkv", 2), kw.get("d", 64),
                                         kw.get("base", 10000.0), kw.get("flags", 0), None)
    assert f(q=None) == 1
    assert f(sp=None) == 1
    assert f(B=65) == 2
    assert f(Hq=7) == 3
    assert f(d=32) == 4
    assert f(flags=8) == 5
    assert f(flags=6) == 5  # explicit positions exclude the no-copy ablation
    assert f(flags=4, k=MISALIGNED) == 7  # positions accepted: stops at the alignment check
    assert f(base=0.0) == 9
    assert f(base=float("inf")) == 9
    assert f(k=MISALIGNED) == 7


def test_accept_host_errors(lib):
    f = lambda **kw: lib.simsd_accept(kw.get("p", FAKE), kw.get("q", FAKE), FAKE, FAKE, FAKE,
                                      kw.get("b", 1), kw.get("B", 4), kw.get("V", 16),
                                      kw.get("L", FAKE), FAKE, None, kw.get("ws", FAKE),
                                      kw.get("wsb", 1 << 30), None)
    assert f(p=None) == 1
    assert f(L=None) == 1
    assert f(b=0) == 2
    assert f(B=65) == 2
    assert f(V=0) == 2
    assert f(V=(1 << 21) + 1) == 2
    assert f(q=MISALIGNED) == 7
    assert f(ws=None) == 6
    assert f(ws=MISALIGNED) == 6
    assert f(wsb=lib.simsd_accept_workspace(1, 4, 16) - 1) == 6


def test_accept_logits_host_errors(lib):
    f = lambda **kw: lib.simsd_accept_logits(kw.get("zt", FAKE), kw.get("zd", FAKE), kw.get("T", 1.0), FAKE,
                                             FAKE, FAKE, kw.get("b", 1), kw.get("B", 4), kw.get("V", 16),
                                             kw.get("L", FAKE), FAKE, None, kw.get("ws", FAKE),
                                             kw.get("wsb", 1 << 30), None)
    assert f(zt=None) == 1
    assert f(L=None) == 1
    assert f(b=0) == 2
    assert f(B=65) == 2
    assert f(V=(1 << 21) + 1) == 2
    assert f(T=0.0) == 9
    assert f(T=float("inf")) == 9
    assert f(zd=MISALIGNED) == 7
    assert f(ws=None) == 6
    assert f(wsb=lib.simsd_accept_logits_workspace(1, 4, 16) - 1) == 6
    n = lib.simsd_accept_logits_workspace(8, 16, 151936)
    assert n > lib.simsd_accept_workspace(8, 16, 151936) and n % 256 == 0
    assert lib.simsd_accept_logits_workspace(65536, 64, 1 << 21) == 0  # statistics units over 2^24
    # a statistics grid of 2^24 workgroups of 256 threads would be 2^32
    # work-items, one past a dispatch's limit: refused; one segment less fits
    assert lib.simsd_accept_logits_workspace(4096, 64, 32 * 4096) == 0
    assert lib.simsd_accept_logits_workspace(4096, 64, 31 * 4096) > 0


def test_attention_mask_host_errors(lib):
    def f(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, kp=FAKE, vp=FAKE, off=FAKE, m=FAKE, out=FAKE, lse=None, b=2, R=24,
                 Hq=8, Hkv=2, d=128, maxp=100, scale=0.0, flags=0, status=None, ws=FAKE, wsb=1 << 30)
        a.update(kw)
        return lib.simsd_verify_attention_mask(a["q"], a["k"], a["v"], a["kp"], a["vp"], a["off"], a["m"], a["out"],
                                               a["lse"], a["b"], a["R"], a["Hq"], a["Hkv"], a["d"], a["maxp"],
                                               a["scale"], a["flags"], a["status"], a["ws"], a["wsb"], None)
    assert f(m=None) == 1
    assert f(R=0) == 2
    assert f(R=129) == 2
    assert f(flags=1) == 5  # data-row rules do not apply
    assert f(m=ctypes.c_void_p(0x100004)) == 7
    assert f(Hq=6, Hkv=4) == 3
    assert f(ws=None) == 6
    assert f(wsb=lib.simsd_verify_attention_mask_workspace(2, 24, 8, 2, 128, 100) - 1) == 6
    assert lib.simsd_verify_attention_mask_workspace(2, 129, 8, 2, 128, 100) == 0


def test_commit_kv_host_errors(lib):
    def f(**kw):
        a = dict(k=FAKE, v=FAKE, tau=ctypes.c_void_p(0x200000), L=ctypes.c_void_p(0x300000), kc=FAKE, vc=FAKE,
                 off=ctypes.c_void_p(0x400000), lens=ctypes.c_void_p(0x400040), pos=None, nxt=None, b=4, B=8,
                 Hkv=2, d=128, flags=0, status=None)
        a.update(kw)
        return lib.simsd_commit_kv(a["k"], a["v"], a["tau"], a["L"], a["kc"], a["vc"], a["off"], a["lens"],
                                   a["pos"], a["nxt"], a["b"], a["B"], a["Hkv"], a["d"], a["flags"], a["status"],
                                   None)
    for name in ("k", "v", "tau", "L", "kc", "vc", "off", "lens"):
        assert f(**{name: None}) == 1, name
    assert f(b=0) == 2
    assert f(B=0) == 2
    assert f(B=65) == 2
    assert f(Hkv=0) == 2
    assert f(d=96) == 4
    assert f(flags=1) == 5
    assert f(flags=16) == 5
    assert f(kc=MISALIGNED) == 7
    assert f(k=MISALIGNED) == 7
    # the lengths may not be tau or accept_len (they are rewritten after every copy read them)
    assert f(lens=ctypes.c_void_p(0x200010)) == 10
    assert f(lens=ctypes.c_void_p(0x300000)) == 10
    assert f(lens=ctypes.c_void_p(0x400008)) == 10  # inside cache_offsets
    # next positions need this round's positions, may overwrite them in place,
    # and may not overlap any other input ([b][B] int32 = 128 bytes here)
    P0, N0 = ctypes.c_void_p(0x500000), ctypes.c_void_p(0x600000)
    assert f(nxt=N0) == 1
    # accepted: these stop at the alignment check, which follows the aliasing one
    assert f(pos=P0, nxt=N0, k=MISALIGNED) == 7
    assert f(pos=P0, nxt=P0, k=MISALIGNED) == 7
    assert f(pos=P0, nxt=ctypes.c_void_p(0x500040)) == 10
    assert f(pos=P0, nxt=ctypes.c_void_p(0x200040)) == 10  # over tau
    assert f(pos=P0, nxt=ctypes.c_void_p(0x3FFFF0)) == 10  # over cache_offsets
