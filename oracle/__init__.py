"""CPU oracle for the SimSD verification path -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the CPU-baseline leg of the benchmark
may import this package. The product path (the HIP library and its binding)
never does, and the two share no code.

The arithmetic lives in ``simsd_oracle.c`` (plain C, fp64 attention and RoPE,
fp32 accept/reject decisions); this module only marshals numpy arrays into it.
Every function cites the page section it follows in the C source.

Parity status of each function (what pins it, all in ``tests/test_oracle_*``):
  allowed / mask_matrix   pinned: hand-derived mask fixture, counting and
                          permutation invariants.
  verify_attention        pinned: library attention on explicitly gathered keys,
                          closed forms, perturbation and permutation invariance.
                          The rule for data-token rows is this build's reading
                          (the pages define only mask-slot rows): pinned only
                          to that stated reading.
  rope_copy               pinned: complex-number form, closed forms, relative-
                          position property, the copy rule.
  accept                  pinned: vocabulary-4 enumeration of acceptance and
                          residual laws, the lossless identity, special cases.
  attention_masked        pinned: equals verify_attention bit for bit on the
                          tau-derived mask; numpy softmax attention over
                          explicitly gathered keys for random masks; empty rows.
  softmax_rows            pinned: scipy's softmax, closed forms (uniform and
                          two-valued rows), exact shift and temperature
                          identities, the limits of large and small T.
  accept_logits           softmax_rows then accept (both pinned), plus the
                          decision margins a differently rounded softmax may
                          cross (ratio_boundary).
  next_positions / committed_positions
                          integer bookkeeping of the round loop: pinned by
                          closed forms (L = 0, L = B, identity order), the
                          B smallest uncached positions found by brute force,
                          and over several rounds with partial acceptance the
                          committed and next-round positions covering a
                          contiguous range exactly once.
  commit_kv / pack_regions
                          pure row movement (numpy indexing, no arithmetic):
                          pinned by closed forms (identity and reversed tau,
                          L = 0 and L = B), one-token-at-a-time appends, the
                          untouched rest of the cache, the overflow and bad-tau
                          cases, and by the context property -- the first
                          rejected data row attends over the committed cache to
                          the same result it had in the round that rejected it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "simsd_oracle.c")
LIB = os.path.join(HERE, "libsimsd_oracle.so")

DATA_CAUSAL, DATA_BIDIR, DATA_SKIP = 0, 1, 2
# per-sequence status bits of commit_kv
BAD_TAU, COMMIT_OVERFLOW = 1, 64

_lib = None


def compile_source(src: str, out: str) -> None:
    """gcc -O2, no fast-math, no FMA contraction: the one way the oracle is built."""
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
                           "-fno-fast-math", src, "-o", out, "-lm"])


def build(force: bool = False) -> str:
    """Compile the oracle (only when the source is newer than the library)."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp%d" % os.getpid()
        compile_source(SRC, tmp)
        os.replace(tmp, LIB)
    return LIB


# The test of the pins themselves (tests/test_oracle_mutants.py) runs the pin
# tests against copies of the oracle with one planted mistake each; such a copy
# is loaded from the path in this variable instead of the library built here.
MUTANT_ENV = "SIMSD_ORACLE_MUTANT_LIB"


def _load():
    global _lib
    if _lib is None:
        path = os.environ.get(MUTANT_ENV) or build()
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        I = ctypes.c_int
        D = ctypes.c_double
        lib.simsd_oracle_tau_inverse.argtypes = [P, I, P]
        lib.simsd_oracle_tau_inverse.restype = I
        lib.simsd_oracle_allowed.argtypes = [I, P, I, I, I]
        lib.simsd_oracle_allowed.restype = I
        lib.simsd_oracle_attention_row.argtypes = [P, P, P, I, P, P, P, I, I, I, I, I, D, I, P, P]
        lib.simsd_oracle_attention_row.restype = None
        lib.simsd_oracle_verify_attention.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, D, I, P, P]
        lib.simsd_oracle_verify_attention.restype = I
        lib.simsd_oracle_rope_copy.argtypes = [P, P, P, I, I, I, I, D, I, I]
        lib.simsd_oracle_rope_copy.restype = None
        lib.simsd_oracle_accept.argtypes = [P, P, P, P, P, I, I, I, P, P, P, P]
        lib.simsd_oracle_accept.restype = None
        lib.simsd_oracle_softmax_rows.argtypes = [P, I, I, D, P]
        lib.simsd_oracle_softmax_rows.restype = None
        lib.simsd_oracle_attention_masked.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, D, P, P]
        lib.simsd_oracle_attention_masked.restype = None
        _lib = lib
    return _lib


def _f64(a) -> np.ndarray:
    a = np.asarray(a, dtype=np.float64)
    return np.ascontiguousarray(a)


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32))


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def tau_inverse(tau):
    """Return (inv, ok): inv[t-1] = 0-based position with label t."""
    t = _i32(tau)
    inv = np.empty(t.shape[0], dtype=np.int32)
    bad = _load().simsd_oracle_tau_inverse(_p(t), t.shape[0], _p(inv))
    return inv, bad == 0


def allowed(B: int, tau, data_rule: int, qr: int, kr: int) -> bool:
    t = _i32(tau)
    return bool(_load().simsd_oracle_allowed(B, _p(t), data_rule, qr, kr))


def mask_matrix(tau, data_rule: int = DATA_CAUSAL) -> np.ndarray:
    """[2B][2B] boolean block mask (row = query block row, col = key block row)."""
    t = _i32(tau)
    B = t.shape[0]
    lib = _load()
    m = np.zeros((2 * B, 2 * B), dtype=bool)
    for i in range(2 * B):
        for j in range(2 * B):
            m[i, j] = bool(lib.simsd_oracle_allowed(B, _p(t), data_rule, i, j))
    return m


def attention_row(q_row, k_pre_s, v_pre_s, k_blk_s, v_blk_s, tau_s, g: int, qr: int,
                  scale: float | None = None, data_rule: int = DATA_CAUSAL):
    """One query row. k_pre_s/v_pre_s [P][Hkv][d], k_blk_s/v_blk_s [2B][Hkv][d]."""
    q = _f64(q_row)
    kp, vp, kb, vb = _f64(k_pre_s), _f64(v_pre_s), _f64(k_blk_s), _f64(v_blk_s)
    t = _i32(tau_s)
    d = q.shape[0]
    Hkv = kb.shape[1]
    B = t.shape[0]
    P = kp.shape[0]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    out = np.empty(d, dtype=np.float64)
    lse = np.empty(1, dtype=np.float64)
    _load().simsd_oracle_attention_row(_p(q), _p(kp), _p(vp), P, _p(kb), _p(vb), _p(t), B, Hkv, d,
                                       g, qr, float(scale), data_rule, _p(out), _p(lse))
    return out, float(lse[0])


def verify_attention(q_blk, k_blk, v_blk, k_pre, v_pre, prefix_offsets, tau,
                     scale: float | None = None, data_rule: int = DATA_CAUSAL,
                     threads: int = 1):
    """Whole-batch verify attention. Returns (out [b][2B][Hq][d], lse [b][2B][Hq]) in fp64.

    Rows skipped under DATA_SKIP are left as NaN. ``threads`` > 1 runs
    sequences concurrently (the C call releases the GIL); results do not depend
    on it.
    """
    q, kb, vb = _f64(q_blk), _f64(k_blk), _f64(v_blk)
    kp, vp = _f64(k_pre), _f64(v_pre)
    off = _i32(prefix_offsets)
    t = _i32(tau)
    b, twoB, Hq, d = q.shape
    Hkv = kb.shape[2]
    B = twoB // 2
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    out = np.full(q.shape, np.nan)
    lse = np.full((b, twoB, Hq), np.nan)
    lib = _load()

    def one(s):
        o0 = int(off[s])
        P = int(off[s + 1]) - o0
        offs = np.array([0, P], dtype=np.int32)
        kps = np.ascontiguousarray(kp[o0:o0 + P])
        vps = np.ascontiguousarray(vp[o0:o0 + P])
        os_ = np.ascontiguousarray(out[s:s + 1])
        ls_ = np.ascontiguousarray(lse[s:s + 1])
        bad = lib.simsd_oracle_verify_attention(
            _p(np.ascontiguousarray(q[s:s + 1])), _p(np.ascontiguousarray(kb[s:s + 1])),
            _p(np.ascontiguousarray(vb[s:s + 1])), _p(kps), _p(vps), _p(offs),
            _p(np.ascontiguousarray(t[s:s + 1])), 1, B, Hq, Hkv, d, float(scale), data_rule,
            _p(os_), _p(ls_))
        out[s] = os_[0]
        lse[s] = ls_[0]
        return bad

    if threads > 1 and b > 1:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(one, range(b)))
    else:
        for s in range(b):
            one(s)
    return out, lse


def rope_copy(x, start_pos, base: float = 10000.0, interleaved: bool = False,
              no_copy: bool = False) -> np.ndarray:
    """Rotated copy of x [b][2B][H][d] (fp64). start_pos is [b] (D_k and D~_k
    at start_pos[s] + k - 1) or [b][B] (explicit positions: D_k and D~_k at
    start_pos[s][k-1])."""
    y = _f64(x).copy()
    sp = _i32(start_pos)
    b, twoB, H, d = y.shape
    if sp.ndim == 2:
        if no_copy:
            raise ValueError("the no-copy ablation takes consecutive positions only")
        if sp.shape != (b, twoB // 2):
            raise ValueError("positions must be [b][B]")
        _load().simsd_oracle_rope_copy(_p(y), None, _p(sp), b, twoB // 2, H, d, float(base),
                                       int(bool(interleaved)), 0)
    else:
        _load().simsd_oracle_rope_copy(_p(y), _p(sp), None, b, twoB // 2, H, d, float(base),
                                       int(bool(interleaved)), int(bool(no_copy)))
    return y


def accept(p, q, draft, tau, u):
    """Rejection-sampling acceptance. Returns dict of int32 arrays [b]:
    accept_len, correction, status, boundary."""
    pp, qq = _f32(p), _f32(q)
    dr, t, uu = _i32(draft), _i32(tau), _f32(u)
    b, B, V = pp.shape
    out = {k: np.zeros(b, dtype=np.int32) for k in ("accept_len", "correction", "status", "boundary")}
    _load().simsd_oracle_accept(_p(pp), _p(qq), _p(dr), _p(t), _p(uu), b, B, V,
                                _p(out["accept_len"]), _p(out["correction"]), _p(out["status"]),
                                _p(out["boundary"]))
    return out


def softmax_rows(z, temperature=1.0):
    """Row softmax of fp32 logits at a temperature, fp64 arithmetic, fp32 out
    (same shape as z; the last axis is the vocabulary)."""
    zz = _f32(z)
    V = zz.shape[-1]
    rows = zz.size // V if V else 0
    out = np.zeros_like(zz)
    _load().simsd_oracle_softmax_rows(_p(zz), rows, V, float(temperature), _p(out))
    return out


def accept_logits(zt, zd, temperature, draft, tau, u, ratio_eps=4.0):
    """Acceptance from target / draft logits: p = softmax(zt / T), q =
    softmax(zd / T) (softmax_rows), then accept(p, q, ...). Adds
    ratio_boundary[s] = 1 when an examined step's uniform lies within
    ratio_eps fp32 ulps of its ratio min(1, p/q): a softmax rounded
    differently in the last place may decide that step the other way."""
    p = softmax_rows(zt, temperature)
    q = softmax_rows(zd, temperature)
    out = accept(p, q, draft, tau, u)
    b, B, V = p.shape
    tau_i = _i32(tau)
    dr = _i32(draft)
    uu = _f32(u)
    rb = np.zeros(b, dtype=np.int32)
    for s in range(b):
        if out["status"][s] & 1:
            continue
        inv = np.argsort(tau_i[s])
        L = int(out["accept_len"][s])
        for t in range(min(L + 1, B)):
            k = inv[t]
            x = int(dr[s, k])
            if x < 0 or x >= V:
                continue
            a, c = p[s, k, x], q[s, k, x]
            r = np.float32(min(np.float32(1.0), a / c)) if c > 0 else np.float32(1.0 if a > 0 else 0.0)
            if abs(float(uu[s, t]) - float(r)) <= ratio_eps * float(np.spacing(np.float32(max(r, 1e-30)))):
                rb[s] = 1
    out["ratio_boundary"] = rb
    out["p"], out["q"] = p, q
    return out


def attention_masked(q_blk, k_blk, v_blk, k_pre, v_pre, prefix_offsets, allowed, scale=None):
    """Block rows under an explicit mask: allowed [b][R][R] (bool; row r may
    see block key c), plus the whole cached prefix. Returns (out, lse) fp64;
    rows with no visible key give out 0, lse -inf."""
    q, kb, vb = _f64(q_blk), _f64(k_blk), _f64(v_blk)
    kp, vp = _f64(k_pre), _f64(v_pre)
    off = _i32(prefix_offsets)
    al = np.ascontiguousarray(np.asarray(allowed, dtype=np.uint8))
    b, R, Hq, d = q.shape
    Hkv = kb.shape[2]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    out = np.zeros(q.shape)
    lse = np.zeros((b, R, Hq))
    _load().simsd_oracle_attention_masked(_p(q), _p(kb), _p(vb), _p(kp), _p(vp), _p(off), _p(al), b, R,
                                          Hq, Hkv, d, float(scale), _p(out), _p(lse))
    return out, lse


def pack_regions(cache, offsets, lens, head_major: bool = False):
    """The packed prefix (cumulative-offset layout) of a cache that gives every
    sequence a region of rows [offsets[s], offsets[s+1]) of which the first
    lens[s] are in use. cache is [C][Hkv][d] (or [Hkv][C][d] with head_major).
    Returns (packed [sum lens][Hkv][d] or [Hkv][sum lens][d], packed_offsets)."""
    c = np.asarray(cache)
    off = _i32(offsets)
    ln = _i32(lens)
    b = ln.shape[0]
    rows = [np.arange(off[s], off[s] + ln[s]) for s in range(b)]
    idx = np.concatenate(rows) if b else np.zeros(0, dtype=np.int64)
    packed = c[:, idx] if head_major else c[idx]
    po = np.zeros(b + 1, dtype=np.int32)
    po[1:] = np.cumsum(ln)
    return packed, po


def next_positions(pos, tau, accept_len):
    """Response positions of the next round of each sequence ([nl]/[fr]
    Methodologie 1 and 4: each pair (D_k, D~_k) is one response position;
    the longest prefix accepted along the temporal order is committed and the
    round repeats over what is still open).

    pos [b][B] holds the positions this round verified, tau [b][B] its step
    labels, accept_len [b] the accepted lengths L. The drafts at tau^-1(1..L)
    enter the cache; the next round verifies the B smallest positions not in
    the cache: when L < B, first the position tau^-1(L+1), whose correction
    token is committed but has no key/value row yet (the next round computes
    it, as that round's data token at temporal step 1), then the other open
    positions tau^-1(L+2..B) in increasing order, then L positions following
    the largest one of this block. A sequence whose tau is not a permutation or
    whose L is outside 0..B commits nothing and keeps its block.

    Returns next [b][B] int32."""
    ps, t, L_all = _i32(pos), _i32(tau), _i32(accept_len)
    b, B = t.shape
    nxt = ps.copy()
    for s in range(b):
        inv, ok = tau_inverse(t[s])
        L = int(L_all[s])
        if not ok or L < 0 or L > B:
            continue
        frontier = int(ps[s].max()) + 1
        row = []
        if L < B:
            row.append(int(ps[s, inv[L]]))  # the correction's position
            row += sorted(int(ps[s, inv[j]]) for j in range(L + 1, B))
        row += [frontier + i for i in range(L)]
        nxt[s] = row
    return nxt


def committed_positions(pos, tau, accept_len):
    """The positions whose key/value rows a commit appends, per sequence, in
    temporal order: pos[s][tau^-1(t)] for t = 1..L (empty for a sequence that
    commits nothing)."""
    ps, t, L_all = _i32(pos), _i32(tau), _i32(accept_len)
    out = []
    for s in range(t.shape[0]):
        inv, ok = tau_inverse(t[s])
        L = int(L_all[s])
        out.append([int(ps[s, inv[j]]) for j in range(L)] if ok and 0 <= L <= t.shape[1] else [])
    return out


def commit_kv(k_blk, v_blk, tau, accept_len, k_cache, v_cache, cache_offsets, cache_lens,
              head_major: bool = False):
    """Commit the accepted drafts of one verification round to the KV cache
    ([nl]/[fr] Methodologie 4, Acceptance / Acceptation: the longest prefix
    accepted along the temporal order is committed and the round repeats).

    Sequence s accepted its first L = accept_len[s] drafts in temporal order:
    the data tokens D_k with tau(k) <= L. Their key and value rows (block rows
    k - 1 < B of k_blk / v_blk [b][2B][Hkv][d], already rotated at their own
    positions) are written, in temporal order t = 1..L (k = tau^-1(t)), to rows
    cache_lens[s] + t - 1 of the sequence's region [cache_offsets[s],
    cache_offsets[s+1]) of k_cache / v_cache ([C][Hkv][d], or [Hkv][C][d] with
    head_major), and the sequence's used length becomes cache_lens[s] + L.
    Nothing of sequence s is written, and its length is kept, when tau[s] is not
    a permutation (status BAD_TAU) or when L is outside 0..B, the length is
    negative, or the region cannot hold L more rows (COMMIT_OVERFLOW).

    Returns (k_cache', v_cache', lens', status[b]) as new arrays.
    """
    kb, vb = np.asarray(k_blk), np.asarray(v_blk)
    kc, vc = np.array(k_cache, copy=True), np.array(v_cache, copy=True)
    off = _i32(cache_offsets)
    ln = _i32(cache_lens).copy()
    t = _i32(tau)
    L_all = _i32(accept_len)
    b, B = t.shape
    status = np.zeros(b, dtype=np.int32)
    for s in range(b):
        inv, ok = tau_inverse(t[s])
        if not ok:
            status[s] |= BAD_TAU
            continue
        L = int(L_all[s])
        cap = int(off[s + 1]) - int(off[s])
        if L < 0 or L > B or ln[s] < 0 or int(ln[s]) + L > cap:
            status[s] |= COMMIT_OVERFLOW
            continue
        for step in range(L):
            k = int(inv[step])  # 0-based position of the draft with label step + 1
            row = int(off[s]) + int(ln[s]) + step
            if head_major:
                kc[:, row] = kb[s, k]
                vc[:, row] = vb[s, k]
            else:
                kc[row] = kb[s, k]
                vc[row] = vb[s, k]
        ln[s] += L
    return kc, vc, ln, status
