"""The paired K/V cache layout (SIMSD_KV_PAIRED): the key row and the value
row of each (token, KV head) sit next to each other in one buffer
([..][..][2][d]). Attention over such a cache gives bit for bit what it gives
over the same values held in two tensors (tau rule, fused RoPE, explicit
mask; token-major and head-major), and the KV commit into a paired cache
writes exactly the rows and lengths it writes into two tensors."""
import numpy as np
import pytest
import torch

from masked_attention_simsd_amd import binding, synth
from gpu_util import say, to_dev

pytestmark = pytest.mark.gpu


def paired(k, v):
    kv = torch.stack([k, v], dim=2).contiguous()
    return (kv,) + binding.kv_pair_views(kv)


@pytest.mark.parametrize("shape", [(3, 32, 8, 128, 8, (0, 2100)), (2, 4, 1, 64, 5, (40, 700))])
@pytest.mark.parametrize("head_major", [False, True])
def test_attention_paired_equals_two_tensors(shape, head_major):
    b, Hq, Hkv, d, B, pre = shape
    say(f"paired attention {shape} head_major={head_major}")
    w = synth.custom(b=b, Hq=Hq, Hkv=Hkv, d=d, B=B, prefix=pre)
    x = synth.make_inputs(w, with_accept=False, seed=21)
    g = to_dev(x)
    k, v = g["k_pre"], g["v_pre"]
    if head_major:
        k, v = k.transpose(0, 1).contiguous(), v.transpose(0, 1).contiguous()
    kv, kp, vp = paired(k, v)
    hm = binding.SIMSD_KV_HEAD_MAJOR if head_major else 0
    mp = int(x["prefix_lens"].max())
    for rule in (binding.SIMSD_DATA_CAUSAL, binding.SIMSD_DATA_BIDIR):
        lse_r = torch.zeros(g["q_blk"].shape[:3], device="cuda")
        lse_p = torch.zeros_like(lse_r)
        ref = binding.simsd_verify_attention(g["q_blk"], g["k_blk"], g["v_blk"], k, v, g["prefix_offsets"],
                                             g["tau"], lse=lse_r, max_prefix=mp, flags=hm | rule)
        got = binding.simsd_verify_attention(g["q_blk"], g["k_blk"], g["v_blk"], kp, vp, g["prefix_offsets"],
                                             g["tau"], lse=lse_p, max_prefix=mp,
                                             flags=hm | rule | binding.SIMSD_KV_PAIRED)
        torch.cuda.synchronize()
        assert torch.equal(got, ref) and torch.equal(lse_p, lse_r), f"rule {rule}"
    # fused RoPE
    kr_r, kr_p = torch.zeros_like(g["k_blk"]), torch.zeros_like(g["k_blk"])
    ref = binding.simsd_verify_attention_rope(g["q_blk"], g["k_blk"], g["v_blk"], k, v, g["prefix_offsets"],
                                              g["tau"], g["start_pos"], 10000.0, k_rot=kr_r, max_prefix=mp,
                                              flags=hm)
    got = binding.simsd_verify_attention_rope(g["q_blk"], g["k_blk"], g["v_blk"], kp, vp, g["prefix_offsets"],
                                              g["tau"], g["start_pos"], 10000.0, k_rot=kr_p, max_prefix=mp,
                                              flags=hm | binding.SIMSD_KV_PAIRED)
    torch.cuda.synchronize()
    assert torch.equal(got, ref) and torch.equal(kr_p, kr_r), "fused"
    # explicit block mask (a random one over the 2B block rows)
    R = 2 * B
    gen = torch.Generator().manual_seed(5)
    bits = torch.randint(0, 2, (b, R, R), generator=gen, dtype=torch.int64)
    words = torch.zeros(b, R, (R + 63) // 64, dtype=torch.int64)
    for c in range(R):
        words[:, :, c // 64] |= bits[:, :, c] << (c % 64)
    words = words.cuda()
    ref = binding.simsd_verify_attention_mask(g["q_blk"], g["k_blk"], g["v_blk"], k, v, g["prefix_offsets"],
                                              words, max_prefix=mp, flags=hm)
    got = binding.simsd_verify_attention_mask(g["q_blk"], g["k_blk"], g["v_blk"], kp, vp, g["prefix_offsets"],
                                              words, max_prefix=mp, flags=hm | binding.SIMSD_KV_PAIRED)
    torch.cuda.synchronize()
    assert torch.equal(got, ref), "mask"


@pytest.mark.parametrize("head_major", [False, True])
def test_commit_paired_equals_two_tensors(head_major):
    b, B, Hkv, d = 4, 8, 8, 128
    say(f"paired commit head_major={head_major}")
    rng = np.random.default_rng(3)
    lens = rng.integers(0, 40, size=b).astype(np.int32)
    caps = lens + rng.integers(0, B + 3, size=b)
    off = np.zeros(b + 1, np.int32)
    off[1:] = np.cumsum(caps)
    C = int(off[-1])
    gen = torch.Generator().manual_seed(9)
    kb = torch.randn(b, 2 * B, Hkv, d, generator=gen).to(torch.bfloat16).cuda()
    vb = torch.randn(b, 2 * B, Hkv, d, generator=gen).to(torch.bfloat16).cuda()
    shape_c = (Hkv, C, d) if head_major else (C, Hkv, d)
    kc = torch.randn(*shape_c, generator=gen).to(torch.bfloat16).cuda()
    vc = torch.randn(*shape_c, generator=gen).to(torch.bfloat16).cuda()
    kv, kp, vp = paired(kc, vc)
    tau = torch.from_numpy(np.stack([rng.permutation(B) + 1 for _ in range(b)]).astype(np.int32)).cuda()
    L = torch.from_numpy(rng.integers(0, B + 1, size=b).astype(np.int32)).cuda()
    hm = binding.SIMSD_KV_HEAD_MAJOR if head_major else 0
    ext_r = torch.tensor(np.concatenate([off, lens]), dtype=torch.int32, device="cuda")
    ext_p = ext_r.clone()
    st_r = torch.zeros(b, dtype=torch.int32, device="cuda")
    st_p = torch.zeros_like(st_r)
    binding.simsd_commit_kv(kb, vb, tau, L, kc, vc, ext_r[:b + 1], ext_r[b + 1:], flags=hm, status=st_r)
    binding.simsd_commit_kv(kb, vb, tau, L, kp, vp, ext_p[:b + 1], ext_p[b + 1:],
                            flags=hm | binding.SIMSD_KV_PAIRED, status=st_p)
    torch.cuda.synchronize()
    assert torch.equal(ext_p, ext_r) and torch.equal(st_p, st_r)
    assert torch.equal(kv[:, :, 0], kc) and torch.equal(kv[:, :, 1], vc)


def test_paired_views_are_checked():
    kv = torch.zeros(10, 2, 2, 64, dtype=torch.bfloat16, device="cuda")
    kp, vp = binding.kv_pair_views(kv)
    q = torch.zeros(1, 2, 2, 64, dtype=torch.bfloat16, device="cuda")
    kb = torch.zeros(1, 2, 2, 64, dtype=torch.bfloat16, device="cuda")
    off = torch.tensor([0, 10], dtype=torch.int32, device="cuda")
    tau = torch.ones(1, 1, dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):  # halves swapped
        binding.simsd_verify_attention(q, kb, kb, vp, kp, off, tau, max_prefix=10,
                                       flags=binding.SIMSD_KV_PAIRED)
