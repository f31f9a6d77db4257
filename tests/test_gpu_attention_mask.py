"""Attention under an explicit block mask (simsd_verify_attention_mask) on the
GPU: the tau rule written as a mask gives exactly the tau kernel's bits, and
random / tree-shaped masks (draft graphs) match the oracle within the
attention tolerance."""
import numpy as np
import pytest
import torch

import oracle
from masked_attention_simsd_amd import binding, synth
from gpu_util import f64, pack_mask, say, to_dev

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2
TOL_F32 = 4e-3


def run_mask(x, allowed, flags=0):
    g = to_dev(x)
    b, R, Hq, _ = x["q_blk"].shape
    lens = x["prefix_offsets"][1:] - x["prefix_offsets"][:-1]
    lse = torch.full((b, R, Hq), float("nan"), device="cuda")
    out = binding.simsd_verify_attention_mask(g["q_blk"], g["k_blk"], g["v_blk"], g["k_pre"], g["v_pre"],
                                              g["prefix_offsets"], pack_mask(allowed).cuda(), lse=lse,
                                              max_prefix=int(lens.max()), flags=flags)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("shape", [(3, 8, 2, 128, 8, (100, 700)), (2, 32, 8, 128, 16, (1000, 2500)),
                                   (2, 4, 1, 64, 5, (0, 70)), (1, 32, 8, 128, 64, (300, 300))])
def test_tau_as_mask_is_bit_identical(shape):
    b, Hq, Hkv, d, B, pre = shape
    say(f"mask = tau rule {shape}")
    w = synth.custom(b=b, Hq=Hq, Hkv=Hkv, d=d, B=B, prefix=pre)
    x = synth.make_inputs(w, with_accept=False, seed=hash(shape) % 1000)
    g = to_dev(x)
    lse_t = torch.full((b, 2 * B, Hq), float("nan"), device="cuda")
    ref = binding.simsd_verify_attention(g["q_blk"], g["k_blk"], g["v_blk"], g["k_pre"], g["v_pre"],
                                         g["prefix_offsets"], g["tau"], lse=lse_t, max_prefix=pre[1])
    allowed = np.stack([oracle.mask_matrix(t) for t in x["tau"].numpy()])
    out, lse = run_mask(x, allowed)
    assert torch.equal(out, ref) and torch.equal(lse, lse_t)


def random_case(b, R, Hq, Hkv, d, pre, seed, density=0.5):
    w = synth.custom(b=b, Hq=Hq, Hkv=Hkv, d=d, B=1, prefix=pre)
    x = synth.make_inputs(w, with_accept=False, seed=seed)
    gen = torch.Generator().manual_seed(seed)
    rnd = lambda *shape: (torch.randn(shape, generator=gen)).to(torch.bfloat16)
    x["q_blk"], x["k_blk"], x["v_blk"] = rnd(b, R, Hq, d), rnd(b, R, Hkv, d), rnd(b, R, Hkv, d)
    allowed = np.random.default_rng(seed).random((b, R, R)) < density
    return x, allowed


@pytest.mark.parametrize("R", [1, 5, 37, 64, 100, 128])
def test_random_masks_match_oracle(R):
    say(f"random mask R={R}")
    x, allowed = random_case(3, R, 16, 4, 128, (0, 900), seed=R)
    ref, ref_lse = oracle.attention_masked(f64(x["q_blk"]), f64(x["k_blk"]), f64(x["v_blk"]), f64(x["k_pre"]),
                                           f64(x["v_pre"]), x["prefix_offsets"].numpy(), allowed)
    out, lse = run_mask(x, allowed, binding.SIMSD_OUT_F32)
    fin = np.isfinite(ref_lse)
    err = float(np.abs(f64(out) - ref).max())
    lerr = float(np.abs(f64(lse)[fin] - ref_lse[fin]).max()) if fin.any() else 0.0
    say(f"  fp32 out max-abs {err:.3e}, lse {lerr:.3e}, empty rows {int((~fin).sum())}")
    assert err <= TOL_F32 and lerr <= 2e-3
    assert np.all(f64(lse)[~fin] == -np.inf)
    out, _ = run_mask(x, allowed, 0)
    assert float(np.abs(f64(out) - ref).max()) <= TOL_BF16


def test_draft_tree_mask_head_major():
    # a draft graph: rows form a tree, each row sees itself and its ancestors
    rng = np.random.default_rng(3)
    b, R = 4, 48
    parent = np.array([-1] + [int(rng.integers(0, i)) for i in range(1, R)])
    allowed = np.zeros((b, R, R), bool)
    for r in range(R):
        a = r
        while a >= 0:
            allowed[:, r, a] = True
            a = parent[a]
    x, _ = random_case(b, R, 32, 8, 128, (200, 3000), seed=77)
    say("draft-tree mask, head-major cache")
    ref, _ = oracle.attention_masked(f64(x["q_blk"]), f64(x["k_blk"]), f64(x["v_blk"]), f64(x["k_pre"]),
                                     f64(x["v_pre"]), x["prefix_offsets"].numpy(), allowed)
    y = dict(x)
    y["k_pre"] = x["k_pre"].transpose(0, 1).contiguous()
    y["v_pre"] = x["v_pre"].transpose(0, 1).contiguous()
    out, _ = run_mask(y, allowed, binding.SIMSD_KV_HEAD_MAJOR | binding.SIMSD_OUT_F32)
    err = float(np.abs(f64(out) - ref).max())
    say(f"  max-abs {err:.3e}")
    assert err <= TOL_F32


def test_empty_rows_and_zero_prefix():
    # sequence 0 has no prefix; rows 0 and 7 of it see nothing -> 0 output, -inf lse.
    # sequence 1 has a prefix, so its fully masked rows still attend to the prefix.
    b, R = 2, 9
    w = synth.custom(b=b, Hq=8, Hkv=2, d=128, B=1, prefix=(0, 0))
    x = synth.make_inputs(w, with_accept=False, seed=5)
    lens = np.array([0, 300])
    x["prefix_offsets"] = torch.tensor([0, 0, 300], dtype=torch.int32)
    gen = torch.Generator().manual_seed(5)
    rnd = lambda *shape: torch.randn(shape, generator=gen).to(torch.bfloat16)
    x["k_pre"], x["v_pre"] = rnd(int(lens.sum()), 2, 128), rnd(int(lens.sum()), 2, 128)
    x["q_blk"], x["k_blk"], x["v_blk"] = rnd(b, R, 8, 128), rnd(b, R, 2, 128), rnd(b, R, 2, 128)
    allowed = np.tril(np.ones((R, R), bool))[None].repeat(b, 0)
    allowed[:, 0, :] = False
    allowed[:, 7, :] = False
    say("empty rows, zero prefix")
    ref, ref_lse = oracle.attention_masked(f64(x["q_blk"]), f64(x["k_blk"]), f64(x["v_blk"]), f64(x["k_pre"]),
                                           f64(x["v_pre"]), x["prefix_offsets"].numpy(), allowed)
    assert np.all(ref_lse[0, [0, 7]] == -np.inf) and np.all(np.isfinite(ref_lse[1]))
    for flags in (binding.SIMSD_OUT_F32, 0):
        out, lse = run_mask(x, allowed, flags)
        o = f64(out)
        assert np.all(o[0, [0, 7]] == 0.0)
        assert np.all(f64(lse)[0, [0, 7]] == -np.inf)
        fin = np.isfinite(ref_lse)
        assert np.abs(f64(lse)[fin] - ref_lse[fin]).max() <= 2e-3
        assert np.abs(o - ref).max() <= (TOL_F32 if flags else TOL_BF16)
