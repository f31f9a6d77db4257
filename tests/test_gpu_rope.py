"""RoPE-copy on the GPU against the oracle (bf16 outputs vs the oracle's fp64
rotation rounded once to bf16)."""
import zlib

import numpy as np
import pytest
import torch

import oracle
from masked_attention_simsd_amd import binding, synth
from gpu_util import bf16_round, bf16_ulp, f64, inputs, say

pytestmark = pytest.mark.gpu


def angle_slack(x, positions, base, interleaved=False):
    """Per-element absolute slack from the fp64 angle itself: an angle A is
    only known to about one fp64 ulp (2^-52 A), and the device's sin / cos of
    angles of 1e9 rad and more behave like an argument moved by about that
    much, so a rotated pair (x_a, x_b) may move by 4 * 2^-52 * A * (|x_a| +
    |x_b|). Below ~1e6 rad this is far under a bf16 ulp; it matters only where
    the rotation cancels to an output much smaller than its inputs.
    x [b][2B][H][d], positions [b][B] (or [b], consecutive)."""
    x = np.asarray(x, dtype=np.float64)
    b, twoB, H, d = x.shape
    B, half = twoB // 2, d // 2
    pos = np.asarray(positions, dtype=np.float64)
    if pos.ndim == 1:
        pos = pos[:, None] + np.arange(B)[None, :]
    freq = base ** (-2.0 * np.arange(half) / d)
    e = np.arange(d)
    i = e // 2 if interleaved else e % half
    mate = (e ^ 1) if interleaved else (e + half) % d
    ang = np.abs(pos[:, np.r_[0:B, 0:B]][:, :, None, None] * freq[i][None, None, None, :])
    return 4.0 * 2.0 ** -52 * ang * (np.abs(x) + np.abs(x[..., mate]))


def _check(gpu, ref_f64, what, slack=None):
    ref = bf16_round(ref_f64)
    got = f64(gpu)
    diff = np.abs(got - ref)
    exact = float(np.mean(diff == 0))
    bound = bf16_ulp(ref) if slack is None else np.maximum(bf16_ulp(ref), slack)
    ulps = float((diff / bf16_ulp(ref)).max())
    over = float((diff / bound).max())
    say(f"  {what}: exact {exact:.6f}, max {ulps:.2f} ulp, max {over:.2f} of the bound")
    assert over <= 1.0, what
    assert exact >= 0.9999, what


@pytest.mark.parametrize("cfg", ["tiny", "b4", "b8", "b16", "ragged"])
@pytest.mark.parametrize("flags", [0, binding.SIMSD_ROPE_INTERLEAVED, binding.SIMSD_ROPE_NO_COPY])
def test_rope_copy_matches_oracle(cfg, flags):
    say(f"rope {cfg} flags={flags}")
    x = inputs(cfg)
    w = x["workload"]
    q = x["q_blk"].cuda()
    k = x["k_blk"].cuda()
    binding.simsd_rope_copy(q, k, x["start_pos"].cuda(), w.rope_base, flags)
    torch.cuda.synchronize()
    kw = dict(base=w.rope_base, interleaved=bool(flags & 1), no_copy=bool(flags & 2))
    _check(q, oracle.rope_copy(f64(x["q_blk"]), x["start_pos"].numpy(), **kw), "q")
    _check(k, oracle.rope_copy(f64(x["k_blk"]), x["start_pos"].numpy(), **kw), "k")


def _scattered_positions(b, B, rng, hi):
    """Distinct positions per sequence, in no particular order (a later round
    of a block verifies whatever positions are still open)."""
    return np.stack([rng.choice(hi, size=B, replace=False) for _ in range(b)]).astype(np.int32)


@pytest.mark.parametrize("cfg", ["b8", "b16", "ragged"])
@pytest.mark.parametrize("flags", [0, binding.SIMSD_ROPE_INTERLEAVED])
def test_rope_at_explicit_positions_matches_oracle(cfg, flags):
    say(f"rope positions {cfg} flags={flags}")
    x = inputs(cfg)
    w = x["workload"]
    rng = np.random.default_rng(zlib.crc32(cfg.encode()))
    pos = _scattered_positions(w.b, w.B, rng, 2**31 - 64)
    pos[0] = np.arange(w.B)[::-1] + 4096  # one ordinary block, reversed
    q, k = x["q_blk"].cuda(), x["k_blk"].cuda()
    binding.simsd_rope_copy(q, k, torch.from_numpy(pos).cuda(), w.rope_base,
                            flags | binding.SIMSD_ROPE_POSITIONS)
    torch.cuda.synchronize()
    kw = dict(base=w.rope_base, interleaved=bool(flags & 1))
    for t, src, n in ((q, x["q_blk"], "q"), (k, x["k_blk"], "k")):
        _check(t, oracle.rope_copy(f64(src), pos, **kw), n, angle_slack(f64(src), pos, **kw))


def test_consecutive_positions_give_the_start_position_bits():
    w = synth.custom(b=4, Hq=8, Hkv=2, d=128, B=16, prefix=(0, 5000))
    x = synth.make_inputs(w, with_accept=False, seed=3)
    sp = x["start_pos"]
    pos = (sp[:, None] + torch.arange(16, dtype=torch.int32)[None, :]).contiguous()
    for flags in (0, binding.SIMSD_ROPE_INTERLEAVED):
        q0, k0 = x["q_blk"].cuda(), x["k_blk"].cuda()
        q1, k1 = x["q_blk"].cuda(), x["k_blk"].cuda()
        binding.simsd_rope_copy(q0, k0, sp.cuda(), 10000.0, flags)
        binding.simsd_rope_copy(q1, k1, pos.cuda(), 10000.0, flags | binding.SIMSD_ROPE_POSITIONS)
        torch.cuda.synchronize()
        assert torch.equal(q0, q1) and torch.equal(k0, k1), flags


def test_copy_rule_is_bit_exact_on_gpu():
    # identical vectors in D_k and D~_k must leave the kernel bit-identical
    w = synth.custom(b=3, Hq=8, Hkv=2, d=128, B=8, prefix=(100, 9000))
    x = synth.make_inputs(w, with_accept=False)
    q = x["q_blk"].clone()
    q[:, 8:] = q[:, :8]
    k = x["k_blk"].clone()
    k[:, 8:] = k[:, :8]
    qd, kd = q.cuda(), k.cuda()
    binding.simsd_rope_copy(qd, kd, x["start_pos"].cuda(), 10000.0, 0)
    assert torch.equal(qd[:, :8], qd[:, 8:]) and torch.equal(kd[:, :8], kd[:, 8:])
    qn, kn = q.cuda(), k.cuda()
    binding.simsd_rope_copy(qn, kn, x["start_pos"].cuda(), 10000.0, binding.SIMSD_ROPE_NO_COPY)
    assert not torch.equal(qn[:, :8], qn[:, 8:])
    # data rows are the same with or without the copy rule
    assert torch.equal(qn[:, :8], qd[:, :8])


def test_rope_d64_and_B1():
    for w in (synth.custom(b=2, Hq=4, Hkv=4, d=64, B=1, prefix=(0, 5)),
              synth.custom(b=1, Hq=2, Hkv=1, d=64, B=64, prefix=(70000, 70000))):
        say(f"rope {w}")
        x = synth.make_inputs(w, with_accept=False)
        q, k = x["q_blk"].cuda(), x["k_blk"].cuda()
        binding.simsd_rope_copy(q, k, x["start_pos"].cuda(), 500.0, 0)
        _check(q, oracle.rope_copy(f64(x["q_blk"]), x["start_pos"].numpy(), base=500.0), "q")
        _check(k, oracle.rope_copy(f64(x["k_blk"]), x["start_pos"].numpy(), base=500.0), "k")


@pytest.mark.parametrize("flags", [0, binding.SIMSD_ROPE_NO_COPY])
def test_rope_large_positions(flags):
    # angles beyond 2^30 rad (frequency 1 at positions near the int32 limit)
    # take the large-argument reduction of the fp64 sin/cos
    w = synth.custom(b=2, Hq=4, Hkv=2, d=128, B=8, prefix=(16, 16))
    x = synth.make_inputs(w, with_accept=False, seed=11)
    x["start_pos"] = torch.tensor([2**31 - 20, 2**30 + 7], dtype=torch.int32)
    say(f"rope large positions {x['start_pos'].tolist()} flags={flags}")
    q, k = x["q_blk"].cuda(), x["k_blk"].cuda()
    binding.simsd_rope_copy(q, k, x["start_pos"].cuda(), 10000.0, flags)
    torch.cuda.synchronize()
    kw = dict(base=10000.0, no_copy=bool(flags & 2))
    _check(q, oracle.rope_copy(f64(x["q_blk"]), x["start_pos"].numpy(), **kw), "q")
    _check(k, oracle.rope_copy(f64(x["k_blk"]), x["start_pos"].numpy(), **kw), "k")
