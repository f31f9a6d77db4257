"""RoPE-copy on the GPU against the oracle (bf16 outputs vs the oracle's fp64
rotation rounded once to bf16)."""
import numpy as np
import pytest
import torch

import oracle
from masked_attention_simsd_amd import binding, synth
from gpu_util import bf16_round, bf16_ulp, f64, inputs, say

pytestmark = pytest.mark.gpu


def _check(gpu, ref_f64, what):
    ref = bf16_round(ref_f64)
    got = f64(gpu)
    diff = np.abs(got - ref)
    exact = float(np.mean(diff == 0))
    ulps = float((diff / bf16_ulp(ref)).max())
    say(f"  {what}: exact {exact:.6f}, max {ulps:.2f} ulp")
    assert ulps <= 1.0, what
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
