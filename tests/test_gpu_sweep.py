"""A seeded sweep of random verify-attention shapes against the oracle:
batch size, head counts and grouping, head dimension, block size (including
the extremes 1 and 64), ragged and empty prefixes, all three data-row rules,
all four cache layouts and both output types. Each case is printed before it
runs. Tolerances as in the other attention tests: max-abs 2e-2 for bf16
output, 4e-3 for fp32 output, 2e-3 for the log-sum-exp."""
import numpy as np
import pytest
import torch

import oracle
from masked_attention_simsd_amd import binding, synth
from gpu_util import ORACLE_THREADS, bf16_round, bf16_ulp, f64, say, to_dev

pytestmark = pytest.mark.gpu

HM, PAIRED = binding.SIMSD_KV_HEAD_MAJOR, binding.SIMSD_KV_PAIRED
LAYOUTS = [0, HM, PAIRED, HM | PAIRED]


def draw_cases(n, seed=20261202):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        d = int(rng.choice([64, 128]))
        Hkv = int(rng.choice([1, 2, 4, 8]))
        G = int(rng.choice([1, 2, 4, 8]))
        B = int(rng.choice([1, 2, 3, 5, 8, 13, 16, 20, 32, 64]))
        b = int(rng.integers(1, 5))
        lo = int(rng.choice([0, 1, 17, 200]))
        hi = lo + int(rng.integers(0, 1400))
        # bound the oracle's work (rows x keys x d) so the sweep stays in seconds
        while b * 2 * B * G * Hkv * (hi + 2 * B) * d > 6e8 and (b > 1 or hi > lo):
            if b > 1:
                b -= 1
            else:
                hi = lo + (hi - lo) // 2
        cases.append(dict(id=i, b=b, Hq=G * Hkv, Hkv=Hkv, d=d, B=B, prefix=(lo, hi),
                          layout=LAYOUTS[int(rng.integers(0, 4))], rule=int(rng.integers(0, 3)),
                          f32=bool(rng.integers(0, 2))))
    return cases


CASES = draw_cases(120)


def _layout(g, layout):
    k, v = g["k_pre"], g["v_pre"]
    if layout & HM:
        k, v = k.transpose(0, 1).contiguous(), v.transpose(0, 1).contiguous()
    if layout & PAIRED:
        kv = torch.stack([k, v], dim=2).contiguous()
        k, v = binding.kv_pair_views(kv)
    return k, v


@pytest.mark.parametrize("case", CASES, ids=[f"case{c['id']}" for c in CASES])
def test_random_shapes_match_oracle(case):
    say(f"sweep {case}")
    w = synth.custom(b=case["b"], Hq=case["Hq"], Hkv=case["Hkv"], d=case["d"], B=case["B"],
                     prefix=case["prefix"])
    x = synth.make_inputs(w, with_accept=False, seed=5000 + case["id"])
    g = to_dev(x)
    k, v = _layout(g, case["layout"])
    flags = case["layout"] | case["rule"] | (binding.SIMSD_OUT_F32 if case["f32"] else 0)
    b, twoB, Hq = x["q_blk"].shape[:3]
    lse = torch.full((b, twoB, Hq), float("nan"), device="cuda")
    out = binding.simsd_verify_attention(g["q_blk"], g["k_blk"], g["v_blk"], k, v, g["prefix_offsets"],
                                         g["tau"], lse=lse, max_prefix=int(x["prefix_lens"].max()),
                                         flags=flags)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.verify_attention(f64(x["q_blk"]), f64(x["k_blk"]), f64(x["v_blk"]),
                                           f64(x["k_pre"]), f64(x["v_pre"]), x["prefix_offsets"].numpy(),
                                           x["tau"].numpy(), data_rule=case["rule"], threads=ORACLE_THREADS)
    rows = slice(None) if case["rule"] != 2 else slice(twoB // 2, None)
    err = float(np.abs(f64(out)[:, rows] - ref[:, rows]).max())
    lerr = float(np.abs(f64(lse)[:, rows] - ref_lse[:, rows]).max())
    say(f"  max-abs {err:.3e}, lse {lerr:.3e}")
    assert err <= (4e-3 if case["f32"] else 2e-2)
    assert lerr <= 2e-3


@pytest.mark.parametrize("case", CASES[:60], ids=[f"case{c['id']}" for c in CASES[:60]])
def test_random_shapes_fused_rope_match_oracle(case):
    """RoPE-copy fused into the attention, on unrotated block rows, against the
    oracle chain (RoPE in fp64 rounded to bf16, as the boundary stores it, then
    attention); the rotated block keys it writes against the oracle's RoPE."""
    say(f"sweep fused {case}")
    w = synth.custom(b=case["b"], Hq=case["Hq"], Hkv=case["Hkv"], d=case["d"], B=case["B"],
                     prefix=case["prefix"])
    x = synth.make_inputs(w, with_accept=False, seed=7000 + case["id"])
    g = to_dev(x)
    k, v = _layout(g, case["layout"])
    flags = case["layout"] | case["rule"] | (binding.SIMSD_OUT_F32 if case["f32"] else 0)
    b, twoB, Hq = x["q_blk"].shape[:3]
    lse = torch.full((b, twoB, Hq), float("nan"), device="cuda")
    k_rot = torch.empty_like(g["k_blk"])
    out = binding.simsd_verify_attention_rope(g["q_blk"], g["k_blk"], g["v_blk"], k, v, g["prefix_offsets"],
                                              g["tau"], g["start_pos"], w.rope_base, k_rot=k_rot, lse=lse,
                                              max_prefix=int(x["prefix_lens"].max()), flags=flags)
    torch.cuda.synchronize()
    sp = x["start_pos"].numpy()
    q_r = bf16_round(oracle.rope_copy(f64(x["q_blk"]), sp, w.rope_base))
    k_r = bf16_round(oracle.rope_copy(f64(x["k_blk"]), sp, w.rope_base))
    kerr = float((np.abs(f64(k_rot) - k_r) / bf16_ulp(k_r)).max())
    ref, ref_lse = oracle.verify_attention(q_r, k_r, f64(x["v_blk"]), f64(x["k_pre"]), f64(x["v_pre"]),
                                           x["prefix_offsets"].numpy(), x["tau"].numpy(),
                                           data_rule=case["rule"], threads=ORACLE_THREADS)
    rows = slice(None) if case["rule"] != 2 else slice(twoB // 2, None)
    err = float(np.abs(f64(out)[:, rows] - ref[:, rows]).max())
    lerr = float(np.abs(f64(lse)[:, rows] - ref_lse[:, rows]).max())
    say(f"  max-abs {err:.3e}, lse {lerr:.3e}, k_rot {kerr:.2f} ulp")
    assert kerr <= 1.0
    assert err <= (4e-3 if case["f32"] else 2e-2)
    assert lerr <= 2e-3
