"""RoPE-copy fused into verify attention (simsd_verify_attention_rope).

The fused entry point must give the same bits as simsd_rope_copy followed by
simsd_verify_attention (out, lse and the rotated block keys), leave q_blk and
k_blk untouched, and agree with the oracle chain (oracle RoPE rounded to bf16,
then oracle attention) within the attention tolerance."""
import numpy as np
import pytest
import torch

import oracle
from masked_attention_simsd_amd import binding, synth
from gpu_util import ORACLE_THREADS, bf16_round, f64, inputs, say, subset_sequences, to_dev

pytestmark = pytest.mark.gpu


def two_call(g, w_base, rope_flags, flags, max_prefix):
    q = g["q_blk"].clone()
    k = g["k_blk"].clone()
    binding.simsd_rope_copy(q, k, g["start_pos"], w_base, rope_flags)
    lse = torch.full(q.shape[:3], float("nan"), device="cuda")
    out = binding.simsd_verify_attention(q, k, g["v_blk"], g["k_pre"], g["v_pre"], g["prefix_offsets"],
                                         g["tau"], lse=lse, max_prefix=max_prefix, flags=flags)
    return out, lse, k


def fused(g, w_base, rope_flags, flags, max_prefix):
    k_rot = torch.zeros_like(g["k_blk"])
    lse = torch.full(g["q_blk"].shape[:3], float("nan"), device="cuda")
    out = binding.simsd_verify_attention_rope(g["q_blk"], g["k_blk"], g["v_blk"], g["k_pre"], g["v_pre"],
                                              g["prefix_offsets"], g["tau"], g["start_pos"], w_base,
                                              rope_flags, k_rot=k_rot, lse=lse, max_prefix=max_prefix,
                                              flags=flags)
    return out, lse, k_rot


def prep(x, head_major):
    g = to_dev(x)
    if head_major:
        g["k_pre"] = g["k_pre"].transpose(0, 1).contiguous()
        g["v_pre"] = g["v_pre"].transpose(0, 1).contiguous()
    return g


CASES = [
    # (b, Hq, Hkv, d, B, prefix range, rope flags, attention flags)
    (3, 8, 2, 128, 8, (100, 700), 0, 0),
    (2, 32, 8, 128, 16, (1000, 2500), 0, binding.SIMSD_KV_HEAD_MAJOR),
    (2, 32, 8, 128, 8, (0, 300), binding.SIMSD_ROPE_INTERLEAVED, binding.SIMSD_OUT_F32),
    (2, 16, 4, 128, 5, (40, 900), binding.SIMSD_ROPE_NO_COPY, binding.SIMSD_DATA_BIDIR),
    (2, 4, 1, 64, 3, (0, 70), binding.SIMSD_ROPE_INTERLEAVED | binding.SIMSD_ROPE_NO_COPY,
     binding.SIMSD_DATA_SKIP),
    (1, 8, 8, 128, 1, (0, 0), 0, 0),
    (1, 4, 1, 64, 64, (130, 130), binding.SIMSD_ROPE_NO_COPY, binding.SIMSD_OUT_F32),
    (1, 32, 8, 128, 64, (300, 300), 0, binding.SIMSD_KV_HEAD_MAJOR),
    # 64-row workgroups whose 64-position table does not fit beside the 64 x 3
    # ring: the fused launch takes 64 x 2, the two-launch reference 64 x 3 (the
    # ring's depth changes no arithmetic), and one whose 48 positions fit
    (1, 8, 8, 128, 32, (300, 300), binding.SIMSD_ROPE_NO_COPY, 0),
    (2, 16, 16, 128, 32, (600, 2000), binding.SIMSD_ROPE_NO_COPY,
     binding.SIMSD_KV_HEAD_MAJOR | binding.SIMSD_OUT_F32),
    (2, 8, 8, 128, 24, (500, 1800), binding.SIMSD_ROPE_NO_COPY, 0),
    (1, 8, 2, 128, 32, (500, 500), binding.SIMSD_ROPE_NO_COPY, 0),
    # a position per pair (a later round of a block)
    (3, 8, 2, 128, 8, (100, 700), binding.SIMSD_ROPE_POSITIONS, 0),
    (2, 32, 8, 128, 16, (1000, 2500), binding.SIMSD_ROPE_POSITIONS | binding.SIMSD_ROPE_INTERLEAVED,
     binding.SIMSD_KV_HEAD_MAJOR | binding.SIMSD_OUT_F32),
    (2, 32, 8, 128, 8, (0, 3000), binding.SIMSD_ROPE_POSITIONS, binding.SIMSD_DATA_SKIP),
    (1, 32, 8, 128, 40, (300, 300), binding.SIMSD_ROPE_POSITIONS, 0),
]


def table_falls_back(Hq, Hkv, d, B, rflags, flags):
    """Whether the fused launch of a 128-row workgroup (head_dim 128) cannot
    put its fp64 cos/sin table (1 KB per position) and the 1 KB of staged
    frequencies beside the 128-key ring (about 28 KB of LDS are left, so 26
    positions fit) and takes the 64-key two-wave variant instead."""
    rows = (B if (flags & 3) == binding.SIMSD_DATA_SKIP else 2 * B) * (Hq // Hkv)
    npos = 2 * B if rflags & binding.SIMSD_ROPE_NO_COPY else B
    return d == 128 and rows > 64 and npos > 26


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_fused_equals_two_calls_bit_exact(case):
    b, Hq, Hkv, d, B, pre, rflags, flags = case
    say(f"fused rope+attention {case}")
    w = synth.custom(b=b, Hq=Hq, Hkv=Hkv, d=d, B=B, prefix=pre)
    x = synth.make_inputs(w, with_accept=False, seed=hash(case) % 1000)
    # positions far from 0 (the rotation matters) and different per sequence
    x["start_pos"] = x["start_pos"] + torch.arange(b, dtype=torch.int32) * 977 + 50000
    if rflags & binding.SIMSD_ROPE_POSITIONS:
        # one position per pair, scattered and unordered
        gen = torch.Generator().manual_seed(B)
        x["start_pos"] = torch.stack([torch.randperm(4 * B, generator=gen)[:B] * 37 + int(p0)
                                      for p0 in x["start_pos"]]).to(torch.int32).contiguous()
    g = prep(x, flags & binding.SIMSD_KV_HEAD_MAJOR)
    q0, k0 = g["q_blk"].clone(), g["k_blk"].clone()
    mp = int(pre[1])
    # the reference takes the variant the fused launch falls back to when its
    # table does not fit beside the default ring
    with binding.tuning(attn_pipe=7 if table_falls_back(Hq, Hkv, d, B, rflags, flags) else -1):
        ref_out, ref_lse, ref_k = two_call(g, 10000.0, rflags, flags, mp)
    out, lse, k_rot = fused(g, 10000.0, rflags, flags, mp)
    torch.cuda.synchronize()
    assert torch.equal(g["q_blk"], q0) and torch.equal(g["k_blk"], k0), "inputs modified"
    assert torch.equal(k_rot, ref_k), "rotated keys differ"
    rows = slice(B, None) if (flags & 3) == binding.SIMSD_DATA_SKIP else slice(None)
    assert torch.equal(out[:, rows], ref_out[:, rows]), "out differs"
    assert torch.equal(lse[:, rows], ref_lse[:, rows]), "lse differs"


@pytest.mark.parametrize("cfg,seqs", [("b8", None), ("b16", None), ("ragged", None)])
def test_fused_workloads_match_oracle_chain(cfg, seqs):
    say(f"fused workload {cfg}")
    x = inputs(cfg)
    w = x["workload"]
    g = prep(x, True)
    out, _, k_rot = fused(g, w.rope_base, 0, binding.SIMSD_KV_HEAD_MAJOR, int(w.prefix[1]))
    ref_out, _, ref_k = two_call(g, w.rope_base, 0, binding.SIMSD_KV_HEAD_MAJOR, int(w.prefix[1]))
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out) and torch.equal(k_rot, ref_k)
    sub = subset_sequences(x, seqs) if seqs else x
    idx = torch.tensor(seqs if seqs else list(range(w.b)), device="cuda")
    sp = x["start_pos"].numpy()[idx.cpu().numpy()]
    q_r = bf16_round(oracle.rope_copy(f64(sub["q_blk"]), sp, w.rope_base))
    k_r = bf16_round(oracle.rope_copy(f64(sub["k_blk"]), sp, w.rope_base))
    ref, _ = oracle.verify_attention(q_r, k_r, f64(sub["v_blk"]), f64(sub["k_pre"]), f64(sub["v_pre"]),
                                     sub["prefix_offsets"].numpy(), sub["tau"].numpy(),
                                     threads=ORACLE_THREADS)
    err = float(np.abs(f64(out[idx]) - ref).max())
    kerr = float(np.abs(f64(k_rot[idx]) - k_r).max())
    say(f"  max-abs vs oracle chain {err:.3e}; rotated keys max-abs {kerr:.3e}")
    assert err <= 2e-2
    assert kerr <= float(np.abs(k_r).max()) * 2 ** -8


def test_fused_without_k_rot_and_status():
    w = synth.custom(b=2, Hq=8, Hkv=2, d=128, B=4, prefix=(200, 300))
    x = synth.make_inputs(w, with_accept=False, seed=5)
    x["tau"][1, 0] = x["tau"][1, 1]  # not a permutation
    g = prep(x, False)
    status = torch.zeros(2, dtype=torch.int32, device="cuda")
    binding.simsd_verify_attention_rope(g["q_blk"], g["k_blk"], g["v_blk"], g["k_pre"], g["v_pre"],
                                        g["prefix_offsets"], g["tau"], g["start_pos"], status=status)
    torch.cuda.synchronize()
    assert status.cpu().tolist() == [0, binding.SIMSD_DEV_BAD_TAU]


@pytest.mark.parametrize("rflags", [0, binding.SIMSD_ROPE_NO_COPY])
def test_fused_large_positions(rflags):
    # positions near the int32 limit: the fused table takes the same
    # large-argument sin/cos as the RoPE-copy kernel, bit for bit
    w = synth.custom(b=2, Hq=32, Hkv=8, d=128, B=8, prefix=(100, 300))
    x = synth.make_inputs(w, with_accept=False, seed=12)
    x["start_pos"] = torch.tensor([2**31 - 20, 2**30 + 7], dtype=torch.int32)
    say(f"fused large positions {x['start_pos'].tolist()} rflags={rflags}")
    g = prep(x, False)
    ref_out, ref_lse, ref_k = two_call(g, 10000.0, rflags, 0, 300)
    out, lse, k_rot = fused(g, 10000.0, rflags, 0, 300)
    torch.cuda.synchronize()
    assert torch.equal(k_rot, ref_k) and torch.equal(out, ref_out) and torch.equal(lse, ref_lse)
