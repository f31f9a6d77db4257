"""The whole verification step on the GPU (RoPE-copy -> verify attention ->
acceptance, one stream) against the oracle chain. The oracle's RoPE output is
rounded to bf16 before its attention, as the boundary stores it."""
import numpy as np
import pytest
import torch

import oracle
from masked_attention_simsd_amd import binding
from gpu_util import ORACLE_THREADS, bf16_round, f64, inputs, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cfg,paired", [("tiny", False), ("b4", False), ("b8", False), ("b8", True),
                                        ("b16", False), ("b16", True), ("ragged", True)],
                         ids=["tiny", "b4", "b8", "b8_paired_head_major", "b16", "b16_paired_head_major",
                              "ragged_paired_head_major"])
def test_chain_matches_oracle(cfg, paired):
    say(f"chain {cfg} paired head-major {paired}")
    x = inputs(cfg)
    w = x["workload"]
    g = to_dev(x)
    flags = 0
    if paired:
        # the cache layout the benchmark times: [Hkv][sum P][2][d]
        kv = torch.stack([g["k_pre"].transpose(0, 1), g["v_pre"].transpose(0, 1)], dim=2).contiguous()
        g["k_pre"], g["v_pre"] = binding.kv_pair_views(kv)
        flags = binding.SIMSD_KV_HEAD_MAJOR | binding.SIMSD_KV_PAIRED
    status = torch.zeros(w.b, dtype=torch.int32, device="cuda")
    binding.simsd_rope_copy(g["q_blk"], g["k_blk"], g["start_pos"], w.rope_base)
    out = binding.simsd_verify_attention(g["q_blk"], g["k_blk"], g["v_blk"], g["k_pre"], g["v_pre"],
                                         g["prefix_offsets"], g["tau"], max_prefix=w.prefix[1],
                                         flags=flags, status=status)
    L, corr = binding.simsd_accept(g["p"], g["q"], g["draft"], g["tau"], g["u"], status=status)
    torch.cuda.synchronize()

    sp = x["start_pos"].numpy()
    q_r = bf16_round(oracle.rope_copy(f64(x["q_blk"]), sp, w.rope_base))
    k_r = bf16_round(oracle.rope_copy(f64(x["k_blk"]), sp, w.rope_base))
    ref, _ = oracle.verify_attention(q_r, k_r, f64(x["v_blk"]), f64(x["k_pre"]), f64(x["v_pre"]),
                                     x["prefix_offsets"].numpy(), x["tau"].numpy(),
                                     threads=ORACLE_THREADS)
    err = float(np.abs(f64(out) - ref).max())
    acc = oracle.accept(x["p"].numpy(), x["q"].numpy(), x["draft"].numpy(), x["tau"].numpy(),
                        x["u"].numpy())
    say(f"  attention max-abs {err:.3e}; accept lengths {L.cpu().tolist()}")
    assert err <= 2e-2
    assert np.array_equal(L.cpu().numpy(), acc["accept_len"])
    ok = (corr.cpu().numpy() == acc["correction"]) | acc["boundary"].astype(bool)
    assert ok.all()
    assert (status.cpu().numpy() == acc["status"]).all()
