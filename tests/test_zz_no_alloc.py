"""The allocation-free attention entry point (simsd_verify_attention_noalloc)
against simsd_verify_attention with a caller workspace: the same kernels, so
out and lse must be bit-identical. Two calls in a row on the library's fixed
scratch buffer, the second on a smaller input (its counters and partials
start from what the first call left), then a call whose sizes exceed the
buffer is refused before anything is launched."""
import pytest
import torch

from masked_attention_simsd_amd import binding, synth
from gpu_util import say, to_dev

pytestmark = pytest.mark.gpu

LAYOUT = binding.SIMSD_KV_HEAD_MAJOR | binding.SIMSD_KV_PAIRED


def paired(g):
    kv = torch.stack([g["k_pre"].transpose(0, 1), g["v_pre"].transpose(0, 1)], dim=2).contiguous()
    return kv, binding.kv_pair_views(kv)


def both(x, flags, max_prefix):
    g = to_dev(x)
    kv, (kp, vp) = paired(g)
    b, twoB, Hq, d = g["q_blk"].shape
    f32 = bool(flags & binding.SIMSD_OUT_F32)
    mk = lambda: torch.full_like(g["q_blk"], float("nan"), dtype=torch.float32 if f32 else torch.bfloat16)
    lse_ref = torch.full((b, twoB, Hq), float("nan"), device="cuda")
    lse_na = torch.full((b, twoB, Hq), float("nan"), device="cuda")
    ws = torch.zeros(binding.simsd_verify_attention_workspace(b, twoB // 2, Hq, g["k_blk"].shape[2], d,
                                                              max_prefix), dtype=torch.uint8, device="cuda")
    ref = binding.simsd_verify_attention(g["q_blk"], g["k_blk"], g["v_blk"], kp, vp, g["prefix_offsets"],
                                         g["tau"], out=mk(), lse=lse_ref, max_prefix=max_prefix,
                                         flags=flags | LAYOUT, workspace=ws)
    out = binding.simsd_verify_attention_noalloc(g["q_blk"], g["k_blk"], g["v_blk"], kp, vp,
                                                 g["prefix_offsets"], g["tau"], out=mk(), lse=lse_na,
                                                 max_prefix=max_prefix, flags=flags | LAYOUT)
    torch.cuda.synchronize()
    return ref, out, lse_ref, lse_na


def test_noalloc_equals_workspace_entry_point_on_two_calls():
    # call 1: 8 sequences of 16384 cached tokens, B = 16 (four splits per
    # unit: 16.5 MiB of the scratch buffer in use)
    x = synth.make_inputs("b16", with_accept=False)
    say("noalloc call 1: b16 workload")
    ref, out, lse_ref, lse_na = both(x, 0, 16384)
    assert torch.isfinite(ref.float()).all()
    assert torch.equal(out, ref) and torch.equal(lse_na, lse_ref)
    # call 2, smaller: 3 sequences with ragged prefixes (one empty), B = 8, fp32 out
    w = synth.custom(b=3, Hq=16, Hkv=4, d=128, B=8, prefix=(0, 1300))
    x = synth.make_inputs(w, with_accept=False, seed=5)
    say("noalloc call 2: 3 ragged sequences")
    ref, out, lse_ref, lse_na = both(x, binding.SIMSD_OUT_F32, 1300)
    assert torch.isfinite(ref).all()
    assert torch.equal(out, ref) and torch.equal(lse_na, lse_ref)


def test_noalloc_refuses_sizes_beyond_its_buffer():
    x = to_dev(synth.make_inputs(synth.custom(b=8, Hq=32, Hkv=8, d=128, B=16, prefix=(64, 64)),
                                 with_accept=False, seed=6))
    out = torch.zeros_like(x["q_blk"])
    with binding.tuning(attn_target_wg=1 << 20):
        with pytest.raises(binding.SimsdError) as e:
            binding.simsd_verify_attention_noalloc(x["q_blk"], x["k_blk"], x["v_blk"], x["k_pre"], x["v_pre"],
                                                   x["prefix_offsets"], x["tau"], out=out, max_prefix=1 << 24)
    assert e.value.code == binding.SIMSD_ERR_SCRATCH
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(out)) == 0  # nothing launched
