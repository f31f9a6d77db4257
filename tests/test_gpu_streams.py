"""Two independent verification batches in flight at once, each on its own
stream with its own workspaces (RoPE-copy -> attention -> acceptance per
batch), give bit for bit what each gives when run alone: the entry points keep
no state between calls beyond the workspace they are handed."""
import pytest
import torch

from masked_attention_simsd_amd import binding, synth
from gpu_util import say, to_dev

pytestmark = pytest.mark.gpu


def batch(seed, cfg="b8"):
    x = to_dev(synth.make_inputs(cfg, seed=seed))
    w = x["workload"]
    b, B = w.b, w.B
    ws_a = torch.zeros(binding.simsd_verify_attention_workspace(b, B, w.Hq, w.Hkv, w.d, int(w.prefix[1])),
                       dtype=torch.uint8, device="cuda")
    ws_c = torch.zeros(binding.simsd_accept_workspace(b, B, w.V), dtype=torch.uint8, device="cuda")
    return x, ws_a, ws_c


def step(x, ws_a, ws_c, stream):
    """One verification step of batch x on `stream`; returns (out, L, C)."""
    w = x["workload"]
    q, k = x["q_blk"].clone(), x["k_blk"].clone()
    out = torch.empty_like(q)
    L = torch.empty(w.b, dtype=torch.int32, device="cuda")
    C = torch.empty_like(L)
    binding.simsd_rope_copy(q, k, x["start_pos"], w.rope_base, stream=stream)
    binding.simsd_verify_attention(q, k, x["v_blk"], x["k_pre"], x["v_pre"], x["prefix_offsets"], x["tau"],
                                   out=out, max_prefix=int(w.prefix[1]), workspace=ws_a, stream=stream)
    binding.simsd_accept(x["p"], x["q"], x["draft"], x["tau"], x["u"], accept_len=L, correction_token=C,
                         workspace=ws_c, stream=stream)
    return out, L, C


@pytest.mark.parametrize("cfg", ["b8", "ragged"])
def test_two_batches_on_two_streams_match_alone(cfg):
    say(f"two batches on two streams, {cfg}")
    A, B_ = batch(11, cfg), batch(12, cfg)
    cur = torch.cuda.current_stream()
    ref = [step(*A, cur), step(*B_, cur)]
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()  # default priority
    for rep in range(4):
        s1.wait_stream(cur)
        s2.wait_stream(cur)
        with torch.cuda.stream(s1):
            got_a = step(*A, s1)
        with torch.cuda.stream(s2):
            got_b = step(*B_, s2)
        cur.wait_stream(s1)
        cur.wait_stream(s2)
        torch.cuda.synchronize()
        for got, want, name in ((got_a, ref[0], "A"), (got_b, ref[1], "B")):
            for g, r in zip(got, want):
                assert torch.equal(g, r), (rep, name)
    # the acceptance workspaces are left zero for the next call, as after a
    # lone call (the attention workspace keeps only its counters zero)
    for ws in (A[2], B_[2]):
        assert int(torch.count_nonzero(ws)) == 0
