"""The verification step captured once in a HIP graph (torch.cuda.graph) and
replayed: every replay reproduces, bit for bit, what the same calls give
eagerly. The library allocates nothing and issues no memset inside its calls,
and every kernel that uses workspace counters leaves them zero, so a captured
call can be replayed as often as the caller likes. Captured here: RoPE-copy ->
verify attention -> acceptance, the fused RoPE + attention form, and
acceptance from logits (two launches with their own counters). Between
replays the test runs unrelated eager work and synchronises; the in-place
RoPE inputs are restored eagerly before each replay."""
import pytest
import torch

from masked_attention_simsd_amd import binding
from gpu_util import inputs, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cfg", ["b4", "b8", "ragged"])
def test_step_graph_replays_match_eager(cfg):
    say(f"graph replay {cfg}")
    x = inputs(cfg)
    w = x["workload"]
    g = to_dev(x)
    b = w.b
    maxp = int((x["prefix_offsets"][1:] - x["prefix_offsets"][:-1]).max())
    q0, k0 = g["q_blk"].clone(), g["k_blk"].clone()
    q_s, k_s = q0.clone(), k0.clone()
    i32 = dict(dtype=torch.int32, device="cuda")
    bufs = {n: torch.empty(b, **i32) for n in ("L", "C", "Ll", "Cl")}
    out, out_f = torch.empty_like(q0), torch.empty_like(q0)
    k_rot = torch.empty_like(k0)
    status = torch.zeros(b, **i32)

    def step():
        binding.simsd_rope_copy(q_s, k_s, g["start_pos"], w.rope_base)
        binding.simsd_verify_attention(q_s, k_s, g["v_blk"], g["k_pre"], g["v_pre"], g["prefix_offsets"],
                                       g["tau"], out=out, max_prefix=maxp, status=status)
        binding.simsd_accept(g["p"], g["q"], g["draft"], g["tau"], g["u"], accept_len=bufs["L"],
                             correction_token=bufs["C"], status=status)
        binding.simsd_verify_attention_rope(q0, k0, g["v_blk"], g["k_pre"], g["v_pre"], g["prefix_offsets"],
                                            g["tau"], g["start_pos"], w.rope_base, k_rot=k_rot, out=out_f,
                                            max_prefix=maxp)
        binding.simsd_accept_logits(g["target_logits"], g["draft_logits"], g["draft"], g["tau"], g["u"],
                                    accept_len=bufs["Ll"], correction_token=bufs["Cl"])

    def restore():
        q_s.copy_(q0)
        k_s.copy_(k0)
        status.zero_()

    def snapshot():
        return [t.clone() for t in (out, out_f, k_rot, q_s, k_s, status, *bufs.values())]

    # eager reference (also creates the cached workspaces before capture)
    restore()
    step()
    torch.cuda.synchronize()
    ref = snapshot()
    restore()
    step()
    torch.cuda.synchronize()
    for a, r in zip(snapshot(), ref):
        assert torch.equal(a, r), "eager step is not repeatable"

    graph = torch.cuda.CUDAGraph()
    restore()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    names = ("out", "out_fused", "k_rot", "q_rotated", "k_rotated", "status", *bufs)
    noise = torch.randn(512, 512, device="cuda")
    for rep in range(4):
        for t in (out, out_f, k_rot, *bufs.values()):
            t.fill_(-1) if t.dtype == torch.int32 else t.fill_(float("nan"))
        restore()
        graph.replay()
        torch.cuda.synchronize()
        for n, a, r in zip(names, snapshot(), ref):
            assert torch.equal(a, r), f"replay {rep}: {n} differs from the eager step"
        noise = (noise @ noise).tanh_()  # unrelated eager work between replays
        torch.cuda.synchronize()
    say(f"  {cfg}: 4 replays equal the eager step")
