"""Acceptance on the GPU against the oracle: accepted lengths bit-exact;
correction tokens equal except where the oracle marks u*Z within 1e-6*Z of a
CDF step (those cases are counted and printed)."""
import numpy as np
import pytest
import torch

import oracle
from masked_attention_simsd_amd import binding
from gpu_util import inputs, say

pytestmark = pytest.mark.gpu


def run_both(p, q, draft, tau, u):
    dev = lambda a: torch.as_tensor(np.ascontiguousarray(a)).cuda()
    status = torch.zeros(p.shape[0], dtype=torch.int32, device="cuda")
    L, corr = binding.simsd_accept(dev(p), dev(q), dev(draft), dev(tau), dev(u), status=status)
    torch.cuda.synchronize()
    ref = oracle.accept(p, q, draft, tau, u)
    return L.cpu().numpy(), corr.cpu().numpy(), status.cpu().numpy(), ref


def check(p, q, draft, tau, u, what):
    L, corr, st, ref = run_both(p, q, draft, tau, u)
    assert np.array_equal(L, ref["accept_len"]), what
    assert np.array_equal(st, ref["status"]), what
    diff = corr != ref["correction"]
    boundary = ref["boundary"].astype(bool)
    say(f"  {what}: b={len(L)}, mean L {L.mean():.2f}, rejected {np.mean(L < p.shape[1]):.2f}, "
        f"token mismatches {int(diff.sum())} (boundary cases {int(boundary.sum())})")
    assert not (diff & ~boundary).any(), what
    return L, corr


@pytest.mark.parametrize("cfg", ["tiny", "b4", "b8", "b16", "ragged"])
def test_workloads_match_oracle(cfg):
    say(f"accept workload {cfg}")
    x = inputs(cfg)
    check(x["p"].numpy(), x["q"].numpy(), x["draft"].numpy(), x["tau"].numpy(), x["u"].numpy(), cfg)


def rejecting_inputs(V, b, B=8, seed=None):
    # Random distributions and uniformly drawn drafts: nearly every sequence
    # rejects early, so the residual draw runs for almost all of them.
    rng = np.random.default_rng(V if seed is None else seed)
    logits = rng.standard_normal((b, B, V)) * 2.0
    p = np.exp(logits - logits.max(-1, keepdims=True))
    p = (p / p.sum(-1, keepdims=True)).astype(np.float32)
    lq = logits + rng.standard_normal((b, B, V)) * 1.0
    q = np.exp(lq - lq.max(-1, keepdims=True))
    q = (q / q.sum(-1, keepdims=True)).astype(np.float32)
    draft = rng.integers(0, V, (b, B)).astype(np.int32)
    tau = np.stack([rng.permutation(B) + 1 for _ in range(b)]).astype(np.int32)
    u = rng.random((b, B + 1)).astype(np.float32)
    return p, q, draft, tau, u


@pytest.mark.parametrize("V", [4, 7, 32768, 151936])
def test_many_forced_rejections(V):
    check(*rejecting_inputs(V, 256 if V < 100000 else 32), f"V={V}")


@pytest.mark.parametrize("V,b", [(5001, 64), (32768, 64), (151936, 24)])
def test_segment_widths_agree_and_leave_workspace_zero(V, b):
    # Every segment width (entries per thread 4 / 8 / 16) gives the oracle's
    # lengths and, outside counted CDF-boundary cases, its tokens; each call
    # leaves the whole workspace zero for the next one.
    p, q, draft, tau, u = rejecting_inputs(V, b, seed=7)
    ref = oracle.accept(p, q, draft, tau, u)
    boundary = ref["boundary"].astype(bool)
    dev = lambda a: torch.as_tensor(np.ascontiguousarray(a)).cuda()
    args = [dev(a) for a in (p, q, draft, tau, u)]
    ws = torch.zeros(binding.simsd_accept_workspace(b, 8, V), dtype=torch.uint8, device="cuda")
    for per in (4, 8, 16, 4):
        say(f"  V={V} b={b} entries per thread {per}")
        status = torch.zeros(b, dtype=torch.int32, device="cuda")
        with binding.tuning(accept_per=per):
            L, corr = binding.simsd_accept(*args, status=status, workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(L.cpu().numpy(), ref["accept_len"]), per
        assert np.array_equal(status.cpu().numpy(), ref["status"]), per
        diff = corr.cpu().numpy() != ref["correction"]
        assert not (diff & ~boundary).any(), per
        assert int(torch.count_nonzero(ws)) == 0, per


def test_edge_cases():
    rng = np.random.default_rng(3)
    B, V = 64, 100
    b = 8
    p = rng.random((b, B, V)).astype(np.float32)
    p /= p.sum(-1, keepdims=True)
    q = p.copy()
    draft = rng.integers(0, V, (b, B)).astype(np.int32)
    tau = np.stack([rng.permutation(B) + 1 for _ in range(b)]).astype(np.int32)
    u = rng.random((b, B + 1)).astype(np.float32)
    L, corr = check(p, q, draft, tau, u, "p == q, B=64")
    assert (L == B).all() and (corr == -1).all()
    # bad tau, bad token, q(x) = 0, zero residual, single-token vocabulary
    tau2 = tau.copy()
    tau2[0, :2] = 1
    draft2 = draft.copy()
    draft2[1, np.argsort(tau[1])[0]] = V + 5
    q2 = q.copy()
    k = np.argsort(tau[2])[0]
    q2[2, k, draft[2, k]] = 0.0
    p2 = p.copy()
    k3 = np.argsort(tau[3])[0]
    p2[3, k3] = q2[3, k3] * 0.5  # p < q everywhere: residual mass 0
    u2 = u.copy()
    u2[3, 0] = 0.9999
    check(p2, q2, draft2, tau2, u2, "status cases")
    one = np.ones((4, 3, 1), np.float32)
    check(one, one, np.zeros((4, 3), np.int32), np.tile(np.array([[2, 3, 1]], np.int32), (4, 1)),
          rng.random((4, 4)).astype(np.float32), "V=1")
    # a block of one position (B = 1): one ratio, then the correction from that row
    p1 = rng.random((6, 1, 37)).astype(np.float32)
    p1 /= p1.sum(-1, keepdims=True)
    q1 = rng.random((6, 1, 37)).astype(np.float32)
    q1 /= q1.sum(-1, keepdims=True)
    u1 = rng.random((6, 2)).astype(np.float32)
    u1[:3, 0] = 0.9999  # rejected: the correction is drawn
    check(p1, q1, rng.integers(0, 37, (6, 1)).astype(np.int32), np.ones((6, 1), np.int32), u1, "B=1")
