"""Acceptance from logits on the GPU against the oracle (fp64 softmax rounded
to fp32, then the acceptance algorithm): accepted lengths equal except where
the oracle flags a uniform within a few fp32 ulps of its step's ratio; tokens
equal except flagged CDF-boundary cases (both counted and printed)."""
import numpy as np
import pytest
import torch

import oracle
from masked_attention_simsd_amd import binding
from gpu_util import inputs, say

pytestmark = pytest.mark.gpu


def check(zt, zd, draft, tau, u, T, what, ws=None):
    dev = lambda a: torch.as_tensor(np.ascontiguousarray(a)).cuda()
    status = torch.zeros(zt.shape[0], dtype=torch.int32, device="cuda")
    L, corr = binding.simsd_accept_logits(dev(zt), dev(zd), dev(draft), dev(tau), dev(u), temperature=T,
                                          status=status, workspace=ws)
    torch.cuda.synchronize()
    ref = oracle.accept_logits(zt, zd, T, draft, tau, u)
    L, corr, st = L.cpu().numpy(), corr.cpu().numpy(), status.cpu().numpy()
    rb = ref["ratio_boundary"].astype(bool)
    bd = ref["boundary"].astype(bool)
    dl = L != ref["accept_len"]
    dc = (corr != ref["correction"]) & ~dl
    say(f"  {what}: b={len(L)}, mean L {L.mean():.2f}, L mismatches {int(dl.sum())} (ratio-boundary "
        f"{int(rb.sum())}), token mismatches {int(dc.sum())} (CDF-boundary {int(bd.sum())})")
    assert not (dl & ~rb).any(), what
    assert not (dc & ~bd).any(), what
    assert np.array_equal(st[~dl], ref["status"][~dl]), what
    return L, corr


@pytest.mark.parametrize("cfg", ["tiny", "b4", "b8", "b16", "ragged"])
def test_workloads_match_oracle(cfg):
    say(f"accept from logits, workload {cfg}")
    x = inputs(cfg)
    check(x["target_logits"].numpy(), x["draft_logits"].numpy(), x["draft"].numpy(), x["tau"].numpy(),
          x["u"].numpy(), 1.0, cfg)


def random_logits(V, b, B=8, seed=0, spread=2.0, noise=1.0):
    rng = np.random.default_rng(seed)
    zt = (rng.standard_normal((b, B, V)) * spread).astype(np.float32)
    zd = (zt + rng.standard_normal((b, B, V)) * noise).astype(np.float32)
    draft = rng.integers(0, V, (b, B)).astype(np.int32)
    tau = np.stack([rng.permutation(B) + 1 for _ in range(b)]).astype(np.int32)
    u = rng.random((b, B + 1)).astype(np.float32)
    return zt, zd, draft, tau, u


@pytest.mark.parametrize("V,b,T", [(7, 64, 1.0), (5001, 32, 0.6), (32768, 32, 1.7), (151936, 8, 1.0),
                                   (8192, 16, 0.25)])
def test_random_logits_and_temperatures(V, b, T):
    say(f"accept from logits V={V} b={b} T={T}")
    check(*random_logits(V, b, seed=V + b), T, f"V={V} T={T}")


def test_workspace_left_zero_and_reused():
    V, b, B = 10000, 8, 8
    need = binding.simsd_accept_logits_workspace(b, B, V)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for seed in (1, 2, 3):
        check(*random_logits(V, b, B, seed=seed), 1.0, f"reuse {seed}", ws=ws)
        # counters, ready words and row statistics are all zero again
        assert int(torch.count_nonzero(ws)) == 0


@pytest.mark.parametrize("V,b,B", [(4097, 4, 64), (32768, 3, 64), (1000, 64, 1)])
def test_block_sizes_and_workspace_left_zero(V, b, B):
    # B = 64: all 256 threads of a workgroup clear the sequence's 4 B row
    # statistics; B = 1: a single step per sequence
    say(f"accept from logits V={V} b={b} B={B}")
    need = binding.simsd_accept_logits_workspace(b, B, V)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for seed in (1, 2):
        check(*random_logits(V, b, B, seed=seed + V + B), 1.0, f"V={V} b={b} B={B}", ws=ws)
        assert int(torch.count_nonzero(ws)) == 0


def test_workspace_reused_across_sizes():
    # one buffer sized for the largest call, then calls at other sizes: what a
    # call leaves behind must never land in another layout's counters or
    # ready words (statistics of 2 b B rows sit at a size-dependent offset)
    sizes = [(151936, 8, 8), (20480, 16, 8), (151936, 4, 16), (4097, 32, 4), (151936, 8, 8), (64, 2, 3)]
    need = max(binding.simsd_accept_logits_workspace(b, B, V) for V, b, B in sizes)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for i, (V, b, B) in enumerate(sizes):
        say(f"shared workspace, call {i}: V={V} b={b} B={B}")
        check(*random_logits(V, b, B, seed=100 + i, spread=3.0), 1.0, f"shared ws V={V} b={b}", ws=ws)
        assert int(torch.count_nonzero(ws)) == 0


def test_edge_cases():
    rng = np.random.default_rng(4)
    V, B, b = 64, 6, 6
    zt = rng.standard_normal((b, B, V)).astype(np.float32)
    zd = zt.copy()  # p == q: every step accepted
    draft = rng.integers(0, V, (b, B)).astype(np.int32)
    tau = np.stack([rng.permutation(B) + 1 for _ in range(b)]).astype(np.int32)
    u = rng.random((b, B + 1)).astype(np.float32)
    L, corr = check(zt, zd, draft, tau, u, 1.0, "p == q")
    assert (L == B).all() and (corr == -1).all()
    tau2 = tau.copy()
    tau2[0, :2] = 1  # not a permutation
    draft2 = draft.copy()
    draft2[1, np.argsort(tau[1])[0]] = V + 3  # draft id out of range
    zd2 = zd.copy()
    k = np.argsort(tau[2])[0]
    zd2[2, k, :] = -1e30
    zd2[2, k, draft[2, k]] = 0.0  # q one-hot at the draft, p(x) < 1: residual draw from p
    check(zt, zd2, draft2, tau2, u, 1.0, "status cases")
    one = np.zeros((3, 2, 1), np.float32)
    check(one, one, np.zeros((3, 2), np.int32), np.tile(np.array([[2, 1]], np.int32), (3, 1)),
          rng.random((3, 3)).astype(np.float32), 1.0, "V=1")


def test_one_launch_edge_cases():
    # 2 b B V / 4096 >= 4096 statistics workgroups: statistics and acceptance
    # run in one launch, the acceptance waiting for its sequence's published
    # statistics. A draft id outside the vocabulary has no logit word to wait
    # for; a bad tau, a one-hot q and p == q take their usual paths; the
    # workspace is left zero for the next call.
    V, b, B = 32768, 32, 8
    zt, zd, draft, tau, u = random_logits(V, b, B, seed=11)
    tau[0, :2] = 1  # not a permutation
    draft[1, np.argsort(tau[1])[0]] = V + 3  # draft id out of range at step 1
    draft[2, np.argsort(tau[2])[2]] = -1  # out of range at step 3
    k = np.argsort(tau[3])[0]
    zd[3, k, :] = -1e30
    zd[3, k, draft[3, k]] = 0.0  # q one-hot at the draft, p(x) < 1: residual draw from p
    zd[4] = zt[4]  # p == q: every step accepted
    need = binding.simsd_accept_logits_workspace(b, B, V)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for rep in range(2):
        L, corr = check(zt, zd, draft, tau, u, 1.0, f"one launch, status cases {rep}", ws=ws)
        assert L[4] == B and corr[4] == -1
        assert int(torch.count_nonzero(ws)) == 0


def _one_launch_shapes(n, seed):
    # random (b, B, V, T) whose statistics grid, 2 b B ceil(V / 4096)
    # workgroups, is at least 4096 (the one-launch form), logits <= 96 MB
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        b = int(rng.integers(1, 65))
        B = int(rng.choice([1, 3, 8, 16, 33, 64]))
        V = int(rng.integers(1000, 200000))
        units = 2 * b * B * -(-V // 4096)
        if units >= 4096 and 2 * b * B * V * 4 <= 96 << 20:
            out.append((b, B, V, float(rng.choice([0.5, 1.0, 1.3]))))
    return out


@pytest.mark.parametrize("b,B,V,T", _one_launch_shapes(8, 2026))
def test_one_launch_random_shapes(b, B, V, T):
    # statistics and acceptance in one launch over random batch, block and
    # vocabulary sizes (ragged last segments included); the workspace is left
    # zero after each call
    say(f"one launch b={b} B={B} V={V} T={T}")
    need = binding.simsd_accept_logits_workspace(b, B, V)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    check(*random_logits(V, b, B, seed=b * 1000 + B + V), T, f"one launch b={b} B={B} V={V}", ws=ws)
    assert int(torch.count_nonzero(ws)) == 0


@pytest.mark.parametrize("V,b,per", [(151936, 8, 16), (151936, 8, 64), (20480, 16, 64), (12289, 4, 16),
                                     (4097, 32, 64)])
def test_row_statistics_segment_widths(V, b, per):
    # a row's maximum and sum of exp do not depend on how the statistics pass
    # cuts the row into segments (256 per entries each, folded by the row's
    # last arrival); V=4097 leaves a one-entry last segment
    say(f"accept from logits V={V} b={b}, row-statistics segments of {256 * per}")
    with binding.tuning(rowstat_per=per):
        check(*random_logits(V, b, seed=per + V, spread=3.0), 1.0, f"V={V} per={per}")
