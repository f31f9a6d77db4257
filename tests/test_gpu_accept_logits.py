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
    rows = 2 * b * B
    nseg1 = (V + 4095) // 4096
    need = binding.simsd_accept_logits_workspace(b, B, V)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for seed in (1, 2, 3):
        check(*random_logits(V, b, B, seed=seed), 1.0, f"reuse {seed}", ws=ws)
    # everything but the row statistics (the last rows * 16 bytes) is zero again
    stats_bytes = (rows * 16 + 255) // 256 * 256
    assert int(torch.count_nonzero(ws[: need - stats_bytes])) == 0


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
