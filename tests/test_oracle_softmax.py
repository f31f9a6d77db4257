"""Pins of the oracle's row softmax (the distribution the acceptance step reads
from the verification logits, [nl]/[fr] Methodologie 4) and of its logits
acceptance, independent of the oracle's own code: scipy's softmax, closed
forms, exact identities and limits."""
import numpy as np
import pytest
from scipy.special import softmax as sp_softmax

import oracle


def ulps32(a, b):
    a = np.asarray(a, np.float32)
    b = np.asarray(b, np.float32)
    return np.abs(a.astype(np.float64) - b.astype(np.float64)) / np.spacing(np.maximum(np.abs(a), np.abs(b)))


@pytest.mark.parametrize("T", [1.0, 0.7, 2.5])
def test_matches_scipy(T):
    rng = np.random.default_rng(11)
    z = (rng.standard_normal((6, 3000)) * 3.0).astype(np.float32)
    got = oracle.softmax_rows(z, T)
    ref = sp_softmax(z.astype(np.float64) / T, axis=-1)
    assert ulps32(got, ref.astype(np.float32)).max() <= 1.0


def test_uniform_and_two_valued_rows():
    V = 1000
    z = np.zeros((2, V), np.float32)
    z[1, 7] = 2.0
    got = oracle.softmax_rows(z, 1.0)
    assert np.all(got[0] == np.float32(1.0 / V))
    e = np.exp(2.0)
    assert got[1, 7] == np.float32(e / (e + V - 1))
    assert got[1, 0] == np.float32(1.0 / (e + V - 1))


def test_shift_and_temperature_identities_exact():
    rng = np.random.default_rng(5)
    # multiples of 2^-10 in [-4, 4]: adding 8 and halving are exact in fp32
    z = (rng.integers(-4096, 4096, (4, 700)) / 1024.0).astype(np.float32)
    base = oracle.softmax_rows(z, 1.0)
    assert np.array_equal(oracle.softmax_rows(z + np.float32(8.0), 1.0), base)
    assert np.array_equal(oracle.softmax_rows(z, 2.0), oracle.softmax_rows(z / np.float32(2.0), 1.0))


def test_temperature_limits():
    rng = np.random.default_rng(9)
    z = rng.permutation(np.arange(64, dtype=np.float32)).reshape(1, 64) * np.float32(0.25)
    hot = oracle.softmax_rows(z, 1e6)
    assert np.abs(hot - 1 / 64).max() < 1e-6
    cold = oracle.softmax_rows(z, 1e-3)
    assert cold[0, np.argmax(z)] == 1.0 and cold.sum() == 1.0


def test_rows_sum_to_one():
    rng = np.random.default_rng(2)
    z = (rng.standard_normal((8, 32768)) * 2.0).astype(np.float32)
    s = oracle.softmax_rows(z, 1.0).astype(np.float64).sum(-1)
    assert np.abs(s - 1.0).max() < 32768 * 2 ** -24


def test_accept_logits_is_softmax_then_accept():
    # the logits form must make exactly the decisions of accept() on the
    # oracle's own probabilities, and with T = 1 on the workload's logits the
    # probabilities the input generator computed
    from masked_attention_simsd_amd import synth
    x = synth.make_inputs("tiny")
    zt, zd = x["target_logits"].numpy(), x["draft_logits"].numpy()
    out = oracle.accept_logits(zt, zd, 1.0, x["draft"].numpy(), x["tau"].numpy(), x["u"].numpy())
    assert ulps32(out["p"], x["p"].numpy()).max() <= 1.0
    assert ulps32(out["q"], x["q"].numpy()).max() <= 1.0
    ref = oracle.accept(out["p"], out["q"], x["draft"].numpy(), x["tau"].numpy(), x["u"].numpy())
    for k in ("accept_len", "correction", "status", "boundary"):
        assert np.array_equal(out[k], ref[k])


def test_accept_logits_ratio_boundary_flag():
    # a uniform placed exactly on a step's ratio is flagged
    V, B = 16, 2
    zt = np.zeros((1, B, V), np.float32)
    zd = np.zeros((1, B, V), np.float32)
    zd[0, :, 3] = 1.0  # q(3) > p(3): ratio < 1
    draft = np.full((1, B), 3, np.int32)
    tau = np.array([[1, 2]], np.int32)
    p = oracle.softmax_rows(zt)
    q = oracle.softmax_rows(zd)
    r = np.float32(p[0, 0, 3] / q[0, 0, 3])
    u = np.array([[r, 0.5, 0.5]], np.float32)
    out = oracle.accept_logits(zt, zd, 1.0, draft, tau, u)
    assert out["ratio_boundary"][0] == 1
    u[0, 0] = np.float32(0.01)
    assert oracle.accept_logits(zt, zd, 1.0, draft, tau, u)["ratio_boundary"][0] == 0
