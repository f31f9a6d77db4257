"""Pins for the oracle's temporal mask (CPU only).

The mask rule comes from the SimSD pages, Methodologie 2 (temporal attention
mask) on both the Dutch and the French technical summary. The rule for data
token rows is this build's reading; only the hand-derived fixture and the
counting identities below pin it.
"""
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mask_B4_tau2413.txt")


def _read_golden():
    tau, rules, cur = None, {}, None
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        if line.startswith("tau"):
            tau = [int(x) for x in line.split()[1:]]
        elif line.startswith("rule"):
            cur = line.split()[1]
            rules[cur] = []
        else:
            rules[cur].append([c == "1" for c in line])
    return tau, {k: np.array(v) for k, v in rules.items()}


def test_mask_matches_hand_derived_fixture():
    tau, rules = _read_golden()
    assert np.array_equal(oracle.mask_matrix(tau, oracle.DATA_CAUSAL), rules["causal"])
    assert np.array_equal(oracle.mask_matrix(tau, oracle.DATA_BIDIR), rules["bidir"])


@pytest.mark.parametrize("B", [1, 2, 3, 5, 8, 16])
def test_mask_slot_sees_exactly_B_block_keys(B):
    # #{j: tau(j) < tau(i)} + #{j: tau(j) >= tau(i)} = B for every i and tau.
    rng = np.random.default_rng(B)
    for _ in range(5):
        tau = rng.permutation(B) + 1
        m = oracle.mask_matrix(tau)
        assert (m[B:].sum(axis=1) == B).all()
        # data rows under the causal reading see tau(i) data keys and no slot
        assert (m[:B, :B].sum(axis=1) == tau).all()
        assert not m[:B, B:].any()
        # every mask slot sees itself, never a data token of its own step
        for i in range(B):
            assert m[B + i, B + i]
            assert not m[B + i, i]


@pytest.mark.parametrize("B", [2, 4, 7])
def test_mask_permutation_equivariance(B):
    # Relabelling positions by pi (tau' = tau o pi^-1) permutes the mask rows
    # and columns of both sections the same way.
    rng = np.random.default_rng(10 + B)
    for _ in range(5):
        tau = rng.permutation(B) + 1
        pi = rng.permutation(B)  # position k moves to pi[k]
        tau2 = np.empty(B, dtype=np.int64)
        tau2[pi] = tau
        full = np.concatenate([pi, pi + B])
        for rule in (oracle.DATA_CAUSAL, oracle.DATA_BIDIR):
            m, m2 = oracle.mask_matrix(tau, rule), oracle.mask_matrix(tau2, rule)
            assert np.array_equal(m2[np.ix_(full, full)], m)


def test_identity_and_reversed_tau_give_staircases():
    B = 5
    ident = oracle.mask_matrix(np.arange(1, B + 1))
    lower_strict = np.tril(np.ones((B, B), dtype=bool), -1)
    upper = np.triu(np.ones((B, B), dtype=bool))
    # identity order: ~D_i sees D_{<i} and ~D_{>=i} (autoregressive-like)
    assert np.array_equal(ident[B:, :B], lower_strict)
    assert np.array_equal(ident[B:, B:], upper)
    rev = oracle.mask_matrix(np.arange(B, 0, -1))
    assert np.array_equal(rev[B:, :B], lower_strict.T)
    assert np.array_equal(rev[B:, B:], upper.T)


def test_B1_slot_sees_only_itself():
    m = oracle.mask_matrix([1])
    assert np.array_equal(m, np.array([[True, False], [False, True]]))


def test_tau_inverse_and_validation():
    inv, ok = oracle.tau_inverse([2, 4, 1, 3])
    assert ok and list(inv) == [2, 0, 3, 1]
    for bad in ([1, 1, 2], [0, 1, 2], [1, 2, 4]):
        assert not oracle.tau_inverse(bad)[1]
