"""Pins of the round loop's position bookkeeping (oracle.next_positions,
oracle.committed_positions) and of RoPE-copy at explicit positions.

Each pair (D_k, D~_k) is one response position and D~_k takes D_k's RoPE index
([nl]/[fr] Methodologie 1 and 3); the longest prefix accepted along the
temporal order is committed and the process repeats ([nl]/[fr] Methodologie
4). The pins: a hand-derived round (tests/golden/rounds_B4_tau2413.txt);
closed forms for L = 0, L = B and the identity order; the B smallest
uncached positions found by brute force; over several rounds with partial
acceptance the committed and next-round positions covering a contiguous range
exactly once; and RoPE at explicit positions equal to an independent
complex-number rotation row by row."""
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "rounds_B4_tau2413.txt")


def _golden():
    rows = {}
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        k, *v = line.split()
        rows[k] = [int(t) for t in v]
    return rows


def test_hand_derived_round():
    g = _golden()
    pos = np.array([g["pos"]], np.int32)
    tau = np.array([g["tau"]], np.int32)
    L = np.array(g["L"], np.int32)
    assert oracle.committed_positions(pos, tau, L) == [g["committed"]]
    assert oracle.next_positions(pos, tau, L)[0].tolist() == g["next"]


def test_all_accepted_opens_the_next_block():
    rng = np.random.default_rng(0)
    B = 6
    pos = np.array([rng.permutation(B) + 50], np.int32)
    tau = np.array([rng.permutation(B) + 1], np.int32)
    nxt = oracle.next_positions(pos, tau, [B])
    assert nxt[0].tolist() == list(range(56, 62))
    assert sorted(oracle.committed_positions(pos, tau, [B])[0]) == list(range(50, 56))


def test_nothing_accepted_keeps_the_block_with_the_correction_first():
    B = 5
    pos = np.array([[10, 11, 12, 13, 14]], np.int32)
    tau = np.array([[3, 5, 1, 4, 2]], np.int32)  # step 1 is position 12
    assert oracle.next_positions(pos, tau, [0])[0].tolist() == [12, 10, 11, 13, 14]
    assert oracle.committed_positions(pos, tau, [0]) == [[]]


@pytest.mark.parametrize("L", range(0, 9))
def test_identity_order_slides_like_token_by_token_decoding(L):
    B, P = 8, 300
    pos = np.array([np.arange(P, P + B)], np.int32)
    tau = np.array([np.arange(1, B + 1)], np.int32)
    assert oracle.committed_positions(pos, tau, [L])[0] == list(range(P, P + L))
    assert oracle.next_positions(pos, tau, [L])[0].tolist() == list(range(P + L, P + B + L))


def test_bad_tau_or_length_keeps_the_block():
    pos = np.array([[5, 6, 7], [8, 9, 10], [1, 2, 3]], np.int32)
    tau = np.array([[1, 1, 3], [1, 2, 3], [3, 2, 1]], np.int32)
    nxt = oracle.next_positions(pos, tau, [1, 4, -1])
    assert np.array_equal(nxt, pos)


def _play(rng, B, P, rounds, tau_fn):
    """Several rounds from a prefix of P positions: returns per round (pos,
    tau, L, cached set before the round)."""
    cached = set(range(P))
    pos = np.array([np.arange(P, P + B)], np.int32)
    hist = []
    for r in range(rounds):
        tau = np.array([tau_fn(r)], np.int32)
        L = int(rng.integers(0, B + 1))
        hist.append((pos.copy(), tau, L, set(cached)))
        committed = oracle.committed_positions(pos, tau, [L])[0]
        assert not (set(committed) & cached), "a position committed twice"
        cached |= set(committed)
        pos = oracle.next_positions(pos, tau, [L])
    return hist, cached, pos


@pytest.mark.parametrize("seed", range(12))
def test_next_block_is_the_smallest_uncached_positions(seed):
    rng = np.random.default_rng(seed)
    B, P = int(rng.integers(1, 10)), int(rng.integers(0, 40))
    hist, cached, nxt = _play(rng, B, P, 6, lambda r: rng.permutation(B) + 1)
    for pos, tau, L, before in hist:
        free = [p for p in range(P, P + 100 * B) if p not in before]
        assert sorted(pos[0].tolist()) == free[:B]
    free = [p for p in range(P, P + 100 * B) if p not in cached]
    assert sorted(nxt[0].tolist()) == free[:B]


@pytest.mark.parametrize("seed", range(8))
def test_rounds_with_partial_acceptance_cover_the_positions_once(seed):
    # tau != identity and 0 < L < B in every round: the committed positions
    # plus the next round's positions are exactly P .. max(next), each once,
    # and the rejected step's position leads the next block
    rng = np.random.default_rng(100 + seed)
    B, P = 8, 4096
    cached, pos = [], np.array([np.arange(P, P + B)], np.int32)
    for r in range(3):
        tau = np.array([rng.permutation(B) + 1], np.int32)
        while (tau[0] == np.arange(1, B + 1)).all():
            tau = np.array([rng.permutation(B) + 1], np.int32)
        L = int(rng.integers(1, B))
        inv = np.argsort(tau[0])
        cached += oracle.committed_positions(pos, tau, [L])[0]
        nxt = oracle.next_positions(pos, tau, [L])
        seen = cached + nxt[0].tolist()
        assert len(nxt[0]) == B
        assert len(seen) == len(set(seen)), "a position appears twice"
        assert sorted(seen) == list(range(P, max(seen) + 1)), "a position is skipped"
        assert nxt[0, 0] == pos[0, inv[L]]
        pos = nxt


def _complex_rope_rows(x, positions, base):
    """Rotate-half RoPE as a complex multiplication, each block row at the
    position given for its pair: x [b][2B][H][d], positions [b][B]."""
    b, twoB, H, d = x.shape
    B = twoB // 2
    half = d // 2
    freq = base ** (-2.0 * np.arange(half) / d)
    y = np.empty_like(x)
    for s in range(b):
        for r in range(twoB):
            z = x[s, r, :, :half] + 1j * x[s, r, :, half:]
            z = z * np.exp(1j * positions[s, r % B] * freq)
            y[s, r, :, :half], y[s, r, :, half:] = z.real, z.imag
    return y


@pytest.mark.parametrize("d", [8, 64])
def test_rope_at_explicit_positions_matches_complex_rotation(d):
    rng = np.random.default_rng(d)
    b, B, H = 3, 5, 2
    x = rng.standard_normal((b, 2 * B, H, d))
    positions = rng.integers(0, 70000, size=(b, B)).astype(np.int32)
    y = oracle.rope_copy(x, positions, 10000.0)
    # angles reach 7e4 rad, whose fp64 rounding alone moves cos / sin by ~1e-11
    np.testing.assert_allclose(y, _complex_rope_rows(x, positions, 10000.0), atol=1e-9, rtol=0)
    # D_k and D~_k get the same angles: identical inputs give identical outputs
    x2 = x.copy()
    x2[:, B:] = x2[:, :B]
    y2 = oracle.rope_copy(x2, positions, 10000.0)
    assert np.array_equal(y2[:, B:], y2[:, :B])


def test_consecutive_positions_equal_the_start_position_form():
    rng = np.random.default_rng(9)
    b, B, H, d = 2, 4, 3, 16
    x = rng.standard_normal((b, 2 * B, H, d))
    sp = np.array([7, 1000], np.int32)
    positions = (sp[:, None] + np.arange(B)[None, :]).astype(np.int32)
    for inter in (False, True):
        assert np.array_equal(oracle.rope_copy(x, positions, 500.0, interleaved=inter),
                              oracle.rope_copy(x, sp, 500.0, interleaved=inter))
    with pytest.raises(ValueError):
        oracle.rope_copy(x, positions, 500.0, no_copy=True)
