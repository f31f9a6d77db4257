"""Pins of the oracle's KV commit (commit_kv) and region packing
(pack_regions): closed forms for identity / reversed temporal orders and for
L = 0 and L = B, one-token-at-a-time appends, untouched rows, the error
cases, and the context property that ties the commit to the temporal mask --
the first rejected data row (and its mask slot) attends over the committed
cache to exactly what it attended to in the round that rejected it."""
import numpy as np
import pytest

import oracle


def blocks(rng, b, B, Hkv, d):
    kb = rng.standard_normal((b, 2 * B, Hkv, d))
    vb = rng.standard_normal((b, 2 * B, Hkv, d))
    # mask-slot rows carry a sentinel: they must never reach the cache
    kb[:, B:] = 1e6
    vb[:, B:] = -1e6
    return kb, vb


def cache(rng, off, Hkv, d, head_major=False):
    C = int(off[-1])
    kc = rng.standard_normal((C, Hkv, d))
    vc = rng.standard_normal((C, Hkv, d))
    if head_major:
        return kc.transpose(1, 0, 2).copy(), vc.transpose(1, 0, 2).copy()
    return kc, vc


def one_at_a_time(kb, vb, tau, L, kc, vc, off, lens):
    """Append drafts one by one: at step t search tau for the label t."""
    kc, vc, lens = kc.copy(), vc.copy(), np.array(lens, copy=True)
    for s in range(tau.shape[0]):
        for t in range(1, L[s] + 1):
            k = [j for j in range(tau.shape[1]) if tau[s, j] == t][0]
            kc[off[s] + lens[s]] = kb[s, k]
            vc[off[s] + lens[s]] = vb[s, k]
            lens[s] += 1
    return kc, vc, lens


def test_identity_and_reversed_orders_are_slices():
    rng = np.random.default_rng(1)
    b, B, Hkv, d = 2, 6, 2, 8
    off = np.array([0, 20, 40], np.int32)
    lens = np.array([5, 0], np.int32)
    kb, vb = blocks(rng, b, B, Hkv, d)
    kc, vc = cache(rng, off, Hkv, d)
    tau = np.stack([np.arange(1, B + 1), np.arange(B, 0, -1)]).astype(np.int32)
    L = np.array([4, 3], np.int32)
    k2, v2, l2, st = oracle.commit_kv(kb, vb, tau, L, kc, vc, off, lens)
    assert st.tolist() == [0, 0] and l2.tolist() == [9, 3]
    assert np.array_equal(k2[5:9], kb[0, 0:4]) and np.array_equal(v2[5:9], vb[0, 0:4])
    assert np.array_equal(k2[20:23], kb[1, [5, 4, 3]]) and np.array_equal(v2[20:23], vb[1, [5, 4, 3]])


@pytest.mark.parametrize("head_major", [False, True])
def test_matches_one_at_a_time_and_leaves_the_rest(head_major):
    rng = np.random.default_rng(2)
    b, B, Hkv, d = 4, 8, 2, 8
    off = np.array([0, 30, 30, 55, 70], np.int32)  # sequence 1 has no room
    lens = np.array([10, 0, 17, 0], np.int32)
    kb, vb = blocks(rng, b, B, Hkv, d)
    kc, vc = cache(rng, off, Hkv, d)
    tau = np.stack([rng.permutation(B) + 1 for _ in range(b)]).astype(np.int32)
    L = np.array([0, 0, 8, 5], np.int32)
    ek, ev, el = one_at_a_time(kb, vb, tau, L, kc, vc, off, lens)
    if head_major:
        kch, vch = kc.transpose(1, 0, 2).copy(), vc.transpose(1, 0, 2).copy()
        k2, v2, l2, st = oracle.commit_kv(kb, vb, tau, L, kch, vch, off, lens, head_major=True)
        k2, v2 = k2.transpose(1, 0, 2), v2.transpose(1, 0, 2)
    else:
        k2, v2, l2, st = oracle.commit_kv(kb, vb, tau, L, kc, vc, off, lens)
    assert st.tolist() == [0, 0, 0, 0]
    assert np.array_equal(l2, el) and np.array_equal(k2, ek) and np.array_equal(v2, ev)
    # L = 0 leaves sequence 0 alone; L = B brings every data row of sequence 2, in tau order
    assert np.array_equal(k2[0:30], kc[0:30])
    assert sorted(map(tuple, k2[30 + 17:30 + 25].reshape(8, -1))) == sorted(map(tuple, kb[2, :B].reshape(8, -1)))
    assert (np.abs(k2) < 1e5).all() and (np.abs(v2) < 1e5).all()  # no mask-slot row
    # rows outside the appended ranges are the input's
    touched = np.zeros(int(off[-1]), bool)
    touched[47:55] = True
    touched[55:60] = True
    assert np.array_equal(k2[~touched], kc[~touched]) and np.array_equal(v2[~touched], vc[~touched])


def test_errors_leave_the_sequence_alone():
    rng = np.random.default_rng(3)
    b, B, Hkv, d = 4, 4, 1, 8
    off = np.array([0, 6, 12, 18, 24], np.int32)
    lens = np.array([3, 0, -1, 2], np.int32)
    kb, vb = blocks(rng, b, B, Hkv, d)
    kc, vc = cache(rng, off, Hkv, d)
    tau = np.array([[1, 2, 3, 4], [1, 1, 3, 4], [4, 3, 2, 1], [2, 1, 4, 3]], np.int32)
    L = np.array([4, 1, 1, 5], np.int32)  # 3 + 4 > 6; bad tau; negative length; L > B
    k2, v2, l2, st = oracle.commit_kv(kb, vb, tau, L, kc, vc, off, lens)
    assert st.tolist() == [oracle.COMMIT_OVERFLOW, oracle.BAD_TAU, oracle.COMMIT_OVERFLOW,
                           oracle.COMMIT_OVERFLOW]
    assert np.array_equal(l2, lens) and np.array_equal(k2, kc) and np.array_equal(v2, vc)
    # exactly full is fine
    k3, _, l3, st3 = oracle.commit_kv(kb, vb, tau, np.array([3, 0, 0, 0], np.int32), kc, vc, off,
                                      np.array([3, 0, 0, 0], np.int32))
    assert st3.tolist() == [0, oracle.BAD_TAU, 0, 0] and l3.tolist() == [6, 0, 0, 0]
    assert np.array_equal(k3[3:6], kb[0, 0:3])


def test_pack_regions_closed_forms():
    rng = np.random.default_rng(4)
    off = np.array([0, 5, 9, 16], np.int32)
    c = rng.standard_normal((16, 2, 4))
    full, po = oracle.pack_regions(c, off, np.diff(off))
    assert np.array_equal(full, c) and np.array_equal(po, off)
    none, po0 = oracle.pack_regions(c, off, np.zeros(3, np.int32))
    assert none.shape == (0, 2, 4) and po0.tolist() == [0, 0, 0, 0]
    part, pp = oracle.pack_regions(c, off, np.array([2, 0, 3], np.int32))
    assert np.array_equal(part, c[[0, 1, 9, 10, 11]]) and pp.tolist() == [0, 2, 2, 5]
    hm, _ = oracle.pack_regions(c.transpose(1, 0, 2), off, np.array([2, 0, 3], np.int32), head_major=True)
    assert np.array_equal(hm, part.transpose(1, 0, 2))


@pytest.mark.parametrize("seed", [5, 6, 7])
def test_committed_cache_is_the_context_of_the_first_rejected_draft(seed):
    rng = np.random.default_rng(seed)
    b, B, Hq, Hkv, d = 3, 6, 4, 2, 16
    P = np.array([0, 7, 19], np.int32)
    cap = P + B + 3
    off = np.zeros(b + 1, np.int32)
    off[1:] = np.cumsum(cap)
    q = rng.standard_normal((b, 2 * B, Hq, d))
    kb = rng.standard_normal((b, 2 * B, Hkv, d))
    vb = rng.standard_normal((b, 2 * B, Hkv, d))
    kc, vc = cache(rng, off, Hkv, d)
    tau = np.stack([rng.permutation(B) + 1 for _ in range(b)]).astype(np.int32)
    L = rng.integers(0, B, size=b).astype(np.int32)  # every sequence rejects at step L + 1
    kp, po = oracle.pack_regions(kc, off, P)
    vp, _ = oracle.pack_regions(vc, off, P)
    out, _ = oracle.verify_attention(q, kb, vb, kp, vp, po, tau)
    k2, v2, l2, st = oracle.commit_kv(kb, vb, tau, L, kc, vc, off, P)
    assert st.tolist() == [0] * b and np.array_equal(l2, P + L)
    kp2, po2 = oracle.pack_regions(k2, off, l2)
    vp2, _ = oracle.pack_regions(v2, off, l2)
    for s in range(b):
        k_star = int(np.nonzero(tau[s] == L[s] + 1)[0][0])
        rest = [j for j in range(B) if tau[s, j] >= L[s] + 1]
        # data row D_k*: the committed cache plus itself
        one = slice(s, s + 1)
        r_d, _ = oracle.attention_masked(q[one, [k_star]], kb[one, [k_star]], vb[one, [k_star]],
                                         kp2, vp2, np.array([po2[s], po2[s + 1]], np.int32),
                                         np.ones((1, 1, 1), bool))
        # mask slot D~_k*: the committed cache plus the slots of the drafts still open
        rows = [B + j for j in rest]
        slot = rows.index(B + k_star)
        r_m, _ = oracle.attention_masked(q[one][:, rows], kb[one][:, rows], vb[one][:, rows], kp2, vp2,
                                         np.array([po2[s], po2[s + 1]], np.int32),
                                         np.ones((1, len(rows), len(rows)), bool))
        assert np.abs(r_d[0, 0] - out[s, k_star]).max() < 1e-12
        assert np.abs(r_m[0, slot] - out[s, B + k_star]).max() < 1e-12
