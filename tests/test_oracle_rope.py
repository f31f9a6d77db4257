"""Pins for the oracle's RoPE-copy (CPU only).

Copy rule: SimSD pages, Methodologie 3 (position-encoding alignment), each
mask slot reuses the RoPE index of its paired data token. The rotation is the
standard rotary embedding; these tests pin it with an independent complex
number formulation and its closed-form properties.
"""
import numpy as np
import pytest

import oracle


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _complex_rope(x, start_pos, base, no_copy=False):
    """Rotate-half RoPE as multiplication by e^{i pos theta_k} on z = x_k + i x_{k+d/2}."""
    b, twoB, H, d = x.shape
    B = twoB // 2
    half = d // 2
    out = np.empty_like(x)
    theta = base ** (-np.arange(half) * 2.0 / d)
    for s in range(b):
        for r in range(twoB):
            k = r % B
            pos = start_pos[s] + k + (B if (no_copy and r >= B) else 0)
            z = x[s, r, :, :half] + 1j * x[s, r, :, half:]
            z = z * np.exp(1j * pos * theta)[None, :]
            out[s, r, :, :half] = z.real
            out[s, r, :, half:] = z.imag
    return out


@pytest.mark.parametrize("d", [8, 64, 128])
def test_matches_complex_formulation(d):
    x = _rand((2, 8, 3, d), d)
    sp = np.array([0, 1234])
    y = oracle.rope_copy(x, sp, base=10000.0)
    np.testing.assert_allclose(y, _complex_rope(x, sp, 10000.0), atol=1e-12, rtol=0)
    y2 = oracle.rope_copy(x, sp, base=500.0, no_copy=True)
    np.testing.assert_allclose(y2, _complex_rope(x, sp, 500.0, no_copy=True), atol=1e-12, rtol=0)


def test_position_zero_is_identity_and_d2_closed_form():
    x = _rand((1, 2, 1, 4), 1)
    y = oracle.rope_copy(x, [0], base=10000.0)  # B = 1: both rows at position 0
    assert np.array_equal(y, x)
    # d = 2: a single frequency 1, so position p rotates (1, 0) to (cos p, sin p)
    e = np.zeros((1, 6, 1, 2))
    e[..., 0] = 1.0
    y = oracle.rope_copy(e, [5], base=10000.0)
    for r in range(6):
        pos = 5 + r % 3
        np.testing.assert_allclose(y[0, r, 0], [np.cos(pos), np.sin(pos)], atol=1e-15)


def test_pair_norms_preserved_and_relative_position():
    d = 64
    x = _rand((1, 8, 2, d), 2)
    y = oracle.rope_copy(x, [77])
    n = lambda v: v[..., : d // 2] ** 2 + v[..., d // 2:] ** 2
    np.testing.assert_allclose(n(y), n(x), rtol=1e-12)
    # <R_m q, R_n k> depends only on m - n
    q, k = _rand((d,), 3), _rand((d,), 4)

    def rot(v, pos):
        z = np.zeros((1, 2, 1, d))
        z[0, 0, 0] = v
        return oracle.rope_copy(z, [pos])[0, 0, 0]

    a = rot(q, 10) @ rot(k, 3)
    b = rot(q, 1010) @ rot(k, 1003)
    assert abs(a - b) < 1e-10
    assert abs(a - rot(q, 10) @ rot(k, 4)) > 1e-6


def test_interleaved_is_rotate_half_on_permuted_dims():
    d = 16
    x = _rand((1, 6, 2, d), 5)
    perm = np.concatenate([np.arange(0, d, 2), np.arange(1, d, 2)])  # (2i, 2i+1) -> (i, i+d/2)
    y_half = oracle.rope_copy(x[..., perm], [9])
    y_int = oracle.rope_copy(x, [9], interleaved=True)
    np.testing.assert_allclose(y_int[..., perm], y_half, atol=1e-14)


def test_copy_rule_pairs_get_identical_rotation():
    # D_k and ~D_k share a position, so identical input vectors must give
    # bit-identical outputs; without the copy they sit B positions apart.
    B, d = 4, 32
    x = _rand((2, 2 * B, 3, d), 6)
    x[:, B:] = x[:, :B]
    y = oracle.rope_copy(x, [0, 500])
    assert np.array_equal(y[:, :B], y[:, B:])
    y2 = oracle.rope_copy(x, [0, 500], no_copy=True)
    assert not np.allclose(y2[:, :B], y2[:, B:])
