"""Pins of the RoPE oracle (oracle/rope_ref.py) to closed forms and identities
that a wrong sign, pairing, frequency or position would break."""
import math

import numpy as np
import pytest

from oracle import pack_ref, rope_ref


def _rng(seed=0):
    return np.random.default_rng(seed)


def test_position_zero_is_identity():
    x = _rng().standard_normal((5, 3, 16))
    np.testing.assert_array_equal(rope_ref.rope(x, np.zeros(5, np.int64)), x)


@pytest.mark.parametrize("p", [1, 2, 7, 1000, 131071])
def test_d2_closed_form(p):
    # D = 2: one pair with frequency base**0 = 1, so (1, 0) -> (cos p, sin p)
    # and (0, 1) -> (-sin p, cos p)
    x = np.array([[[1.0, 0.0]], [[0.0, 1.0]]])
    y = rope_ref.rope(x, np.array([p, p]))
    np.testing.assert_allclose(y[0, 0], [math.cos(p), math.sin(p)], rtol=0, atol=1e-12)
    np.testing.assert_allclose(y[1, 0], [-math.sin(p), math.cos(p)], rtol=0, atol=1e-12)


def test_d4_closed_form_frequencies():
    # D = 4, base 10000: pair 0 = dims (0, 2) turns by p, pair 1 = dims (1, 3)
    # by p * 10000**(-1/2) = p / 100
    p = 3
    x = np.array([[[1.0, 1.0, 0.0, 0.0]]])
    y = rope_ref.rope(x, np.array([p]))[0, 0]
    np.testing.assert_allclose(y, [math.cos(3), math.cos(0.03), math.sin(3), math.sin(0.03)], atol=1e-12)
    # another base
    y = rope_ref.rope(x, np.array([p]), base=400.0)[0, 0]
    np.testing.assert_allclose(y, [math.cos(3), math.cos(0.15), math.sin(3), math.sin(0.15)], atol=1e-12)


def test_matches_complex_multiplication():
    # z_i = x_i + j x_{i+D/2} multiplied by exp(j theta_i)
    rng = _rng(1)
    T, H, D = 9, 2, 32
    x = rng.standard_normal((T, H, D))
    pos = rng.integers(0, 5000, T)
    z = x[..., : D // 2] + 1j * x[..., D // 2:]
    theta = pos[:, None, None] * (10000.0 ** (-np.arange(0, D, 2) / D))[None, None, :]
    w = z * np.exp(1j * theta)
    y = rope_ref.rope(x, pos)
    np.testing.assert_allclose(y[..., : D // 2], w.real, atol=1e-12)
    np.testing.assert_allclose(y[..., D // 2:], w.imag, atol=1e-12)


def test_rotation_preserves_pair_norms_and_inverse_restores():
    rng = _rng(2)
    x = rng.standard_normal((7, 4, 64))
    pos = rng.integers(0, 40000, 7)
    y = rope_ref.rope(x, pos)
    n_x = x[..., :32] ** 2 + x[..., 32:] ** 2
    n_y = y[..., :32] ** 2 + y[..., 32:] ** 2
    np.testing.assert_allclose(n_y, n_x, rtol=1e-12)
    np.testing.assert_allclose(rope_ref.rope(y, pos, inverse=True), x, atol=1e-10)


def test_scores_depend_on_relative_position_only():
    rng = _rng(3)
    D = 16
    q = rng.standard_normal((1, 1, D))
    k = rng.standard_normal((1, 1, D))
    for m, n in [(5, 2), (100, 37), (9, 9)]:
        a = np.dot(rope_ref.rope(q, [m])[0, 0], rope_ref.rope(k, [n])[0, 0])
        b = np.dot(rope_ref.rope(q, [m - n + 11])[0, 0], rope_ref.rope(k, [11])[0, 0])
        assert abs(a - b) < 1e-10


def test_packed_row_equals_documents_rotated_alone():
    # positions from the packer's indexes restart per segment, so rotating the
    # packed row equals rotating each document alone from position 0
    rng = _rng(4)
    docs = [list(rng.integers(1, 50000, n)) for n in [5, 9, 3, 12, 7]]
    rows = pack_ref.build_pack(docs, 2, 8)
    T = sum(len(r["input_ids"]) for r in rows)
    idx = np.concatenate([r["indexes"] for r in rows])
    x = rng.standard_normal((T, 2, 8))
    y = rope_ref.rope(x, idx)
    p = 0
    for r in rows:
        cu = r["cu_seqlens"]
        for s, e in zip(cu[:-1], cu[1:]):
            alone = rope_ref.rope(x[p + s: p + e], np.arange(e - s))
            np.testing.assert_allclose(y[p + s: p + e], alone, atol=1e-12)
        p += len(r["input_ids"])
