"""Pins of the oracle's RoPE: the 4-element toy of the atyun explainer [RoPE]
(pairs (x1,x2), (x3,x4) rotated by theta_0 and 2*theta_0), checked against
complex multiplication; plus properties every rotary embedding has."""
import cmath
import math

import numpy as np
import pytest

from oracle import rope, rope_frequencies, rotate_pairs


def _complex_rotate(x, angles):
    """Independent formulation: pair (a, b) is the complex number a + ib times e^{i phi}."""
    out = []
    for k, phi in enumerate(angles):
        z = complex(x[2 * k], x[2 * k + 1]) * cmath.exp(1j * phi)
        out += [z.real, z.imag]
    return out


def test_toy_four_vector():
    x = [0.3, -1.2, 2.0, 0.7]
    th0 = 0.37
    got = rotate_pairs(np.array(x), np.array([th0, 2 * th0]))
    np.testing.assert_allclose(got, _complex_rotate(x, [th0, 2 * th0]), rtol=0, atol=1e-15)


def test_rotation_sense():
    # a quarter turn takes the first axis onto the second (counter-clockwise)
    got = rotate_pairs(np.array([1.0, 0.0]), np.array([math.pi / 2]))
    np.testing.assert_allclose(got, [0.0, 1.0], atol=1e-15)


def test_frequencies():
    th = rope_frequencies(64, 10000.0)
    assert th.shape == (32,)
    assert th[0] == 1.0
    np.testing.assert_allclose(th[-1], 10000.0 ** (-62 / 64), rtol=1e-15)
    np.testing.assert_allclose(th[1:] / th[:-1], 10000.0 ** (-2 / 64), rtol=1e-14)
    with pytest.raises(ValueError):
        rope_frequencies(7, 10000.0)


def test_position_one_first_pair_turns_one_radian():
    x = np.zeros(8); x[0] = 1.0
    got = rope(x, 1, 10000.0)
    np.testing.assert_allclose(got[:2], [math.cos(1.0), math.sin(1.0)], atol=1e-15)


def test_matches_complex_form_random():
    rng = np.random.default_rng(5)
    x = rng.standard_normal(64)
    for pos in [0, 1, 17, 4095, 131071]:
        th = rope_frequencies(64, 10000.0) * pos
        np.testing.assert_allclose(rope(x, pos, 10000.0), _complex_rotate(list(x), list(th)),
                                   rtol=0, atol=1e-12)


def test_identity_norm_composition_relative():
    rng = np.random.default_rng(1)
    q = rng.standard_normal(64)
    k = rng.standard_normal(64)
    np.testing.assert_array_equal(rope(q, 0, 10000.0), q)
    r = rope(q, 12345, 10000.0)
    np.testing.assert_allclose(np.hypot(r[0::2], r[1::2]), np.hypot(q[0::2], q[1::2]), rtol=1e-14)
    np.testing.assert_allclose(rope(rope(q, 40, 10000.0), 2, 10000.0), rope(q, 42, 10000.0), atol=1e-13)
    for m, n in [(7, 3), (100, 250), (4095, 0)]:
        lhs = rope(q, m, 10000.0) @ rope(k, n, 10000.0)
        rhs = rope(q, m - n, 10000.0) @ k
        assert abs(lhs - rhs) < 1e-11


def test_batched_positions_broadcast():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, 8))
    pos = np.arange(5) * 3
    got = rope(x, pos, 10000.0)
    for i in range(5):
        np.testing.assert_allclose(got[i], rope(x[i], pos[i], 10000.0), rtol=0, atol=0)
