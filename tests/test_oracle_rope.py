"""Pins of the fp64 re-rotation oracle: hand-worked values, complex arithmetic, group laws."""
import os

import numpy as np
import pytest

from oracle import rope

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(seed, *shape):
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(shape)


def test_hand_worked_D4_values():
    rows = np.loadtxt(os.path.join(GOLDEN, "rope_D4.txt"))
    for row in rows:
        d = row[0]
        x = rope.rotate(np.array([1.0, 0, 0, 0]), d, 10000.0)
        y = rope.rotate(np.array([0, 0, 0, 1.0]), d, 10000.0)
        np.testing.assert_allclose(x, row[1:5], rtol=0, atol=1e-14)
        np.testing.assert_allclose(y, row[5:9], rtol=0, atol=1e-14)


@pytest.mark.parametrize("style", [rope.ROTATE_HALF, rope.INTERLEAVED])
def test_equals_complex_multiplication(style):
    D, base = 16, 1e6
    x = rnd(1, 5, D)
    delta = np.array([0, 1, -7, 12345, 131072])
    a, b = rope.pair_index(D, style)
    z = (x[:, a] + 1j * x[:, b]) * np.exp(1j * delta[:, None] * base ** (-np.arange(D // 2) * 2.0 / D))
    got = rope.rotate(x, delta, base, style)
    np.testing.assert_allclose(got[:, a], z.real, rtol=0, atol=1e-12)
    np.testing.assert_allclose(got[:, b], z.imag, rtol=0, atol=1e-12)


def test_group_laws_and_norm():
    D, base = 128, 1e6
    x = rnd(2, 3, D)
    for p, d in [(5, 9), (-100, 7), (131072 - 8192, 4096), (0, 0)]:
        np.testing.assert_allclose(rope.rotate(rope.rotate(x, p, base), d, base), rope.rotate(x, p + d, base),
                                   rtol=0, atol=1e-10)
        np.testing.assert_allclose(rope.rotate(rope.rotate(x, d, base), -d, base), x, rtol=0, atol=1e-12)
        np.testing.assert_allclose(np.linalg.norm(rope.rotate(x, d, base), axis=-1), np.linalg.norm(x, axis=-1),
                                   rtol=1e-14)


def test_relative_position_property():
    """<R(p) q, R(r) k> depends only on p - r: the reason moving a document by delta is one rotation."""
    D, base = 64, 1e4
    q, k = rnd(3, D), rnd(4, D)
    for p, r in [(10, 3), (1000, 999), (5, 50)]:
        lhs = rope.rotate(q, p, base) @ rope.rotate(k, r, base)
        rhs = rope.rotate(q, p - r, base) @ k
        assert abs(lhs - rhs) < 1e-10


def test_frequencies_closed_form():
    th = rope.inv_freq(128, 1e6)
    assert th[0] == 1.0
    assert abs(th[-1] - 1e6 ** (-126 / 128)) < 1e-20
    assert np.all(np.diff(th) < 0)


def test_rerotation_from_offline_position_equals_direct_rope_at_actual_position():
    """A key rotated at offline position o and moved by delta equals the key rotated directly at o + delta."""
    D, base = 128, 1e6
    k_raw = rnd(5, 4, D)
    o = np.array([0, 17, 90000, 3])
    delta = np.array([122880, -17, 100, 0])
    offline = rope.rotate(k_raw, o, base)
    np.testing.assert_allclose(rope.rotate(offline, delta, base), rope.rotate(k_raw, o + delta, base),
                               rtol=0, atol=1e-9)


def test_interleaved_is_a_channel_permutation_of_rotate_half():
    D = 8
    x = rnd(6, D)
    perm = np.empty(D, int)
    perm[0::2] = np.arange(D // 2)
    perm[1::2] = np.arange(D // 2) + D // 2
    np.testing.assert_allclose(rope.rotate(x[perm], 33, 500.0, rope.INTERLEAVED),
                               rope.rotate(x, 33, 500.0, rope.ROTATE_HALF)[perm], rtol=0, atol=1e-15)
