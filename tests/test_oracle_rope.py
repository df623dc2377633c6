"""Pins for the RoPE oracle: closed-form frequencies and angles, the complex-number
formulation of rotate-half, the relative-position identity, and gather-by-value."""
import cmath
import math

import numpy as np

from oracle import rope


def test_inv_freq_closed_form():
    # D = 4, theta = 1e4: exponents 0 and -2/4 -> [1, 1e-2]
    assert np.allclose(rope.inv_freq(4, 1.0e4), [1.0, 0.01], rtol=0, atol=1e-15)
    # D = 8, theta = 1e4: [1, 1e-1, 1e-2, 1e-3]
    assert np.allclose(rope.inv_freq(8, 1.0e4), [1.0, 0.1, 0.01, 0.001], rtol=1e-14, atol=0)


def test_table_values():
    cos, sin = rope.table(4, 1.0e4, 100)
    assert cos.shape == (101, 2) and sin.shape == (101, 2)
    # position 1, j = 0: angle 1 rad; position 100, j = 1: angle 100 * 0.01 = 1 rad
    for (p, j) in [(1, 0), (100, 1)]:
        assert abs(cos[p, j] - 0.5403023058681398) < 1e-15
        assert abs(sin[p, j] - 0.8414709848078965) < 1e-15
    assert (cos[0] == 1).all() and (sin[0] == 0).all()


def test_rotate_half_equals_complex_multiplication():
    rng = np.random.default_rng(1)
    D, theta = 8, 500.0
    x = rng.standard_normal((5, 2, D))
    pos = np.array([0, 3, 17, 1000, 7])
    got = rope.rotate(x, pos, theta)
    for r in range(5):
        for h in range(2):
            for j in range(D // 2):
                z = complex(x[r, h, j], x[r, h, j + D // 2])
                w = z * cmath.exp(1j * pos[r] * theta ** (-2.0 * j / D))
                assert abs(got[r, h, j] - w.real) < 1e-12
                assert abs(got[r, h, j + D // 2] - w.imag) < 1e-12


def test_relative_position_identity():
    rng = np.random.default_rng(2)
    D, theta = 16, 1.0e4
    q = rng.standard_normal((1, 1, D))
    k = rng.standard_normal((1, 1, D))
    for a, b in [(5, 2), (100, 99), (40000, 3)]:
        lhs = float(np.sum(rope.rotate(q, [a], theta) * rope.rotate(k, [b], theta)))
        rhs = float(np.sum(rope.rotate(q, [a - b], theta) * k))
        assert abs(lhs - rhs) < 1e-9


def test_gather_by_value_not_index():
    # The rotation of a row depends on its position value only: permuting rows and
    # positions together commutes, positions may repeat, skip or exceed the length.
    rng = np.random.default_rng(3)
    x = rng.standard_normal((6, 1, 8))
    pos = np.array([9, 2, 2, 40, 0, 5])
    full = rope.rotate(x, pos, 1.0e4)
    perm = rng.permutation(6)
    assert np.allclose(rope.rotate(x[perm], pos[perm], 1.0e4), full[perm], atol=0, rtol=0)
    # arange positions: row i rotated by angle i (the contiguous-slice case)
    ar = rope.rotate(x, np.arange(6), 1.0e4)
    for i in range(6):
        assert np.array_equal(ar[i], rope.rotate(x[i:i + 1], [i], 1.0e4)[0])
    # pair norms are preserved
    n0 = x[..., :4] ** 2 + x[..., 4:] ** 2
    n1 = full[..., :4] ** 2 + full[..., 4:] ** 2
    assert np.allclose(n0, n1, rtol=1e-13)


def test_row_positions_restart_per_sequence():
    # two sequences [0,3) and [3,7); depth 0 keeps all, depth 1 keeps anchors 1 and 4
    idx = [0, 1, 2, 3, 4, 5, 6, 1, 4]
    depth_off = [0, 7, 9]
    cu = [0, 3, 7]
    # depth 0: p - a_s ; depth 1: anchor 1 -> 1 + 1, anchor 4 -> (4 - 3) + 1
    assert rope.row_positions(idx, depth_off, cu).tolist() == [0, 1, 2, 0, 1, 2, 3, 2, 2]
