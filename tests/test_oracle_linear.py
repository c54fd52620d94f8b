"""Pins of the oracle's linear projection (the projections around the mixer, slides eqs. (5),
(9), (10)): a hand-worked product, numpy's matmul (an independent implementation), the
identity weight, bias only, and linearity."""
import numpy as np

import oracle


def test_hand_example():
    a = np.array([[1.0, 2.0], [3.0, 4.0]])
    w = np.array([[5.0, 6.0], [7.0, 8.0], [9.0, 10.0]])   # 3 outputs x 2 inputs
    # c[i][j] = sum_l a[i][l] w[j][l], worked by hand: 1*5 + 2*6 = 17, 1*7 + 2*8 = 23, ...
    want = np.array([[17.0, 23.0, 29.0], [39.0, 53.0, 67.0]])
    assert np.array_equal(oracle.linear(a, w), want)
    assert np.array_equal(oracle.linear(a, w, np.array([1.0, -1.0, 0.5])),
                          want + np.array([1.0, -1.0, 0.5]))


def test_against_numpy_matmul():
    rng = np.random.default_rng(5)
    for m, k, n in [(1, 1, 1), (7, 13, 5), (64, 96, 40), (3, 384, 3472 // 8)]:
        a = rng.standard_normal((m, k))
        w = rng.standard_normal((n, k))
        b = rng.standard_normal(n)
        got = oracle.linear(a, w, b)
        want = np.matmul(a, w.T) + b
        assert np.max(np.abs(got - want)) <= 1e-12 * max(1.0, np.max(np.abs(want))) * k


def test_identity_bias_and_linearity():
    rng = np.random.default_rng(6)
    a = rng.standard_normal((5, 4, 24))          # leading dims flatten to rows
    assert np.array_equal(oracle.linear(a, np.eye(24)), a)
    b = rng.standard_normal(7)
    assert np.array_equal(oracle.linear(np.zeros((3, 24)), rng.standard_normal((7, 24)), b),
                          np.broadcast_to(b, (3, 7)))
    w = rng.standard_normal((9, 24))
    a2 = rng.standard_normal(a.shape)
    lhs = oracle.linear(a + 2.0 * a2, w)
    rhs = oracle.linear(a, w) + 2.0 * oracle.linear(a2, w)
    assert np.max(np.abs(lhs - rhs)) <= 1e-12
