"""Pins of the oracle's low-rank key gate (slides eq. (5): the logits are (x W_a1) W_a2 +
b_alpha, here lowrank_gate_logits), independent of the formula it evaluates:

* selection weights: a W_a2 whose row (h, c) is a unit vector e_j reproduces factor column j
  plus the bias, so a transposed W, a swapped head/key order in the reshape or a dropped bias
  fails;
* linearity in the factor and in W, against separate evaluations;
* a tiny case (one head, rank 2) written out by hand, and a head whose W row block is zero
  with bias b has the constant gate logsigmoid(b) / tau in every position.
"""
import numpy as np

import oracle


def test_selection_weights_pick_factor_columns():
    rng = np.random.default_rng(5)
    B, L, H, dk, R = 2, 7, 3, 5, 16
    f = rng.standard_normal((B, L, R))
    bias = rng.standard_normal(H * dk)
    w = np.zeros((H * dk, R))
    pick = {}
    for h in range(H):
        for c in range(dk):
            j = (h + 3 * c) % R
            w[h * dk + c, j] = 1.0
            pick[h, c] = j
    z = oracle.lowrank_gate_logits(f, w, bias, H, dk)
    assert z.shape == (B, L, H, dk)
    for h in range(H):
        for c in range(dk):
            np.testing.assert_array_equal(z[:, :, h, c], f[:, :, pick[h, c]] + bias[h * dk + c])


def test_linear_in_factor_and_weight():
    rng = np.random.default_rng(6)
    B, L, H, dk, R = 1, 9, 2, 4, 16
    f1, f2 = rng.standard_normal((2, B, L, R))
    w1, w2 = rng.standard_normal((2, H * dk, R))
    z = lambda f, w, b=None: oracle.lowrank_gate_logits(f, w, b, H, dk)
    np.testing.assert_allclose(z(f1 + 2 * f2, w1), z(f1, w1) + 2 * z(f2, w1), rtol=0, atol=1e-12)
    np.testing.assert_allclose(z(f1, w1 - w2), z(f1, w1) - z(f1, w2), rtol=0, atol=1e-12)
    np.testing.assert_array_equal(z(f1, 0 * w1, np.full(H * dk, 0.5)), np.full((B, L, H, dk), 0.5))


def test_tiny_case_written_out():
    # one head, d_k = 2, rank 2: z[t, c] = b[c] + f[t,0] w[c,0] + f[t,1] w[c,1]
    f = np.array([[[1.0, 2.0], [-1.0, 0.5], [0.0, 3.0]]])
    w = np.array([[0.5, -1.0], [2.0, 0.25]])
    b = np.array([0.1, -0.2])
    want = np.array([[[0.1 + 0.5 - 2.0, -0.2 + 2.0 + 0.5],
                      [0.1 - 0.5 - 0.5, -0.2 - 2.0 + 0.125],
                      [0.1 + 0.0 - 3.0, -0.2 + 0.0 + 0.75]]])[:, :, None, :]
    np.testing.assert_allclose(oracle.lowrank_gate_logits(f, w, b, 1, 2), want, rtol=0, atol=1e-15)


def test_zero_weight_head_has_constant_gate():
    rng = np.random.default_rng(7)
    B, L, H, dk, R, tau = 1, 12, 2, 3, 16, 16.0
    f = rng.standard_normal((B, L, R))
    w = rng.standard_normal((H * dk, R))
    w[dk:] = 0.0                       # head 1: logits are the bias alone
    bias = np.concatenate([np.zeros(dk), [-2.0, 0.5, 3.0]])
    z = oracle.lowrank_gate_logits(f, w, bias, H, dk)
    la = oracle.gate_logalpha(z, tau)
    for c, bc in enumerate([-2.0, 0.5, 3.0]):
        np.testing.assert_allclose(la[:, :, 1, c], oracle.logsigmoid(bc) / tau, rtol=1e-15)
