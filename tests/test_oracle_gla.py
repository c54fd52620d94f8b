"""Pins for the fp64 oracle's GLA mixer (forward and backward), independent of the oracle.

Each test checks the oracle against something it does not share code with: brute-force
causal linear attention, the closed parallel form, a hand-worked example, torch's own
logsigmoid / rms_norm / silu, torch autograd through the parallel form, and central finite
differences.  Recurrence and gate follow the DiG study-group slides, eqs. (5)-(10).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _parallel_form(q, k, v, loga):
    """o_t = sum_{s<=t} sum_c q_tc k_sc exp(B_tc - B_sc) v_s with B = cumsum(log alpha)."""
    B_, L, H, dk = q.shape
    Bc = np.cumsum(loga, axis=1)
    o = np.zeros(q.shape[:3] + (v.shape[-1],))
    for t in range(L):
        # weights [B, s<=t, H] = sum_c q_t k_s exp(B_t - B_s)
        dec = np.exp(Bc[:, t:t + 1] - Bc[:, :t + 1])            # [B, t+1, H, dk]
        w = np.sum(q[:, t:t + 1] * k[:, :t + 1] * dec, axis=-1)  # [B, t+1, H]
        o[:, t] = np.einsum("bsh,bshe->bhe", w, v[:, :t + 1])
    return o


def test_hand_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "gla_hand_example.json")))
    for key in ("vector_case", "scalar_case"):
        c = g[key]
        L = len(c["q"])
        q = np.array(c["q"], dtype=float).reshape(1, L, 1, -1)
        k = np.array(c["k"], dtype=float).reshape(1, L, 1, -1)
        v = np.array(c["v"], dtype=float).reshape(1, L, 1, -1)
        loga = np.log(np.array(c["alpha"], dtype=float)).reshape(1, L, 1, -1)
        o = oracle.gla_recurrence(q, k, v, loga)
        np.testing.assert_allclose(o.reshape(L, -1), np.array(c["o"]).reshape(L, -1), rtol=0, atol=1e-14)


def test_alpha_one_is_causal_linear_attention():
    rng = np.random.default_rng(1)
    q, k = _rand(rng, 2, 37, 3, 5), _rand(rng, 2, 37, 3, 5)
    v = _rand(rng, 2, 37, 3, 7)
    o = oracle.gla_recurrence(q, k, v, np.zeros_like(q))
    for b in range(2):
        for h in range(3):
            A = np.tril(q[b, :, h] @ k[b, :, h].T)
            np.testing.assert_allclose(o[b, :, h], A @ v[b, :, h], rtol=1e-12, atol=1e-12)


def test_alpha_zero_keeps_only_current_token():
    rng = np.random.default_rng(2)
    q, k = _rand(rng, 1, 20, 2, 4), _rand(rng, 1, 20, 2, 4)
    v = _rand(rng, 1, 20, 2, 6)
    o = oracle.gla_recurrence(q, k, v, np.full(q.shape, -np.inf))
    ref = np.sum(q * k, axis=-1, keepdims=True) * v
    np.testing.assert_allclose(o, ref, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("scale", [0.05, 1.0, 4.0])
def test_recurrence_equals_parallel_form(scale):
    rng = np.random.default_rng(3)
    q, k = _rand(rng, 2, 48, 2, 6), _rand(rng, 2, 48, 2, 6)
    v = _rand(rng, 2, 48, 2, 5)
    loga = -np.abs(_rand(rng, 2, 48, 2, 6)) * scale
    o = oracle.gla_recurrence(q, k, v, loga)
    np.testing.assert_allclose(o, _parallel_form(q, k, v, loga), rtol=1e-11, atol=1e-12)


def test_q_scale_and_linearity():
    rng = np.random.default_rng(4)
    q, k = _rand(rng, 1, 30, 2, 4), _rand(rng, 1, 30, 2, 4)
    v1, v2 = _rand(rng, 1, 30, 2, 3), _rand(rng, 1, 30, 2, 3)
    loga = -np.abs(_rand(rng, 1, 30, 2, 4)) * 0.3
    o1 = oracle.gla_recurrence(q, k, v1, loga)
    o2 = oracle.gla_recurrence(q, k, v2, loga)
    o12 = oracle.gla_recurrence(q, k, v1 + 2.0 * v2, loga)
    np.testing.assert_allclose(o12, o1 + 2.0 * o2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(oracle.gla_recurrence(q, k, v1, loga, q_scale=0.25),
                               0.25 * o1, rtol=1e-13, atol=1e-14)


def test_gate_matches_torch_logsigmoid():
    z = np.concatenate([np.linspace(-60, 60, 2001), [0.0, 1e-8, -1e-8, 700.0, -700.0]])
    ref = torch.nn.functional.logsigmoid(torch.from_numpy(z)).numpy()
    got = oracle.gate_logalpha(z, 16.0)
    np.testing.assert_allclose(got, ref / 16.0, rtol=1e-14, atol=1e-300)
    assert oracle.logsigmoid(0.0) == pytest.approx(-math.log(2.0), rel=1e-15)
    # alpha = sigmoid(z)^(1/tau) lies in (0, 1): exp of a negative number
    assert np.all(got < 0)


def test_output_stage_closed_forms():
    eps = 1e-5
    # constant pre-norm vector c*1: RMSNorm gives c / sqrt(c^2 + eps) in every entry
    for c in (-3.0, 0.5, 2.0):
        o = np.full((1, 1, 1, 8), c)
        r = np.linspace(-2, 2, 8).reshape(1, 1, 1, 8)
        y, rstd = oracle.output_stage(o, r, None, eps)
        sw = r / (1 + np.exp(-r))
        np.testing.assert_allclose(y, c / math.sqrt(c * c + eps) * sw, rtol=1e-14, atol=1e-15)
        assert rstd[0, 0, 0] == pytest.approx(1 / math.sqrt(c * c + eps), rel=1e-14)
    # Swish(0) = 0
    y, _ = oracle.output_stage(np.ones((1, 2, 1, 4)), np.zeros((1, 2, 1, 4)))
    assert np.all(y == 0.0)


def test_output_stage_matches_torch():
    rng = np.random.default_rng(5)
    o, r = _rand(rng, 2, 9, 3, 12), _rand(rng, 2, 9, 3, 12)
    g = 1 + 0.3 * _rand(rng, 12)
    y, _ = oracle.output_stage(o, r, g, 1e-5)
    t = torch.from_numpy
    ref = torch.nn.functional.rms_norm(t(o), (12,), t(g), eps=1e-5) * torch.nn.functional.silu(t(r))
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-12, atol=1e-13)


# ------------------------------------------------------------------ backward pins
def _torch_layer(q, k, v, z, r, gamma, tau, eps):
    """Whole layer through the parallel form, in torch fp64 (autograd-able)."""
    loga = torch.nn.functional.logsigmoid(z) / tau
    Bc = torch.cumsum(loga, dim=1)
    L = q.shape[1]
    outs = []
    for t in range(L):
        dec = torch.exp(Bc[:, t:t + 1] - Bc[:, :t + 1])
        w = torch.sum(q[:, t:t + 1] * k[:, :t + 1] * dec, dim=-1)
        outs.append(torch.einsum("bsh,bshe->bhe", w, v[:, :t + 1]))
    o = torch.stack(outs, dim=1)
    n = o * torch.rsqrt(torch.mean(o * o, dim=-1, keepdim=True) + eps)
    return n * gamma * torch.nn.functional.silu(r)


@pytest.mark.parametrize("gate_shift", [0.0, -4.0, 3.0])
def test_backward_matches_autograd_of_parallel_form(gate_shift):
    rng = np.random.default_rng(6)
    B, L, H, dk, dv = 2, 24, 2, 5, 6
    q, k, z = (_rand(rng, B, L, H, dk) for _ in range(3))
    z = 2.0 * z + gate_shift
    v, r, dy = (_rand(rng, B, L, H, dv) for _ in range(3))
    gamma = 1 + 0.3 * _rand(rng, dv)
    got = oracle.gla_bwd(q, k, v, z, r, dy, gamma, tau=16.0)
    ts = [torch.tensor(a, requires_grad=True) for a in (q, k, v, z, r, gamma)]
    y = _torch_layer(*ts, 16.0, 1e-5)
    (y * torch.from_numpy(dy)).sum().backward()
    for name, t in zip(("dq", "dk", "dv", "dz", "dr", "dgamma"), ts):
        np.testing.assert_allclose(got[name], t.grad.numpy(), rtol=1e-9, atol=1e-11, err_msg=name)
    yf, _, _ = oracle.gla_fwd(q, k, v, z, r, gamma)
    np.testing.assert_allclose(yf, y.detach().numpy(), rtol=1e-11, atol=1e-12)


def test_backward_central_differences():
    rng = np.random.default_rng(7)
    B, L, H, dk, dv = 1, 16, 2, 4, 5
    q, k, z = (_rand(rng, B, L, H, dk) for _ in range(3))
    v, r, dy = (_rand(rng, B, L, H, dv) for _ in range(3))
    gamma = 1 + 0.3 * _rand(rng, dv)
    g = oracle.gla_bwd(q, k, v, z, r, dy, gamma)
    args = dict(q=q, k=k, v=v, z=z, r=r)

    def loss(**kw):
        a = dict(args)
        a.update(kw)
        gm = kw.get("gamma", gamma)
        y, _, _ = oracle.gla_fwd(a["q"], a["k"], a["v"], a["z"], a["r"], gm)
        return float(np.sum(y * dy))

    h = 1e-6
    for name in ("q", "k", "v", "z", "r", "gamma"):
        base = gamma if name == "gamma" else args[name]
        u = rng.standard_normal(base.shape)
        fd = (loss(**{name: base + h * u}) - loss(**{name: base - h * u})) / (2 * h)
        an = float(np.sum(g["d" + name] * u))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


def test_dloga_two_formulas_agree():
    """d log(alpha_u) = sum_{t >= u} (q_t dq_t - k_t dk_t): reverse cumsum over the sequence."""
    rng = np.random.default_rng(8)
    B, L, H, dk, dv = 1, 40, 2, 4, 6
    q, k = _rand(rng, B, L, H, dk), _rand(rng, B, L, H, dk)
    v, r, dy = (_rand(rng, B, L, H, dv) for _ in range(3))
    loga = -np.abs(_rand(rng, B, L, H, dk)) * 0.2
    g = oracle.gla_bwd_logalpha(q, k, v, loga, r, dy)
    contrib = q * g["dq"] - k * g["dk"]
    rc = np.flip(np.cumsum(np.flip(contrib, axis=1), axis=1), axis=1)
    # at u = 0 the sum is the derivative of a common shift of every B_t: zero
    np.testing.assert_allclose(g["dloga"], rc, rtol=1e-10, atol=1e-11)
