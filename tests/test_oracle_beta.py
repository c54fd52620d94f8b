"""Pins for the oracle's mixer with the outer-product gate G_t = alpha_t^T beta_t
(DiG study-group slides, slide "GLA の導入", eq. (5): a key-side gate alpha and a value-side
gate beta, both sigmoid(logit)^(1/tau)).

The oracle runs the token-by-token recurrence; these tests hold it against what it shares no
code with: the closed parallel form written in torch fp64 (forward, and autograd through it for
every gradient), central finite differences, the beta = 1 limit (the key-gate-only mixer, pinned
on its own), and a brute-force scalar case with alpha = 1.
"""
import numpy as np
import pytest
import torch

import oracle


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _torch_layer_beta(q, k, v, z, w, r, gamma, tau, eps):
    """Whole layer in the parallel form:
    o_t[e] = sum_{s<=t} sum_c q_t[c] k_s[c] v_s[e] exp(B_t[c] - B_s[c] + C_t[e] - C_s[e]),
    B, C the running sums of log alpha = logsigmoid(z)/tau and log beta = logsigmoid(w)/tau."""
    Bc = torch.cumsum(torch.nn.functional.logsigmoid(z) / tau, dim=1)   # [B, L, H, dk]
    Cc = torch.cumsum(torch.nn.functional.logsigmoid(w) / tau, dim=1)   # [B, L, H, dv]
    L = q.shape[1]
    outs = []
    for t in range(L):
        dk_ = torch.exp(Bc[:, t:t + 1] - Bc[:, :t + 1])                  # [B, s, H, dk]
        dv_ = torch.exp(Cc[:, t:t + 1] - Cc[:, :t + 1])                  # [B, s, H, dv]
        a = q[:, t:t + 1] * k[:, :t + 1] * dk_                          # [B, s, H, dk]
        b = v[:, :t + 1] * dv_                                          # [B, s, H, dv]
        outs.append(torch.einsum("bshc,bshe->bhe", a, b))
    o = torch.stack(outs, dim=1)
    n = o * torch.rsqrt(torch.mean(o * o, dim=-1, keepdim=True) + eps)
    return n * gamma * torch.nn.functional.silu(r), o


@pytest.mark.parametrize("zs,ws", [(0.0, 0.0), (-4.0, 2.0), (3.0, -5.0)])
def test_beta_matches_autograd_of_parallel_form(zs, ws):
    rng = np.random.default_rng(21)
    B, L, H, dk, dv = 2, 20, 2, 4, 5
    q, k, z = (_rand(rng, B, L, H, dk) for _ in range(3))
    v, w, r, dy = (_rand(rng, B, L, H, dv) for _ in range(4))
    z, w = 2.0 * z + zs, 2.0 * w + ws
    gamma = 1 + 0.3 * _rand(rng, dv)
    tau, eps = 16.0, 1e-5
    got = oracle.gla_bwd_beta(q, k, v, z, w, r, dy, gamma, tau=tau, eps=eps)
    ts = [torch.tensor(a, requires_grad=True) for a in (q, k, v, z, w, r, gamma)]
    y, o = _torch_layer_beta(*ts, tau, eps)
    (y * torch.from_numpy(dy)).sum().backward()
    for name, t in zip(("dq", "dk", "dv", "dz", "dw", "dr", "dgamma"), ts):
        np.testing.assert_allclose(got[name], t.grad.numpy(), rtol=1e-9, atol=1e-11, err_msg=name)
    yf, of, _ = oracle.gla_fwd_beta(q, k, v, z, w, r, gamma, tau=tau, eps=eps)
    np.testing.assert_allclose(yf, y.detach().numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(of, o.detach().numpy(), rtol=1e-11, atol=1e-12)


def test_beta_with_q_scale_and_tau():
    rng = np.random.default_rng(22)
    B, L, H, dk, dv = 1, 12, 2, 3, 4
    q, k, z = (_rand(rng, B, L, H, dk) for _ in range(3))
    v, w, r, dy = (_rand(rng, B, L, H, dv) for _ in range(4))
    got = oracle.gla_bwd_beta(q, k, v, z, w, r, dy, None, tau=2.0, q_scale=0.5)
    ts = [torch.tensor(a, requires_grad=True) for a in (q, k, v, z, w, r)]
    y, _ = _torch_layer_beta(ts[0] * 0.5, *ts[1:], torch.ones(dv, dtype=torch.float64), 2.0, 1e-5)
    (y * torch.from_numpy(dy)).sum().backward()
    for name, t in zip(("dq", "dk", "dv", "dz", "dw", "dr"), ts):
        np.testing.assert_allclose(got[name], t.grad.numpy(), rtol=1e-9, atol=1e-11, err_msg=name)


def test_beta_one_is_the_key_gate_mixer():
    # w -> +inf: logsigmoid(w) is exactly 0 in fp64, beta = 1, and dw = 0
    rng = np.random.default_rng(23)
    B, L, H, dk, dv = 2, 33, 3, 5, 7
    q, k, z = (_rand(rng, B, L, H, dk) for _ in range(3))
    v, r, dy = (_rand(rng, B, L, H, dv) for _ in range(3))
    w = np.full((B, L, H, dv), 1000.0)
    gamma = 1 + 0.2 * _rand(rng, dv)
    y1, o1, s1 = oracle.gla_fwd_beta(q, k, v, z, w, r, gamma)
    y0, o0, s0 = oracle.gla_fwd(q, k, v, z, r, gamma)
    np.testing.assert_allclose(y1, y0, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(o1, o0, rtol=1e-13, atol=1e-14)
    g1 = oracle.gla_bwd_beta(q, k, v, z, w, r, dy, gamma)
    g0 = oracle.gla_bwd(q, k, v, z, r, dy, gamma)
    for n in ("dq", "dk", "dv", "dz", "dr", "dgamma"):
        np.testing.assert_allclose(g1[n], g0[n], rtol=1e-12, atol=1e-13, err_msg=n)
    assert np.all(g1["dw"] == 0.0)


def test_alpha_one_scalar_key_is_a_decayed_running_sum():
    # d_k = 1, q = k = 1, alpha = 1: o_t[e] = sum_{s<=t} v_s[e] prod_{s<u<=t} beta_u[e]
    rng = np.random.default_rng(24)
    L, dv, tau = 15, 4, 3.0
    v = _rand(rng, 1, L, 1, dv)
    w = 1.5 * _rand(rng, 1, L, 1, dv)
    beta = (1.0 / (1.0 + np.exp(-w))) ** (1.0 / tau)
    ones = np.ones((1, L, 1, 1))
    _, o, _ = oracle.gla_fwd_beta(ones, ones, v, np.full((1, L, 1, 1), 1000.0), w,
                                  np.ones((1, L, 1, dv)), tau=tau)
    ref = np.zeros((L, dv))
    for t in range(L):
        for s in range(t + 1):
            f = np.ones(dv)
            for u in range(s + 1, t + 1):
                f = f * beta[0, u, 0]
            ref[t] += v[0, s, 0] * f
    np.testing.assert_allclose(o[0, :, 0], ref, rtol=1e-12, atol=1e-13)


def test_beta_backward_central_differences():
    rng = np.random.default_rng(25)
    B, L, H, dk, dv = 1, 14, 2, 3, 4
    q, k, z = (_rand(rng, B, L, H, dk) for _ in range(3))
    v, w, r, dy = (_rand(rng, B, L, H, dv) for _ in range(4))
    gamma = 1 + 0.3 * _rand(rng, dv)
    g = oracle.gla_bwd_beta(q, k, v, z, w, r, dy, gamma)
    args = dict(q=q, k=k, v=v, z=z, w=w, r=r)

    def loss(**kw):
        a = dict(args)
        a.update(kw)
        gm = kw.get("gamma", gamma)
        y, _, _ = oracle.gla_fwd_beta(a["q"], a["k"], a["v"], a["z"], a["w"], a["r"], gm)
        return float(np.sum(y * dy))

    h = 1e-6
    for name in ("q", "k", "v", "z", "w", "r", "gamma"):
        base = gamma if name == "gamma" else args[name]
        u = rng.standard_normal(base.shape)
        fd = (loss(**{name: base + h * u}) - loss(**{name: base - h * u})) / (2 * h)
        an = float(np.sum(g["d" + name] * u))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)
