"""Pins of the oracle's DiG block (slides Figure 4; write-up section 3 "DiG Block"): the
adaptive RMSNorm against torch's rms_norm, GELU and SiLU against closed forms, a textbook value
and torch, the conditioning regression's special cases, and the whole block against an
independent torch composition (parallel form of the GLA, torch convolution), its alpha = 0
reduction to the SREM conv, its affinity in alpha_1, and the fused reorient of its output."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads as wl


def test_rmsnorm_modulate_against_torch_and_groups():
    rng = np.random.default_rng(11)
    B, L, D = 3, 5, 24
    x = rng.standard_normal((B, L, D))
    scale = rng.standard_normal((B, D))
    shift = rng.standard_normal((B, D))
    got = oracle.rmsnorm_modulate(x, scale, shift, eps=1e-5)
    n = F.rms_norm(torch.from_numpy(x), (D,), eps=1e-5).numpy()
    want = n * scale[:, None, :] + shift[:, None, :]    # image b uses its own rows
    assert np.max(np.abs(got - want)) <= 1e-12


def test_rmsnorm_modulate_special_rows():
    D = 16
    scale = np.linspace(-1.0, 2.0, D)[None]
    shift = np.linspace(0.5, -0.5, D)[None]
    for c in (3.0, -0.25):                              # constant row: RMSNorm gives sign(c)
        got = oracle.rmsnorm_modulate(np.full((1, 1, D), c), scale, shift, eps=0.0)[0, 0]
        assert np.max(np.abs(got - (math.copysign(1.0, c) * scale[0] + shift[0]))) <= 1e-15
    got = oracle.rmsnorm_modulate(np.zeros((1, 2, D)), scale, shift, eps=1e-5)
    assert np.array_equal(got[0], np.broadcast_to(shift[0], (2, D)))   # zero row: the shift


def test_gelu_closed_forms_and_torch():
    assert oracle.gelu(np.array([0.0]))[0] == 0.0
    # Phi(1) = 0.8413447460685429 (standard normal table): GELU(1) = Phi(1)
    assert abs(oracle.gelu(np.array([1.0]))[0] - 0.8413447460685429) <= 1e-15
    x = np.linspace(-6.0, 6.0, 241)
    g = oracle.gelu(x)
    # x Phi(x) - (-x) Phi(-x) = x (Phi(x) + Phi(-x)) = x
    assert np.max(np.abs(g - oracle.gelu(-x) - x)) <= 1e-14
    want = F.gelu(torch.from_numpy(x), approximate="none").numpy()
    assert np.max(np.abs(g - want)) <= 1e-14
    assert abs(oracle.gelu(np.array([40.0]))[0] - 40.0) <= 1e-12


def test_silu_closed_forms_and_torch():
    x = np.linspace(-8.0, 8.0, 161)
    s = oracle.silu(x)
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    assert np.max(np.abs(s - oracle.silu(-x) - x)) <= 1e-14     # x sigma(x) + x sigma(x) - x
    assert np.max(np.abs(s - F.silu(torch.from_numpy(x)).numpy())) <= 1e-14


def test_block_cond():
    rng = np.random.default_rng(12)
    c = rng.standard_normal((2, 8))
    b = rng.standard_normal(48)
    assert np.array_equal(oracle.block_cond(c, np.zeros((48, 8)), b), np.broadcast_to(b, (2, 48)))
    w = rng.standard_normal((48, 8))
    want = F.linear(F.silu(torch.from_numpy(c)), torch.from_numpy(w), torch.from_numpy(b)).numpy()
    assert np.max(np.abs(oracle.block_cond(c, w, b) - want)) <= 1e-12


# ------------------------------------------------------------------- whole block
SMALL = wl.Config("block_tiny", 2, 4, 5, 16, 2, 4, 8, 16, "bf16", rank=8)


def _small_case(seed=13):
    rng = np.random.default_rng(seed)
    wts = wl.make_dig_block_weights(SMALL, rng)
    x = rng.standard_normal((SMALL.batch, SMALL.seq_len, SMALL.d_model))
    mod = rng.standard_normal((SMALL.batch, 6 * SMALL.d_model)) * 0.5
    mod[:, 0:16] += 1.0
    mod[:, 48:64] += 1.0
    return x, mod, wts


def _fwd(x, mod, wts, layout=wl.ROW, out_layout=wl.ROW):
    c = SMALL
    return oracle.block_forward(x, mod, wts, c.grid_h, c.grid_w, c.heads, c.d_k, c.d_v,
                                layout, out_layout, tau=c.tau)


def _torch_block_row(x, mod, wts):
    """The same block in torch, row scan order, with the GLA in its parallel form
    o_t = sum_{s <= t} sum_c q_tc k_sc exp(B_tc - B_sc) v_s, B = cumsum(logsigmoid(z) / tau)."""
    c = SMALL
    t = {k: torch.from_numpy(np.asarray(v, dtype=np.float64)) for k, v in wts.items()}
    x, mod = torch.from_numpy(x), torch.from_numpy(mod)
    B, L, D = x.shape
    H, dk, dv = c.heads, c.d_k, c.d_v
    g1, b1, a1, g2, b2, a2 = (mod[:, None, i * D:(i + 1) * D] for i in range(6))
    h = F.rms_norm(x, (D,), eps=1e-5) * g1 + b1
    proj = F.linear(h, t["w_in"], t["b_in"])
    q, k, v, u, r = torch.split(proj, [H * dk, H * dk, H * dv, c.rank, H * dv], dim=-1)
    z = F.linear(u, t["w_gate"], t["b_gate"])
    hd = lambda a, d: a.reshape(B, L, H, d).permute(0, 2, 1, 3)      # [B, H, L, d]
    q, k, v, z, r = hd(q, dk), hd(k, dk), hd(v, dv), hd(z, dk), hd(r, dv)
    cum = torch.cumsum(F.logsigmoid(z) / c.tau, dim=2)
    dec = cum[:, :, :, None, :] - cum[:, :, None, :, :]                # [B, H, t, s, c]
    mask = torch.tril(torch.ones(L, L, dtype=torch.bool))[None, None, :, :, None]
    wgt = torch.where(mask, torch.exp(torch.where(mask, dec, torch.zeros_like(dec))),
                      torch.zeros_like(dec))
    a = torch.einsum("bhtc,bhsc,bhtsc->bhts", q, k, wgt)
    o = a @ v
    y = F.rms_norm(o, (dv,), weight=t["gla_norm_w"], eps=1e-5) * F.silu(r)
    y = y.permute(0, 2, 1, 3).reshape(B, L, H * dv)
    x1 = x + a1 * F.linear(y, t["w_out"], t["b_out"])
    h2 = F.rms_norm(x1, (D,), eps=1e-5) * g2 + b2
    x2 = x1 + a2 * F.linear(F.gelu(F.linear(h2, t["w_ffn1"], t["b_ffn1"])), t["w_ffn2"],
                            t["b_ffn2"])
    img = x2.reshape(B, c.grid_h, c.grid_w, D).permute(0, 3, 1, 2)
    out = F.conv2d(img, t["conv_w"][:, None], t["conv_b"], padding=1, groups=D)
    return out.permute(0, 2, 3, 1).reshape(B, L, D).numpy()


def test_block_against_torch_composition():
    x, mod, wts = _small_case()
    got = _fwd(x, mod, wts)
    want = _torch_block_row(x, mod, wts)
    assert np.max(np.abs(got - want)) <= 1e-10 * np.max(np.abs(want))


def test_block_zero_alpha_is_the_conv():
    x, mod, wts = _small_case(14)
    mod[:, 32:48] = 0.0
    mod[:, 80:96] = 0.0
    for layout, out_layout in [(wl.ROW, wl.ROW_REV), (wl.COL, wl.COL_REV), (wl.COL_REV, wl.ROW)]:
        got = _fwd(x, mod, wts, layout, out_layout)
        want = oracle.dwconv3x3(x, wts["conv_w"], SMALL.grid_h, SMALL.grid_w, layout, out_layout,
                                wts["conv_b"])
        assert np.array_equal(got, want)


def test_block_affine_in_alpha1():
    x, mod, wts = _small_case(15)
    mod[:, 80:96] = 0.0                                   # alpha_2 = 0: no feedforward branch
    outs = []
    for s in (0.0, 1.0, 2.0):
        m = mod.copy()
        m[:, 32:48] *= s
        outs.append(_fwd(x, m, wts, wl.COL, wl.COL_REV))
    assert np.max(np.abs((outs[2] - outs[1]) - (outs[1] - outs[0]))) <= 1e-12
    assert np.max(np.abs(outs[1] - outs[0])) > 1e-3      # the GLA branch contributes


@pytest.mark.parametrize("layout,out_layout", [(wl.ROW_REV, wl.COL), (wl.COL, wl.COL_REV)])
def test_block_fused_reorient(layout, out_layout):
    x, mod, wts = _small_case(16)
    plain = _fwd(x, mod, wts, layout, layout)
    fused = _fwd(x, mod, wts, layout, out_layout)
    assert np.array_equal(fused, oracle.reorient(plain, SMALL.grid_h, SMALL.grid_w, layout,
                                                 out_layout))
