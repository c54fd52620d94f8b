"""Pins for the fp64 oracle's SREM step: scan permutations, reorient, 3x3 depthwise conv.

The SREM (DiG study-group slides, slide "SREM の導入"; DiG write-up, section 3 "DiG Block")
reshapes the sequence to 2-D, applies a 3x3 depthwise conv and transposes / flips the token
matrix to set the next block's scan direction.  The oracle is checked against explicit
numpy transposes and flips, torch's grouped conv2d, autograd and adjoint identities.
"""
import itertools

import numpy as np
import pytest
import torch

import oracle
from oracle import COL, COL_REV, ROW, ROW_REV

DIRS = (ROW, ROW_REV, COL, COL_REV)
GRIDS = [(1, 1), (1, 5), (4, 1), (3, 5), (8, 8), (7, 4)]


def _explicit_order(d, gh, gw):
    """Canonical ids in scan order d, from numpy transposes / flips of the id grid."""
    ids = np.arange(gh * gw).reshape(gh, gw)
    if d == ROW:
        return ids.reshape(-1)
    if d == ROW_REV:
        return ids.reshape(-1)[::-1]
    if d == COL:
        return ids.T.reshape(-1)
    return ids.T.reshape(-1)[::-1]


@pytest.mark.parametrize("gh,gw", GRIDS)
def test_permutations_are_the_four_scans(gh, gw):
    L = gh * gw
    for d in DIRS:
        perm, inv = oracle.scan_perm(d, gh, gw)
        assert sorted(perm.tolist()) == list(range(L))          # bijection
        np.testing.assert_array_equal(perm, _explicit_order(d, gh, gw))
        np.testing.assert_array_equal(inv[perm], np.arange(L))   # inverse


@pytest.mark.parametrize("gh,gw", GRIDS)
def test_reorient_round_trip_and_payload(gh, gw):
    L = gh * gw
    rng = np.random.default_rng(0)
    # integer payload: each row carries its canonical id, plus random bytes
    for frm, to in itertools.product(DIRS, DIRS):
        canon = _explicit_order(frm, gh, gw)
        x = np.concatenate([np.broadcast_to(canon[None, :, None], (2, L, 1)),
                            rng.integers(0, 2**31, size=(2, L, 3))], axis=2).astype(np.int64)
        y = oracle.reorient(x, gh, gw, frm, to)
        np.testing.assert_array_equal(y[:, :, 0], np.broadcast_to(_explicit_order(to, gh, gw), (2, L)))
        back = oracle.reorient(y, gh, gw, to, frm)
        np.testing.assert_array_equal(back, x)


def test_schedule_has_period_four():
    gh, gw = 5, 3
    x = np.arange(2 * 15 * 2, dtype=np.int32).reshape(2, 15, 2)
    cur = x
    seq = (ROW, ROW_REV, COL, COL_REV, ROW)
    for a, b in zip(seq[:-1], seq[1:]):
        cur = oracle.reorient(cur, gh, gw, a, b)
    np.testing.assert_array_equal(cur, x)


def test_reorient_bf16_bytes_exact():
    rng = np.random.default_rng(1)
    x = rng.integers(0, 2**16, size=(3, 12, 7), dtype=np.uint16)
    y = oracle.reorient(x, 3, 4, ROW, COL_REV)
    perm_from = _explicit_order(ROW, 3, 4)
    perm_to = _explicit_order(COL_REV, 3, 4)
    pos = {c: p for p, c in enumerate(perm_from)}
    np.testing.assert_array_equal(y, x[:, [pos[c] for c in perm_to]])


def _torch_dwconv(xg, w, bias):
    """xg [B, rows, cols, D] -> [B, rows, cols, D] via grouped conv2d (cross-correlation)."""
    t = torch.from_numpy(xg).permute(0, 3, 1, 2)
    out = torch.nn.functional.conv2d(t, torch.from_numpy(w)[:, None], None if bias is None
                                     else torch.from_numpy(bias), padding=1, groups=w.shape[0])
    return out.permute(0, 2, 3, 1).numpy()


@pytest.mark.parametrize("gh,gw", [(1, 1), (3, 5), (8, 8), (6, 2)])
@pytest.mark.parametrize("with_bias", [False, True])
def test_dwconv_matches_torch_on_current_grid(gh, gw, with_bias):
    rng = np.random.default_rng(2)
    B, D, L = 2, 5, gh * gw
    w = rng.standard_normal((D, 3, 3)) / 3
    bias = rng.standard_normal(D) if with_bias else None
    for layout, out in itertools.product(DIRS, DIRS):
        x = rng.standard_normal((B, L, D))
        rows, cols = (gw, gh) if layout in (COL, COL_REV) else (gh, gw)
        yc = _torch_dwconv(x.reshape(B, rows, cols, D), w, bias).reshape(B, L, D)
        ref = oracle.reorient(yc, gh, gw, layout, out)
        got = oracle.dwconv3x3(x, w, gh, gw, layout, out, bias)
        np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-13)


def test_dwconv_identity_kernel_is_exact_reorient():
    rng = np.random.default_rng(3)
    w = np.zeros((4, 3, 3))
    w[:, 1, 1] = 1.0
    x = rng.standard_normal((2, 20, 4))
    for layout, out in itertools.product(DIRS, DIRS):
        np.testing.assert_array_equal(oracle.dwconv3x3(x, w, 4, 5, layout, out),
                                      oracle.reorient(x, 4, 5, layout, out))


def test_current_order_conv_is_canonical_conv_with_transformed_kernel():
    """Conv on the current-order grid == canonical-grid conv with K, rot180 K, K^T, rot180 K^T."""
    rng = np.random.default_rng(4)
    gh, gw, D = 5, 7, 3
    w = rng.standard_normal((D, 3, 3))
    x_can = rng.standard_normal((1, gh * gw, D))
    kern = {ROW: w, ROW_REV: w[:, ::-1, ::-1], COL: np.transpose(w, (0, 2, 1)),
            COL_REV: np.transpose(w, (0, 2, 1))[:, ::-1, ::-1]}
    for d in DIRS:
        xd = oracle.reorient(x_can, gh, gw, ROW, d)
        yd = oracle.dwconv3x3(xd, w, gh, gw, d, ROW)          # back in canonical order
        ref = _torch_dwconv(x_can.reshape(1, gh, gw, D), np.ascontiguousarray(kern[d]), None)
        np.testing.assert_allclose(yd, ref.reshape(1, -1, D), rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("layout,out", [(ROW, ROW), (ROW, ROW_REV), (ROW_REV, COL), (COL, COL_REV),
                                        (COL_REV, ROW)])
def test_dwconv_bwd_matches_autograd(layout, out):
    rng = np.random.default_rng(5)
    B, gh, gw, D = 2, 4, 6, 3
    L = gh * gw
    x = rng.standard_normal((B, L, D))
    w = rng.standard_normal((D, 3, 3))
    bias = rng.standard_normal(D)
    dy = rng.standard_normal((B, L, D))
    dx, dw, db = oracle.dwconv3x3_bwd(x, w, dy, gh, gw, layout, out)
    rows, cols = (gw, gh) if layout in (COL, COL_REV) else (gh, gw)
    xt = torch.tensor(x.reshape(B, rows, cols, D), requires_grad=True)
    wt = torch.tensor(w, requires_grad=True)
    bt = torch.tensor(bias, requires_grad=True)
    yc = torch.nn.functional.conv2d(xt.permute(0, 3, 1, 2), wt[:, None], bt, padding=1, groups=D)
    yc = yc.permute(0, 2, 3, 1).reshape(B, L, D)
    perm_to = _explicit_order(out, gh, gw)
    pos_from = np.argsort(_explicit_order(layout, gh, gw))
    y = yc[:, torch.from_numpy(pos_from[perm_to])]
    (y * torch.from_numpy(dy)).sum().backward()
    np.testing.assert_allclose(dx, xt.grad.reshape(B, L, D).numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dw, wt.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(db, bt.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_dwconv_adjoint_identity():
    rng = np.random.default_rng(6)
    B, gh, gw, D = 1, 6, 5, 4
    x = rng.standard_normal((B, gh * gw, D))
    w = rng.standard_normal((D, 3, 3))
    dy = rng.standard_normal((B, gh * gw, D))
    for layout, out in itertools.product(DIRS, DIRS):
        y = oracle.dwconv3x3(x, w, gh, gw, layout, out)
        dx, _, _ = oracle.dwconv3x3_bwd(x, w, dy, gh, gw, layout, out)
        assert np.sum(y * dy) == pytest.approx(np.sum(x * dx), rel=1e-12)
