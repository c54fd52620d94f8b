"""GPU parity of the SREM calls (dig_srem_reorient, dig_dwconv3x3, dig_dwconv3x3_bwd)
against the fp64 oracle.  Reorders are compared bit for bit; convolutions by the normwise
max-relative error (2e-2 bf16, 1e-4 fp32)."""
import itertools

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import TOL, announce, empty, has_gpu, maxrel, nbytes_buf, to_dev, to_f64

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not has_gpu(), reason="needs a GPU")]

DIRS = (W.ROW, W.ROW_REV, W.COL, W.COL_REV)
PAIRS = list(itertools.product(DIRS, DIRS))
DT = {"bf16": 1, "f32": 0}


def _dig():
    import diffusion_backbone_amd as dig
    return dig


def _raw_bits(t):
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy()
    return t.view(torch.int32).cpu().numpy()


@pytest.mark.parametrize("B,gh,gw,D,dtype", [
    (1, 8, 8, 64, "f32"), (2, 16, 16, 384, "bf16"), (1, 3, 5, 6, "bf16"), (2, 7, 4, 5, "bf16"),
    (1, 5, 3, 3, "f32"), (1, 112, 112, 384, "bf16"), (1, 1, 1, 8, "bf16"),
    # row kernel with several 16-byte pieces per lane: 2304-byte rows (3 per lane, DiG-XL/2
    # D = 1152 in bf16), 4608-byte rows (5 per lane, fp32); rows past 8 KiB take the
    # element-wise fallback (D = 2304 fp32: 9216-byte rows)
    (1, 16, 16, 1152, "bf16"), (1, 4, 4, 1152, "f32"), (1, 3, 3, 2304, "f32"),
    (2, 5, 7, 1152, "bf16"),
])
def test_reorient_bit_exact(B, gh, gw, D, dtype):
    dig = _dig()
    rng = np.random.default_rng(0)
    x = W.quantize(rng.standard_normal((B, gh * gw, D)), dtype)
    xd = to_dev(x, dtype)
    raw = W.storage(x, dtype)
    for frm, to in PAIRS:
        announce("reorient %dx%dx%d D=%d %s %d->%d" % (B, gh, gw, D, dtype, frm, to))
        y = empty(xd.shape, dtype)
        dig.dig_srem_reorient(B, gh, gw, D, DT[dtype], frm, to, xd, y)
        ref = oracle.reorient(raw, gh, gw, frm, to)
        got = _raw_bits(y).view(ref.dtype)
        assert np.array_equal(got, ref), (frm, to)


@pytest.mark.parametrize("B,gh,gw,D,dtype,bias", [
    (1, 8, 8, 64, "f32", False), (1, 8, 8, 64, "f32", True), (2, 16, 16, 384, "bf16", False),
    (1, 5, 7, 12, "bf16", True), (2, 3, 4, 5, "f32", True), (1, 1, 1, 8, "bf16", False),
    (1, 9, 2, 1152, "bf16", False), (2, 5, 6, 64, "f32", True),  # fewer than 8 rows: tiles
    # column-strip path (bf16 8-column strips x 64-channel slabs, fp32 16-column strips x
    # 32-channel slabs, row runs of multiples of 8): ragged rows (overlapping last row
    # group) and columns (repeated last column)
    (6, 37, 29, 384, "bf16", True), (11, 29, 37, 128, "f32", False),
])
def test_dwconv_all_layout_pairs(B, gh, gw, D, dtype, bias):
    dig = _dig()
    cfg = W.Config("t", B, gh, gw, D, 1, 1, 1, 16, dtype)
    case = W.make_srem_case(cfg, with_bias=bias)
    xd = to_dev(case.x, dtype)
    wd = torch.from_numpy(case.w.astype(np.float32)).cuda()
    bd = torch.from_numpy(case.bias.astype(np.float32)).cuda() if bias else None
    for lay, out in PAIRS:
        announce("dwconv %dx%dx%d D=%d %s bias=%d %d->%d" % (B, gh, gw, D, dtype, bias, lay, out))
        y = empty(xd.shape, dtype)
        dig.dig_dwconv3x3(B, gh, gw, D, DT[dtype], lay, out, xd, wd, bd, y)
        ref = oracle.dwconv3x3(case.x, case.w, gh, gw, lay, out, case.bias)
        e = maxrel(to_f64(y), ref)
        assert e <= TOL[dtype], (lay, out, e)


def test_dwconv_identity_kernel_equals_reorient():
    dig = _dig()
    cfg = W.CONFIGS["dig_s2_256"]
    case = W.make_srem_case(cfg, identity=True)
    xd = to_dev(case.x, "bf16")
    wd = torch.from_numpy(case.w.astype(np.float32)).cuda()
    for lay, out in PAIRS:
        announce("dwconv identity %d->%d" % (lay, out))
        y = empty(xd.shape, "bf16")
        dig.dig_dwconv3x3(cfg.batch, cfg.grid_h, cfg.grid_w, cfg.d_model, 1, lay, out, xd, wd, None, y)
        y2 = empty(xd.shape, "bf16")
        dig.dig_srem_reorient(cfg.batch, cfg.grid_h, cfg.grid_w, cfg.d_model, 1, lay, out, xd, y2)
        assert torch.equal(y.view(torch.int16), y2.view(torch.int16))


@pytest.mark.parametrize("name", ["dig_s2_1792", "dig_xl2_2048"])
def test_dwconv_full_configs(name):
    dig = _dig()
    cfg = W.CONFIGS[name]
    case = W.make_srem_case(cfg)
    xd = to_dev(case.x, "bf16")
    wd = torch.from_numpy(case.w.astype(np.float32)).cuda()
    lay, out = W.ROW, W.ROW_REV
    announce("dwconv full %s %d->%d" % (name, lay, out))
    y = empty(xd.shape, "bf16")
    dig.dig_dwconv3x3(cfg.batch, cfg.grid_h, cfg.grid_w, cfg.d_model, 1, lay, out, xd, wd, None, y)
    ref = oracle.dwconv3x3(case.x, case.w, cfg.grid_h, cfg.grid_w, lay, out)
    assert maxrel(to_f64(y), ref) <= TOL["bf16"]


@pytest.mark.parametrize("B,gh,gw,D,dtype", [
    (1, 8, 8, 64, "f32"), (2, 16, 16, 384, "bf16"), (1, 5, 7, 12, "bf16"), (2, 3, 4, 5, "f32"),
    (1, 16, 16, 1152, "bf16"), (1, 9, 2, 1152, "bf16"), (2, 5, 6, 64, "f32"),
    (6, 37, 29, 384, "bf16"), (11, 29, 37, 128, "f32"),  # column-strip path, ragged
    (8, 16, 16, 384, "bf16"),  # the benchmarked block (sums finished in the same launch)
])
def test_dwconv_bwd(B, gh, gw, D, dtype):
    dig = _dig()
    cfg = W.Config("t", B, gh, gw, D, 1, 1, 1, 16, dtype)
    case = W.make_srem_case(cfg)
    xd, dyd = to_dev(case.x, dtype), to_dev(case.dy, dtype)
    wd = torch.from_numpy(case.w.astype(np.float32)).cuda()
    wsb = dig.dig_dwconv3x3_bwd_workspace_bytes(B, gh, gw, D)
    ws = nbytes_buf(wsb)
    for lay, out in PAIRS:
        announce("dwconv bwd %dx%dx%d D=%d %s %d->%d" % (B, gh, gw, D, dtype, lay, out))
        dx = empty(xd.shape, dtype)
        dw = torch.full((D, 3, 3), float("nan"), device="cuda")
        db = torch.full((D,), float("nan"), device="cuda")
        dig.dig_dwconv3x3_bwd(B, gh, gw, D, DT[dtype], lay, out, xd, wd, dyd, dx, dw, db, ws, wsb)
        rdx, rdw, rdb = oracle.dwconv3x3_bwd(case.x, case.w, case.dy, gh, gw, lay, out)
        assert maxrel(to_f64(dx), rdx) <= TOL[dtype], "dx"
        assert maxrel(dw.cpu().numpy().astype(np.float64), rdw) <= TOL[dtype], "dw"
        assert maxrel(db.cpu().numpy().astype(np.float64), rdb) <= TOL[dtype], "dbias"
        dw2 = torch.empty_like(dw)
        dig.dig_dwconv3x3_bwd(B, gh, gw, D, DT[dtype], lay, out, xd, wd, dyd, dx, dw2, None, ws, wsb)
        assert torch.equal(dw, dw2), "dw not deterministic"


@pytest.mark.parametrize("name", ["dig_s2_1792", "dig_xl2_2048"])
def test_dwconv_bwd_full_configs(name):
    dig = _dig()
    cfg = W.CONFIGS[name]
    case = W.make_srem_case(cfg)
    B, gh, gw, D = cfg.batch, cfg.grid_h, cfg.grid_w, cfg.d_model
    xd, dyd = to_dev(case.x, "bf16"), to_dev(case.dy, "bf16")
    wd = torch.from_numpy(case.w.astype(np.float32)).cuda()
    wsb = dig.dig_dwconv3x3_bwd_workspace_bytes(B, gh, gw, D)
    ws = nbytes_buf(wsb)
    lay, out = W.COL, W.ROW_REV
    announce("dwconv bwd full %s %d->%d" % (name, lay, out))
    dx = empty(xd.shape, "bf16")
    dw = torch.empty((D, 3, 3), device="cuda")
    db = torch.empty((D,), device="cuda")
    dig.dig_dwconv3x3_bwd(B, gh, gw, D, 1, lay, out, xd, wd, dyd, dx, dw, db, ws, wsb)
    rdx, rdw, rdb = oracle.dwconv3x3_bwd(case.x, case.w, case.dy, gh, gw, lay, out)
    assert maxrel(to_f64(dx), rdx) <= TOL["bf16"], "dx"
    assert maxrel(dw.cpu().numpy().astype(np.float64), rdw) <= TOL["bf16"], "dw"
    assert maxrel(db.cpu().numpy().astype(np.float64), rdb) <= TOL["bf16"], "dbias"
