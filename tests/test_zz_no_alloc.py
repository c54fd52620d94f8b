"""The allocation-free conv backward (dig_dwconv3x3_bwd_noalloc) against the workspace entry
point (dig_dwconv3x3_bwd) and the fp64 oracle: two calls in a row, the second on a smaller
input, so the second runs over the partial sums the first left in the shared scratch array."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import TOL, announce, empty, has_gpu, maxrel, nbytes_buf, to_dev, to_f64

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not has_gpu(), reason="needs a GPU")]


def _case(B, gh, gw, D, dtype, layout, out_layout, seed):
    rng = np.random.default_rng(seed)
    x = W.quantize(rng.standard_normal((B, gh * gw, D)), dtype)
    dy = W.quantize(rng.standard_normal((B, gh * gw, D)), dtype)
    w = W.f32_round(rng.standard_normal((D, 3, 3)) / 3.0)
    return x, dy, w


def _run(dig, fn, B, gh, gw, D, dtype, layout, out_layout, x, dy, w):
    dt = dig.DIG_BF16 if dtype == "bf16" else dig.DIG_F32
    xd, dyd = to_dev(x, dtype), to_dev(dy, dtype)
    wd = torch.from_numpy(w.astype(np.float32)).cuda()
    dx = empty(xd.shape, dtype)
    dw = torch.full((D, 3, 3), float("nan"), device="cuda")
    db = torch.full((D,), float("nan"), device="cuda")
    if fn == "noalloc":
        dig.dig_dwconv3x3_bwd_noalloc(B, gh, gw, D, dt, layout, out_layout, xd, wd, dyd, dx, dw, db)
    else:
        nb = dig.dig_dwconv3x3_bwd_workspace_bytes(B, gh, gw, D)
        ws = nbytes_buf(nb)
        dig.dig_dwconv3x3_bwd(B, gh, gw, D, dt, layout, out_layout, xd, wd, dyd, dx, dw, db, ws, nb)
    torch.cuda.synchronize()
    return to_f64(dx), dw.cpu().numpy().astype(np.float64), db.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_matches_workspace_call(dtype):
    import diffusion_backbone_amd as dig
    # the XL/2 2048-px grid (column strips), then a small grid (8 x 8 tiles), other layouts
    shapes = [(1, 128, 128, 1152, W.COL, W.COL_REV), (2, 6, 9, 64, W.ROW_REV, W.COL)]
    for i, (B, gh, gw, D, lay, out) in enumerate(shapes):
        announce("no-alloc conv backward %s call %d: %dx%dx%dx%d %d->%d" % (dtype, i, B, gh, gw, D, lay, out))
        x, dy, w = _case(B, gh, gw, D, dtype, lay, out, seed=100 + i)
        got = _run(dig, "noalloc", B, gh, gw, D, dtype, lay, out, x, dy, w)
        want = _run(dig, "workspace", B, gh, gw, D, dtype, lay, out, x, dy, w)
        for a, b, n in zip(got, want, ("dx", "dw", "dbias")):
            assert np.array_equal(a, b), (n, "differs from the workspace entry point")
        rdx, rdw, rdb = oracle.dwconv3x3_bwd(x, w, dy, gh, gw, lay, out)
        for a, b, n in zip(got, (rdx, rdw, rdb), ("dx", "dw", "dbias")):
            e = maxrel(a, b)
            print("  %s err %.2e" % (n, e), flush=True)
            assert e <= TOL[dtype], (n, e)


def test_noalloc_rejects_oversized():
    import diffusion_backbone_amd as dig
    cap = dig.dig_dwconv3x3_bwd_noalloc_max_bytes()
    assert cap == 8 << 20
    B, gh, gw, D = 16, 128, 128, 1152  # partials past the scratch array
    assert dig.dig_dwconv3x3_bwd_workspace_bytes(B, gh, gw, D) > cap
    t = torch.empty(16, dtype=torch.float32, device="cuda")
    with pytest.raises(dig.DigError) as ei:
        dig.dig_dwconv3x3_bwd_noalloc(B, gh, gw, D, dig.DIG_BF16, W.ROW, W.ROW, t, t, t, t, t, None)
    assert ei.value.status == dig.DIG_ERR_WORKSPACE
