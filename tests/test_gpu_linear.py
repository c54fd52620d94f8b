"""GPU parity of dig_linear (the projections around the mixer, slides eqs. (5), (9), (10))
against the fp64 oracle: bf16 operands, fp32 accumulation, bf16 output; normwise max relative
error <= 2e-2 per output."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import TOL, announce, empty, has_gpu, maxrel, to_dev, to_f64

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not has_gpu(), reason="needs a GPU")]


def _run(m, k, ns, bias, seed, scale=1.0):
    import torch
    import diffusion_backbone_amd as dig
    rng = np.random.default_rng(seed)
    a = W.quantize(rng.standard_normal((m, k)), "bf16")
    ws = [W.quantize(rng.standard_normal((n, k)) * scale / np.sqrt(k), "bf16") for n in ns]
    bs = [W.f32_round(rng.standard_normal(n)) if bias else None for n in ns]
    ad = to_dev(a, "bf16")
    wd = [to_dev(w, "bf16") for w in ws]
    bd = [torch.from_numpy(b.astype(np.float32)).cuda() if b is not None else None for b in bs]
    cs = [empty((m, n), "bf16") for n in ns]
    dig.dig_linear(m, k, ad, list(zip(cs, wd, bd)))
    torch.cuda.synchronize()
    errs = []
    for c, w, b in zip(cs, ws, bs):
        ref = oracle.linear(a, w, b)
        errs.append(maxrel(to_f64(c), ref))
    return errs


@pytest.mark.parametrize("m,k,ns,bias", [
    (256, 64, [128], False),                 # one tile
    (300, 200, [136, 8, 264], True),          # ragged rows, K tail, narrow and ragged outputs
    (1, 8, [8], True),                        # smallest
    (2048, 384, [192, 192, 384, 16, 384], False),   # DiG-S/2 256 px: q, k, v, gate rank 16, r
    (1000, 16, [576], True),                  # the rank-16 gate up-projection (K = 16) + bias
    (4096, 1152, [576, 576, 1152, 16, 1152], False),  # DiG-XL/2 in-projection, 4096 tokens
    (4096, 1152, [1152], False),              # DiG-XL/2 out-projection
    # >= 1024 tiles of 256 x 256: the sixteen-wave tile, ragged rows and column tiles
    (33000, 64, [1152, 264, 8], True),
])
def test_linear_parity(m, k, ns, bias):
    announce("linear m=%d k=%d n=%s bias=%d" % (m, k, ns, bias))
    errs = _run(m, k, ns, bias, seed=m + k)
    print("  errs " + " ".join("%.2e" % e for e in errs), flush=True)
    for e in errs:
        assert e <= TOL["bf16"], errs


def test_linear_rejects_bad_shapes():
    import torch
    import diffusion_backbone_amd as dig
    t = torch.zeros(64, dtype=torch.bfloat16, device="cuda")
    w = torch.zeros(8, 12, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(dig.DigError) as ei:     # k not a multiple of 8
        dig.dig_linear(1, 12, t, [(t, w, None)])
    assert ei.value.status == dig.DIG_ERR_UNSUPPORTED
    with pytest.raises(dig.DigError) as ei:     # output overlapping the input
        dig.dig_linear(1, 8, t, [(t, torch.zeros(8, 8, dtype=torch.bfloat16, device="cuda"), None)])
    assert ei.value.status == dig.DIG_ERR_ALIAS


@pytest.mark.parametrize("m,k,n,act,gated", [
    (2048, 1536, 384, 0, True),       # DiG-S/2 256 px second feedforward matrix: 48 tiles
    (512, 1152, 384, 0, True),        # an XL/2-width out-projection on a small batch
    (1024, 1152, 1536, 1, False),     # a feedforward matrix with GELU, 96 tiles
    (300, 1000, 136, 0, False),       # ragged rows and K
])
def test_linear_split_k_parity(m, k, n, act, gated):
    """dig_linear_ws: K split into fp32 partial sums in the workspace, finished with the same
    epilogue; against the oracle, and the workspace query is non-zero for these grids."""
    import torch
    import diffusion_backbone_amd as dig
    announce("linear split-K m=%d k=%d n=%d act=%d gated=%d" % (m, k, n, act, gated))
    rng = np.random.default_rng(m + k + n)
    a = W.quantize(rng.standard_normal((m, k)), "bf16")
    w = W.quantize(rng.standard_normal((n, k)) / np.sqrt(k), "bf16")
    b = W.f32_round(rng.standard_normal(n) * 0.5)
    res = W.quantize(rng.standard_normal((m, n)), "bf16")
    gate = W.quantize(rng.standard_normal((2, n)), "bf16")
    rpg = (m + 1) // 2
    c = to_dev(res, "bf16") if gated else empty((m, n), "bf16")
    o = dig.linear_out(c, to_dev(w, "bf16"),
                       torch.from_numpy(b.astype(np.float32)).cuda(), act=act,
                       res=c if gated else None, gate=to_dev(gate, "bf16") if gated else None,
                       gate_ld=n, rows_per_gate=rpg)
    need = dig.dig_linear_workspace_bytes(m, k, [o])
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    dig.dig_linear_ws(m, k, to_dev(a, "bf16"), [o], ws)
    torch.cuda.synchronize()
    t = oracle.linear(a, w, b)
    if act:
        t = oracle.gelu(t)
    ref = res + gate[np.arange(m) // rpg] * t if gated else t
    e = maxrel(to_f64(c), ref)
    print("  err %.2e (workspace %d bytes)" % (e, need), flush=True)
    assert e <= TOL["bf16"]
    with pytest.raises(dig.DigError) as ei:
        dig.dig_linear_ws(m, k, to_dev(a, "bf16"), [o], ws, workspace_bytes=need - 16)
    assert ei.value.status == dig.DIG_ERR_WORKSPACE


def test_linear_split_k_not_needed_on_full_grids():
    import torch
    import diffusion_backbone_amd as dig
    c = torch.empty(16384, 1152, dtype=torch.bfloat16, device="cuda")
    w = torch.empty(1152, 1152, dtype=torch.bfloat16, device="cuda")
    assert dig.dig_linear_workspace_bytes(16384, 1152, [(c, w, None)]) == 0


@pytest.mark.parametrize("m,k,ns,act", [(1000, 1024, [136, 8, 264], 0),
                                        (600, 1152, [264, 136], 1),
                                        (16384, 1152, [576, 576, 1152, 16, 1152], 0)])
def test_linear_packed_outputs(m, k, ns, act):
    """Several outputs with K >= 1024 run with their columns packed side by side (tiles that
    straddle outputs): per-column bias and activation, ragged widths."""
    import torch
    import diffusion_backbone_amd as dig
    announce("linear packed m=%d k=%d n=%s act=%d" % (m, k, ns, act))
    rng = np.random.default_rng(m + k + len(ns))
    a = W.quantize(rng.standard_normal((m, k)), "bf16")
    ws = [W.quantize(rng.standard_normal((n, k)) / np.sqrt(k), "bf16") for n in ns]
    bs = [W.f32_round(rng.standard_normal(n) * 0.5) for n in ns]
    cs = [empty((m, n), "bf16") for n in ns]
    dig.dig_linear(m, k, to_dev(a, "bf16"),
                   [dig.linear_out(c, to_dev(w, "bf16"),
                                   torch.from_numpy(b.astype(np.float32)).cuda(), act=act)
                    for c, w, b in zip(cs, ws, bs)])
    torch.cuda.synchronize()
    errs = []
    for c, w, b in zip(cs, ws, bs):
        ref = oracle.linear(a, w, b)
        errs.append(maxrel(to_f64(c), oracle.gelu(ref) if act else ref))
    print("  errs " + " ".join("%.2e" % e for e in errs), flush=True)
    assert max(errs) <= TOL["bf16"], errs
