"""GPU parity of the DiG-S/2 256-px twelve-block chain (the mixer and SREM step of every block,
four scan directions cycling ROW, ROW_REV, COL, COL_REV).

Block l runs in scan order d(l): its input x_l is projected to q, k, v, z, r (fp64 matmuls,
bf16 operands), the mixer runs, the output projection and the residual give x_l + Y_l W_O, and
the 3x3 conv runs on the current-order grid and writes the next block's order d(l+1) (DiG
write-up, section 3 "DiG Block").  On the GPU the mixer is dig_gla_fwd and the conv
dig_dwconv3x3; the oracle runs the same chain with its own functions.  The oracle's chain runs
free (bf16 at every block boundary); the GPU runs each block on the oracle's input to that
block, so both sides see the same values and no oracle input ever comes from the GPU.  Every
block's mixer output and SREM output are compared.  A second GPU chain fed by its own outputs
runs beside it; its drift from the oracle's chain is logged (tiny rounding differences between
two valid chains grow through the RMSNorm of tokens whose o nearly cancels, so it is a
diagnostic, not a bound).
"""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import TOL, announce, empty, gla_forward, has_gpu, maxrel, to_dev, to_f64

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not has_gpu(), reason="needs a GPU")]


def test_chain_dig_s2_256_twelve_blocks():
    import torch
    import diffusion_backbone_amd as dig
    cfg = W.CONFIGS["dig_s2_256"]
    B, gh, gw, D = cfg.batch, cfg.grid_h, cfg.grid_w, cfg.d_model
    rng = np.random.default_rng(cfg.seed + 77)
    wts = [W.make_block_weights(cfg, rng) for _ in range(cfg.blocks)]
    gamma = np.ones(cfg.d_v)
    x_ref = W.quantize(rng.standard_normal((B, cfg.seq_len, D)), "bf16")   # ROW order
    x_free = x_ref.copy()

    def gpu_block(x, l, d, dn):
        q, k, v, z, r = W.project(cfg, x, wts[l])
        f = gla_forward(W.GLACase(cfg, q, k, v, z, r, gamma, None), cfg.chunk, want_opre=False)
        y = to_f64(f["y"])
        res = W.quantize(x + y.reshape(B, cfg.seq_len, -1) @ wts[l].wo, "bf16")
        wd = torch.from_numpy(wts[l].conv_w.astype(np.float32)).cuda()
        out = empty((B, cfg.seq_len, D), "bf16")
        dig.dig_dwconv3x3(B, gh, gw, D, dig.DIG_BF16, d, dn, to_dev(res, "bf16"), wd, None, out)
        torch.cuda.synchronize()
        return y, to_f64(out)

    for l in range(cfg.blocks):
        d, dn = W.SCHEDULE[l % 4], W.SCHEDULE[(l + 1) % 4]
        announce("chain block %d: %s -> %s" % (l, W.SCAN_NAMES[d], W.SCAN_NAMES[dn]))
        y, x_next = gpu_block(x_ref, l, d, dn)            # the oracle's input to block l
        _, x_free = gpu_block(x_free, l, d, dn)           # the GPU's own chain
        qr, kr, vr, zr, rr = W.project(cfg, x_ref, wts[l])
        yr, _, _ = oracle.gla_fwd(qr, kr, vr, zr, rr, gamma)
        res_r = W.quantize(x_ref + yr.reshape(B, cfg.seq_len, -1) @ wts[l].wo, "bf16")
        x_ref = W.quantize(oracle.dwconv3x3(res_r, wts[l].conv_w, gh, gw, d, dn), "bf16")
        ey = maxrel(y, yr)
        ec = maxrel(x_next, x_ref)
        print("  block %2d %-7s y=%.2e srem=%.2e  GPU's own chain drift %.2e"
              % (l, W.SCAN_NAMES[d], ey, ec, maxrel(x_free, x_ref)), flush=True)
        assert ey <= TOL["bf16"], ("y", l, ey)
        assert ec <= TOL["bf16"], ("srem", l, ec)
