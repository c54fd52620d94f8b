"""GPU parity of the GLA mixer with the low-rank key gate formed inside the chunk kernels
(dig_gla_fwd_lowrank / dig_gla_bwd_lowrank; slides eq. (5): the gate logits are
(x W_a1) W_a2 + b_alpha) against the fp64 oracle, which forms the logits with
lowrank_gate_logits and runs its own mixer on them.

Both sides get the same quantised q, k, v, r, dy, factor, W_a2 (bf16) and b_alpha (fp32);
the GPU's logits are fp32 sums of the bf16 products, the oracle's exact.  Bar: normwise
max-relative error <= 2e-2 per output (bf16 I/O), outputs NaN-poisoned before each call.
Shapes cover the exact head shapes (S: 32/64, XL: 36/72) and a tile class, every chunk size,
ragged tails, one-launch look-back and three-pass plans, strong-decay chunks, and the full
DiG-XL/2 2048-px layer.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import (TOL, announce, empty, gla_backward, gla_forward, has_gpu, maxrel,
                      nbytes_buf, to_dev, to_f64)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not has_gpu(), reason="needs a GPU")]

GRADS = ("dq", "dk", "dv", "dz", "dr")


def _case(name, seed, *, batch=None, seq_len=None, dk=None, dv=None, **gate_kw):
    cfg = W.CONFIGS[name]
    if dk is not None:
        cfg = W.cfg_replace(cfg, d_k=dk, d_v=dv)
    case = W.make_gla_case(cfg, seed, batch=batch, seq_len=seq_len, random_gamma=True)
    B, L, H, d_k = case.q.shape
    gate = W.make_lowrank_gate(cfg, seed + 1000, batch=B, seq_len=L, **gate_kw)
    z = oracle.lowrank_gate_logits(gate.factor, gate.w, gate.bias, H, d_k)
    return W.GLACase(cfg, case.q, case.k, case.v, z, case.r, case.gamma, case.dy), gate


def _check(case, gate, chunk, seg, what, bwd=True):
    f = gla_forward(case, chunk, seg_chunks=seg, want_saved=bwd, lowrank=gate)
    y_ref, o_ref, _ = oracle.gla_fwd(case.q, case.k, case.v, case.z, case.r, case.gamma)
    errs = {"y": maxrel(to_f64(f["y"]), y_ref), "o_pre": maxrel(to_f64(f["o_pre"]), o_ref)}
    if bwd:
        g = gla_backward(case, f)
        ref = oracle.gla_bwd(case.q, case.k, case.v, case.z, case.r, case.dy, case.gamma)
        for n in GRADS:
            errs[n] = maxrel(to_f64(g[n]), ref[n])
        errs["dgamma"] = maxrel(g["dgamma"].cpu().numpy().astype(np.float64), ref["dgamma"])
    print("  %s " % what + " ".join("%s=%.2e" % kv for kv in errs.items()), flush=True)
    for n, e in errs.items():
        assert e <= TOL["bf16"], (n, e)
    return f


@pytest.mark.parametrize("name,batch,seq_len,chunk,seg", [
    ("dig_s2_256", 2, 256, 64, 0),     # S head shape, four chunks: one-launch look-back
    ("dig_s2_256", 1, 600, 64, 2),     # S, ragged, three passes
    ("dig_s2_256", 1, 200, 16, 0),     # S, chunk 16
    ("dig_xl2_2048", 1, 256, 64, 0),   # XL head shape, look-back
    ("dig_xl2_2048", 1, 640, 64, 2),   # XL, three passes (the reading final pass)
    ("dig_xl2_2048", 2, 87, 32, 0),    # XL, ragged, chunk 32
    ("dig_xl2_2048", 1, 300, 64, 100), # XL, one segment (the recomputing final pass)
])
def test_lowrank_exact_shapes(name, batch, seq_len, chunk, seg):
    announce("lowrank %s B=%d L=%d chunk=%d seg=%d" % (name, batch, seq_len, chunk, seg))
    case, gate = _case(name, 11 + seq_len, batch=batch, seq_len=seq_len)
    _check(case, gate, chunk, seg, name)


@pytest.mark.parametrize("dk,dv,chunk,seq_len", [(20, 40, 16, 77), (40, 72, 32, 150),
                                                  (64, 100, 32, 130)])
def test_lowrank_tile_classes(dk, dv, chunk, seq_len):
    announce("lowrank tile class dk=%d dv=%d chunk=%d L=%d" % (dk, dv, chunk, seq_len))
    case, gate = _case("dig_s2_256", 7 + dk, batch=2, seq_len=seq_len, dk=dk, dv=dv)
    _check(case, gate, chunk, 0, "dk=%d dv=%d" % (dk, dv))


@pytest.mark.parametrize("stress", ["wide", "strong_decay", "saturated"])
@pytest.mark.parametrize("seg", [0, 2])
def test_lowrank_gate_stress(stress, seg):
    # wide: logits ~ N(0, 4); strong_decay: b_alpha ~ -20 +- 5 (chunks take the strong-decay
    # path); saturated: b_alpha ~ +12 +- 4 (alpha -> 1, sigmoid(-z) tiny in dz)
    kw = {"wide": dict(w_std=0.5), "strong_decay": dict(w_std=0.5, bias_mean=-20.0, bias_std=5.0),
          "saturated": dict(w_std=0.3, bias_mean=12.0, bias_std=4.0)}[stress]
    announce("lowrank stress %s seg=%d" % (stress, seg))
    case, gate = _case("dig_xl2_2048", 31, batch=1, seq_len=320, **kw)
    _check(case, gate, 64, seg, stress)


def test_lowrank_full_xl2_2048():
    announce("lowrank fwd+bwd dig_xl2_2048 full B=1 L=16384")
    case, gate = _case("dig_xl2_2048", 5)
    _check(case, gate, 64, 0, "xl2_2048")


def test_lowrank_deterministic_and_matches_block_rule():
    # two calls give identical bits (fixed summation order of the logits and of dgamma)
    case, gate = _case("dig_s2_256", 3, batch=2, seq_len=256)
    f1 = _check(case, gate, 64, 0, "first")
    f2 = gla_forward(case, 64, want_saved=True, lowrank=gate)
    assert np.array_equal(to_f64(f1["y"]), to_f64(f2["y"]))
    g1, g2 = gla_backward(case, f1), gla_backward(case, f2)
    for n in GRADS:
        assert np.array_equal(to_f64(g1[n]), to_f64(g2[n])), n


def test_lowrank_rejects_bad_arguments():
    import torch
    import diffusion_backbone_amd as dig
    B, L, H, dk, dv = 1, 128, 2, 32, 64
    desc = dig.make_desc(B, L, H, dk, dv, 64, 16.0, 1.0, 1e-5, "bf16", 0)
    bf = lambda *s: torch.zeros(*s, dtype=torch.bfloat16, device="cuda")
    q, k, z = bf(B, L, H, dk), bf(B, L, H, dk), bf(B, L, H, dk)
    v, r, y = bf(B, L, H, dv), bf(B, L, H, dv), bf(B, L, H, dv)
    f, w = bf(B, L, 16), bf(H * dk, 16)
    b = torch.zeros(H * dk, dtype=torch.float32, device="cuda")
    wsb = dig.dig_gla_fwd_workspace_bytes(desc)
    ws = nbytes_buf(wsb)

    def code(**over):
        a = dict(q=q, k=k, v=v, f=f, w=w, b=b, r=r, y=y, rank=16, desc=desc)
        a.update(over)
        try:
            dig.dig_gla_fwd_lowrank(a["desc"], a["q"], a["k"], a["v"], a["f"], a["w"], a["b"],
                                    a["r"], None, a["y"], None, None, ws, wsb,
                                    gate_rank=a["rank"])
        except dig.DigError as e:
            return e.status
        return dig.DIG_OK

    assert code() == dig.DIG_OK
    torch.cuda.synchronize()
    assert code(rank=8) == dig.DIG_ERR_UNSUPPORTED
    assert code(f=None) == dig.DIG_ERR_NULL
    assert code(w=None) == dig.DIG_ERR_NULL
    fo = bf(B * L * 16 + 8)
    assert code(f=fo[1:]) == dig.DIG_ERR_ALIGN               # factor 2 bytes off
    yw = bf(max(B * L * H * dv, H * dk * 16))
    assert code(y=yw, w=yw) == dig.DIG_ERR_ALIAS              # W_a2 overlapping y
    f32desc = dig.make_desc(B, L, H, dk, dv, 64, 16.0, 1.0, 1e-5, "f32", 0)
    assert code(desc=f32desc) == dig.DIG_ERR_UNSUPPORTED      # bf16 only
