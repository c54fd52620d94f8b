"""GPU parity of the GLA mixer (dig_gla_fwd / dig_gla_bwd) against the fp64 oracle.

Every case feeds identical quantised inputs to both sides and compares element by element
with the normwise max-relative error max|gpu - ref| / max|ref|: <= 2e-2 for bf16 I/O and
<= 1e-4 for fp32 I/O.  Outputs are NaN-poisoned before each call so unwritten elements fail.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import (TOL, announce, gla_backward, gla_forward, has_gpu, maxrel, nbytes_buf,
                      to_dev, to_f64)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not has_gpu(), reason="needs a GPU")]


def _ref_fwd(case, q_scale=1.0, tau=16.0):
    return oracle.gla_fwd(case.q, case.k, case.v, case.z, case.r, case.gamma, tau=tau,
                          q_scale=q_scale)


def _check_fwd(case, out, tol, q_scale=1.0, tau=16.0, what=""):
    y_ref, o_ref, _ = _ref_fwd(case, q_scale, tau)
    ey = maxrel(to_f64(out["y"]), y_ref)
    eo = maxrel(to_f64(out["o_pre"]), o_ref) if out.get("o_pre") is not None else 0.0
    print("  %s err y=%.3e o_pre=%.3e (tol %.0e)" % (what, ey, eo, tol), flush=True)
    assert ey <= tol, ("y", ey)
    assert eo <= tol, ("o_pre", eo)
    return y_ref


def _case(name, **kw):
    cfg = W.CONFIGS[name]
    over = {k: kw.pop(k) for k in list(kw) if k in ("batch", "seq_len")}
    cfg_over = {k: kw.pop(k) for k in list(kw) if k in ("dtype",)}
    if cfg_over:
        cfg = W.cfg_replace(cfg, **cfg_over)
    return W.make_gla_case(cfg, **over, **kw)


# ----------------------------------------------------------------------- forward
@pytest.mark.parametrize("chunk", [16, 32, 64])
@pytest.mark.parametrize("seg", [0, 1])
def test_fwd_tiny_f32(chunk, seg):
    announce("fwd tiny_f32 chunk=%d seg=%d" % (chunk, seg))
    case = _case("tiny_f32", random_gamma=True)
    out = gla_forward(case, chunk, seg_chunks=seg)
    _check_fwd(case, out, TOL["f32"])


@pytest.mark.parametrize("name,batch,seq_len,chunk,seg", [
    ("dig_s2_256", 2, 256, 64, 0),
    ("dig_s2_256", 2, 256, 64, 1),
    ("dig_s2_256", 1, 200, 64, 0),     # ragged tail
    ("dig_s2_256", 1, 777, 32, 2),     # ragged, several segments
    ("dig_s2_256", 1, 100, 16, 1),
    ("dig_xl2_1024", 1, 1000, 64, 0),  # padded head dims 36/72, ragged
    ("dig_xl2_1024", 1, 1000, 64, 3),
    ("dig_xl2_1024", 2, 130, 16, 2),
    ("dig_xl2_1024", 1, 1, 64, 0),     # single token
])
def test_fwd_bf16_shapes(name, batch, seq_len, chunk, seg):
    announce("fwd %s B=%d L=%d chunk=%d seg=%d" % (name, batch, seq_len, chunk, seg))
    case = _case(name, batch=batch, seq_len=seq_len, random_gamma=True)
    out = gla_forward(case, chunk, seg_chunks=seg)
    _check_fwd(case, out, TOL["bf16"])


@pytest.mark.parametrize("stress", ["long_memory", "fast_decay", "wide_logits", "extreme_decay"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_fwd_gate_stress(stress, dtype):
    kw = {"long_memory": dict(gate_bias=6.0), "fast_decay": dict(gate_bias=-6.0),
          "wide_logits": dict(z_std=4.0), "extreme_decay": dict(gate_bias=-40.0, z_std=1.0)}[stress]
    announce("fwd stress %s %s" % (stress, dtype))
    case = _case("dig_s2_256", batch=1, seq_len=300, dtype=dtype, **kw)
    out = gla_forward(case, 64, seg_chunks=2)
    _check_fwd(case, out, TOL[dtype])
    if dtype == "bf16":  # the XL head shape (padded key tiles, four waves) on the same gates
        cx = _case("dig_xl2_2048", batch=1, seq_len=300, dtype=dtype, **kw)
        _check_fwd(cx, gla_forward(cx, 64, seg_chunks=2), TOL[dtype])
    if dtype == "f32":  # fp32 backward at these head dims fits LDS with 32-token chunks
        f = gla_forward(case, 32, seg_chunks=3, want_saved=True)
        _check_fwd(case, f, TOL[dtype])
        _check_bwd(case, gla_backward(case, f), TOL[dtype])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_fwd_cancelling_first_token(dtype):
    """o_0 = (q_0.k_0) v_0; with q_0.k_0 near zero the head-wise RMSNorm magnifies any
    error of that dot product, so the diagonal of the chunk's gated Q K^T must be exact."""
    announce("fwd cancelling first token %s" % dtype)
    case = _case("dig_xl2_1024", batch=1, seq_len=130, dtype=dtype)
    q0, k0 = case.q[:, 0], case.k[:, 0]                       # [B, H, dk]
    proj = np.sum(q0 * k0, -1, keepdims=True) / np.sum(q0 * q0, -1, keepdims=True)
    case.k[:, 0] = W.quantize(k0 - proj * q0, dtype)          # q_0.k_0 ~ rounding level
    out = gla_forward(case, 64 if dtype == "bf16" else 32)   # fp32 XL tiles fit LDS at 32
    _check_fwd(case, out, TOL[dtype])


def test_fwd_q_scale_tau_and_no_gamma():
    announce("fwd q_scale=0.5 tau=4 gamma=None")
    case = _case("dig_xl2_1024", batch=1, seq_len=160)
    out = gla_forward(case, 32, q_scale=0.5, tau=4.0, gamma=False)
    case.gamma = np.ones_like(case.gamma)
    _check_fwd(case, out, TOL["bf16"], q_scale=0.5, tau=4.0)


def test_fwd_chunk_invariance_and_determinism():
    announce("fwd chunk invariance S shapes")
    case = _case("dig_s2_256", batch=2, seq_len=256)
    y_ref, _, _ = _ref_fwd(case)
    outs = []
    for chunk in (16, 32, 64):
        o = gla_forward(case, chunk)
        outs.append(to_f64(o["y"]))
        assert maxrel(outs[-1], y_ref) <= TOL["bf16"]
    for a in outs[1:]:
        assert maxrel(a, outs[0]) <= TOL["bf16"]
    a = to_f64(gla_forward(case, 64, seg_chunks=1)["y"])
    b = to_f64(gla_forward(case, 64, seg_chunks=1)["y"])
    assert np.array_equal(a, b), "two identical runs differ"


# Short sequences whose chunks fit one round of workgroups run the forward as one launch: a
# workgroup per chunk, the state entering it from the earlier chunks through the look-back.
@pytest.mark.parametrize("name,dtype,batch,seq_len,chunk", [
    ("dig_s2_256", "bf16", 8, 256, 64),     # the benchmarked block: 4 chunks, 192 workgroups
    ("dig_s2_256", "bf16", 1, 130, 64),     # 3 chunks, a ragged tail of 2 tokens
    ("dig_s2_256", "bf16", 5, 512, 64),     # 8 chunks, the longest look-back
    ("dig_xl2_2048", "bf16", 1, 450, 64),   # padded head tiles (36, 72), 8 chunks, ragged
    ("dig_xl2_2048", "bf16", 2, 65, 64),    # 2 chunks, the second holds one token
    ("tiny_f32", "bf16", 3, 200, 64),       # (16, 32) heads, four waves
    ("tiny_f32", "f32", 2, 200, 32),        # fp32, 32-token chunks, 7 chunks
])
@pytest.mark.parametrize("saved", [True, False])
def test_fwd_lookback_shapes(name, dtype, batch, seq_len, chunk, saved):
    announce("fwd lookback %s %s B=%d L=%d chunk=%d saved=%d" % (name, dtype, batch, seq_len,
                                                                 chunk, saved))
    case = _case(name, batch=batch, seq_len=seq_len, dtype=dtype, random_gamma=True)
    f = gla_forward(case, chunk, want_saved=saved)
    _check_fwd(case, f, TOL[dtype])
    if saved and dtype == "bf16":  # the saved states feed the backward
        _check_bwd(case, gla_backward(case, f), TOL[dtype])


@pytest.mark.parametrize("stress", ["long_memory", "fast_decay", "wide_logits", "extreme_decay"])
def test_fwd_lookback_gate_stress(stress):
    kw = {"long_memory": dict(gate_bias=6.0), "fast_decay": dict(gate_bias=-6.0),
          "wide_logits": dict(z_std=4.0), "extreme_decay": dict(gate_bias=-40.0, z_std=1.0)}[stress]
    announce("fwd lookback stress %s" % stress)
    for name in ("dig_s2_256", "dig_xl2_2048"):
        case = _case(name, batch=1, seq_len=300, **kw)   # five chunks
        _check_fwd(case, gla_forward(case, 64), TOL["bf16"], what=name)


def test_fwd_lookback_workspace_reuse():
    """One workspace across forward calls with other inputs (stale flags must not match), and
    a repeated call gives the same bits."""
    announce("fwd lookback workspace reuse")
    a = _case("dig_s2_256", batch=4, seq_len=256, random_gamma=True)
    b = W.make_gla_case(W.CONFIGS["dig_s2_256"], seed=4321, batch=4, seq_len=256,
                        random_gamma=True)
    fa = gla_forward(a, 64, want_saved=True)
    ws = fa["ws"]
    fb = gla_forward(b, 64, want_saved=True, ws=ws)
    _check_fwd(b, fb, TOL["bf16"], what="second call")
    fa2 = gla_forward(a, 64, want_saved=True, ws=ws)
    _check_fwd(a, fa2, TOL["bf16"], what="third call")
    assert np.array_equal(to_f64(fa["y"]), to_f64(fa2["y"]))


@pytest.mark.parametrize("batch,seq_len", [
    (16, 512),   # 2 heads x 8 chunks x 16 images = 256 workgroups: the largest look-back grid
    (17, 512),   # 272: one past it (segments and a scan instead)
    (1, 577),    # 10 chunks: past the look-back's longest sequence
])
def test_lookback_plan_boundary(batch, seq_len):
    announce("look-back plan boundary B=%d L=%d" % (batch, seq_len))
    case = _case("tiny_f32", batch=batch, seq_len=seq_len, dtype="bf16", random_gamma=True)
    f = gla_forward(case, 64, want_saved=True)
    _check_fwd(case, f, TOL["bf16"])
    _check_bwd(case, gla_backward(case, f), TOL["bf16"])


def test_lookback_graph_replay():
    """dig_gla_fwd + dig_gla_bwd captured once in a HIP graph (the same look-back tag on every
    replay) and replayed over new inputs, with eager work and synchronisation between the
    replays: each replay must give the eager call's bits for the same inputs (each launch
    clears its flags, so a replay never meets flags raised by an earlier one)."""
    import torch
    import diffusion_backbone_amd as dig
    announce("look-back fwd+bwd graph replay")
    cfg = W.CONFIGS["dig_s2_256"]
    cases = [W.make_gla_case(cfg, seed=sd, batch=4, seq_len=256, random_gamma=True)
             for sd in (11, 12, 13, 11)]
    c0 = cases[0]
    B, L, H, dk = c0.q.shape
    dv = c0.v.shape[-1]
    desc = dig.make_desc(B, L, H, dk, dv, 64, 16.0, 1.0, 1e-5, "bf16", 0)
    names = ("q", "k", "v", "z", "r", "dy")
    inp = {n: to_dev(getattr(c0, n), "bf16") for n in names}
    gam = torch.from_numpy(c0.gamma.astype(np.float32)).cuda()
    y = torch.empty(B, L, H, dv, dtype=torch.bfloat16, device="cuda")
    saved = nbytes_buf(dig.dig_gla_saved_bytes(desc))
    fwb, bwb = dig.dig_gla_fwd_workspace_bytes(desc), dig.dig_gla_bwd_workspace_bytes(desc)
    fws, bws = nbytes_buf(fwb), nbytes_buf(bwb)
    grads = {n: torch.empty(B, L, H, dk, dtype=torch.bfloat16, device="cuda") for n in ("dq", "dk", "dz")}
    grads.update({n: torch.empty(B, L, H, dv, dtype=torch.bfloat16, device="cuda") for n in ("dv", "dr")})
    dgm = torch.empty(dv, device="cuda")

    def step():
        dig.dig_gla_fwd(desc, inp["q"], inp["k"], inp["v"], inp["z"], inp["r"], gam, y, None,
                        saved, fws, fwb)
        dig.dig_gla_bwd(desc, inp["q"], inp["k"], inp["v"], inp["z"], inp["r"], gam, inp["dy"],
                        saved, grads["dq"], grads["dk"], grads["dv"], grads["dz"], grads["dr"],
                        dgm, bws, bwb)

    def load(case):
        for n in names:
            inp[n].copy_(to_dev(getattr(case, n), "bf16"))
        gam.copy_(torch.from_numpy(case.gamma.astype(np.float32)))

    def outputs():
        return [to_f64(y)] + [to_f64(grads[n]) for n in GRADS] + [dgm.cpu().numpy().copy()]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for i, case in enumerate(cases):
        load(case)
        step()                      # eager reference for these inputs
        torch.cuda.synchronize()
        want = outputs()
        y.fill_(float("nan"))
        dgm.fill_(float("nan"))
        for n in GRADS:
            grads[n].fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        got = outputs()
        for a, b in zip(got, want):
            assert np.array_equal(a, b), "replay %d differs from the eager call" % i
    _check_fwd(cases[-1], {"y": y}, TOL["bf16"], what="last replay")


def test_fwd_config_dig_s2_256_full():
    announce("fwd dig_s2_256 full B=8 L=256")
    case = _case("dig_s2_256")
    out = gla_forward(case, 64)
    _check_fwd(case, out, TOL["bf16"], what="dig_s2_256")


def test_fwd_config_dig_s2_1792_full():
    announce("fwd dig_s2_1792 full B=1 L=12544")
    case = _case("dig_s2_1792")
    out = gla_forward(case, 64)
    _check_fwd(case, out, TOL["bf16"], what="dig_s2_1792")


def test_fwd_config_dig_xl2_1024_four_directions():
    cfg = W.CONFIGS["dig_xl2_1024"]
    base = W.make_gla_case(cfg)
    for d in W.SCHEDULE:
        announce("fwd dig_xl2_1024 full direction=%s" % W.SCAN_NAMES[d])
        # the same image tokens, stored in scan order d
        re = lambda a: oracle.reorient(a.reshape(cfg.batch, cfg.seq_len, -1), cfg.grid_h, cfg.grid_w,
                                       W.ROW, d).reshape(a.shape)
        case = W.GLACase(cfg, re(base.q), re(base.k), re(base.v), re(base.z), re(base.r),
                         base.gamma, re(base.dy))
        out = gla_forward(case, 64, want_opre=False)
        _check_fwd(case, out, TOL["bf16"], what="xl2_1024 dir %d" % d)


# ---------------------------------------------------------------------- backward
GRADS = ("dq", "dk", "dv", "dz", "dr")


def _diag(got, ref):
    """Elementwise diagnostics (logged, not asserted): where the normwise error peaks
    (token, head) and the largest elementwise relative error over the elements whose
    reference exceeds 1e-3 of the tensor's max."""
    d = np.abs(got - ref)
    at = np.unravel_index(int(np.argmax(d)), d.shape)
    big = np.abs(ref) > 1e-3 * np.max(np.abs(ref))
    ew = float(np.max(d[big] / np.abs(ref[big]))) if np.any(big) else 0.0
    return "t%d/h%d ew%.1e" % (at[1], at[2], ew)


def _check_bwd(case, g, tol, what=""):
    ref = oracle.gla_bwd(case.q, case.k, case.v, case.z, case.r, case.dy, case.gamma)
    got = {n: to_f64(g[n]) for n in GRADS}
    errs = {n: maxrel(got[n], ref[n]) for n in GRADS}
    if g.get("dgamma") is not None:
        errs["dgamma"] = maxrel(g["dgamma"].cpu().numpy().astype(np.float64), ref["dgamma"])
    print("  %s " % what + " ".join("%s=%.2e" % kv for kv in errs.items()), flush=True)
    print("    at " + " ".join("%s:%s" % (n, _diag(got[n], ref[n])) for n in GRADS), flush=True)
    for n, e in errs.items():
        assert e <= tol, (n, e)
    return errs


@pytest.mark.parametrize("chunk", [16, 32, 64])
@pytest.mark.parametrize("seg", [0, 1])
def test_bwd_tiny_f32(chunk, seg):
    announce("bwd tiny_f32 chunk=%d seg=%d" % (chunk, seg))
    case = _case("tiny_f32", random_gamma=True)
    f = gla_forward(case, chunk, seg_chunks=seg, want_saved=True)
    g = gla_backward(case, f)
    _check_bwd(case, g, TOL["f32"])


@pytest.mark.parametrize("name,batch,seq_len,chunk,seg", [
    ("dig_s2_256", 2, 256, 64, 0),
    ("dig_s2_256", 1, 333, 64, 2),
    ("dig_s2_256", 1, 100, 16, 1),
    ("dig_xl2_2048", 1, 256, 64, 0),   # the 16x16 crop of the 2048-px config
    ("dig_xl2_2048", 1, 256, 64, 1),
    ("dig_xl2_2048", 1, 999, 32, 3),
    ("dig_xl2_2048", 1, 150, 16, 0),   # XL at chunk 16: more column groups than key columns
    ("dig_xl2_2048", 1, 300, 16, 4),
])
def test_bwd_bf16_shapes(name, batch, seq_len, chunk, seg):
    announce("bwd %s B=%d L=%d chunk=%d seg=%d" % (name, batch, seq_len, chunk, seg))
    case = _case(name, batch=batch, seq_len=seq_len, random_gamma=True)
    f = gla_forward(case, chunk, seg_chunks=seg, want_saved=True)
    _check_fwd(case, f, TOL["bf16"])
    g = gla_backward(case, f)
    _check_bwd(case, g, TOL["bf16"])


# head dims outside the exact DiG shapes run in the enclosing 16-wide tile class
@pytest.mark.parametrize("dk,dv,chunk,seq_len,seg", [(20, 40, 16, 77, 0), (40, 72, 32, 150, 0),
                                                     (64, 100, 32, 130, 0), (64, 100, 32, 130, 2),
                                                     (64, 128, 16, 90, 0), (50, 80, 32, 70, 100)])
def test_bwd_bf16_tile_classes(dk, dv, chunk, seq_len, seg):
    announce("bwd tile class dk=%d dv=%d chunk=%d L=%d seg=%d" % (dk, dv, chunk, seq_len, seg))
    cfg = W.cfg_replace(W.CONFIGS["dig_s2_256"], d_k=dk, d_v=dv)
    case = W.make_gla_case(cfg, 7 + dk, batch=2, seq_len=seq_len, random_gamma=True)
    f = gla_forward(case, chunk, seg_chunks=seg, want_saved=True)
    _check_fwd(case, f, TOL["bf16"])
    g = gla_backward(case, f)
    _check_bwd(case, g, TOL["bf16"])


@pytest.mark.parametrize("stress", ["long_memory", "fast_decay", "wide_logits", "extreme_decay"])
@pytest.mark.parametrize("name", ["dig_s2_256", "dig_xl2_2048"])
@pytest.mark.parametrize("seg", [2, 0])   # 0: five chunks, one per workgroup (look-back)
def test_bwd_gate_stress(stress, name, seg):
    kw = {"long_memory": dict(gate_bias=6.0), "fast_decay": dict(gate_bias=-6.0),
          "wide_logits": dict(z_std=4.0), "extreme_decay": dict(gate_bias=-40.0, z_std=1.0)}[stress]
    announce("bwd stress %s %s seg=%d" % (stress, name, seg))
    case = _case(name, batch=1, seq_len=300, **kw)
    f = gla_forward(case, 64, seg_chunks=seg, want_saved=True)
    g = gla_backward(case, f)
    _check_bwd(case, g, TOL["bf16"])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_bwd_cancelling_first_token(dtype):
    """With o_0 parallel to v_0 the RMSNorm gradient makes do_0.v_0 cancel; the gradients of
    the first token must still match."""
    announce("bwd cancelling first token %s" % dtype)
    case = _case("dig_xl2_2048", batch=1, seq_len=96, dtype=dtype)
    q0, k0 = case.q[:, 0], case.k[:, 0]
    proj = np.sum(q0 * k0, -1, keepdims=True) / np.sum(q0 * q0, -1, keepdims=True)
    case.k[:, 0] = W.quantize(k0 - 0.98 * proj * q0, dtype)   # small but not zero q_0.k_0
    f = gla_forward(case, 16 if dtype == "f32" else 64, want_saved=True)  # fp32 XL: LDS fit
    _check_fwd(case, f, TOL[dtype])
    _check_bwd(case, gla_backward(case, f), TOL[dtype])


def test_fwd_bwd_multi_round_grid():
    # three passes with grids that are no multiple of the 8 XCDs and take several rounds of
    # workgroups (37 images x 6 heads x 4 segments: pass A 666 workgroups forward, 888 for the
    # output pass and both backward passes): the work-item order is a bijection of any grid
    announce("fwd+bwd multi-round grid B=37 L=640 seg=3")
    case = _case("dig_s2_256", batch=37, seq_len=640, random_gamma=True)
    f = gla_forward(case, 64, seg_chunks=3, want_saved=True)
    _check_fwd(case, f, TOL["bf16"])
    g = gla_backward(case, f)
    _check_bwd(case, g, TOL["bf16"])


def test_bwd_determinism():
    announce("bwd determinism")
    case = _case("dig_xl2_2048", batch=1, seq_len=512)
    f = gla_forward(case, 64, seg_chunks=2, want_saved=True)
    g1 = gla_backward(case, f)
    g2 = gla_backward(case, f)
    for n in GRADS + ("dgamma",):
        assert np.array_equal(to_f64(g1[n]), to_f64(g2[n])), n
    # the single-launch short-sequence path as well
    case = _case("dig_s2_256", batch=3, seq_len=200)
    f = gla_forward(case, 64, want_saved=True)
    g1 = gla_backward(case, f)
    g2 = gla_backward(case, f)
    assert np.array_equal(to_f64(g1["dgamma"]), to_f64(g2["dgamma"]))


# Short sequences whose chunks fit one round of workgroups run the backward as one launch:
# a workgroup per chunk, the gradient state from the later chunks through the look-back
# (published per chunk, read through flags tagged per call).
@pytest.mark.parametrize("name,dtype,batch,seq_len,chunk", [
    ("dig_s2_256", "bf16", 8, 256, 64),     # the benchmarked block: 4 chunks, 192 workgroups
    ("dig_s2_256", "bf16", 1, 130, 64),     # 3 chunks, a ragged tail of 2 tokens
    ("dig_s2_256", "bf16", 5, 512, 64),     # 8 chunks, the longest look-back
    ("dig_xl2_2048", "bf16", 1, 450, 64),   # padded head tiles (36, 72), 8 chunks, ragged
    ("dig_xl2_2048", "bf16", 2, 65, 64),    # 2 chunks, the second holds one token
    ("tiny_f32", "bf16", 3, 200, 64),       # (16, 32) heads, four waves
    ("tiny_f32", "bf16", 2, 200, 32),       # (16, 32) heads, 32-token chunks, 7 chunks
])
@pytest.mark.parametrize("dgamma", [True, False])
def test_bwd_lookback_shapes(name, dtype, batch, seq_len, chunk, dgamma):
    announce("bwd lookback %s B=%d L=%d chunk=%d dgamma=%d" % (name, batch, seq_len, chunk, dgamma))
    case = _case(name, batch=batch, seq_len=seq_len, dtype=dtype, random_gamma=True)
    f = gla_forward(case, chunk, want_saved=True)
    g = gla_backward(case, f, dgamma=dgamma)
    _check_bwd(case, g, TOL["bf16"])


def test_bwd_lookback_workspace_reuse():
    """One workspace across calls with other inputs: flags left by an earlier call must not
    be taken for this call's, and a repeated call gives the same bits."""
    announce("bwd lookback workspace reuse")
    a = _case("dig_s2_256", batch=4, seq_len=256, random_gamma=True)
    b = W.make_gla_case(W.CONFIGS["dig_s2_256"], seed=1234, batch=4, seq_len=256,
                        random_gamma=True)
    fa = gla_forward(a, 64, want_saved=True)
    fb = gla_forward(b, 64, want_saved=True)
    ga = gla_backward(a, fa)
    ws = ga["ws"]
    gb = gla_backward(b, fb, ws=ws)
    _check_bwd(b, gb, TOL["bf16"], what="second call")
    ga2 = gla_backward(a, fa, ws=ws)
    _check_bwd(a, ga2, TOL["bf16"], what="third call")
    for n in GRADS + ("dgamma",):
        assert np.array_equal(to_f64(ga[n]), to_f64(ga2[n])), n


def test_fwd_bwd_config_dig_xl2_2048_full():
    announce("fwd+bwd dig_xl2_2048 full B=1 L=16384")
    case = _case("dig_xl2_2048")
    f = gla_forward(case, 64, want_saved=True)
    _check_fwd(case, f, TOL["bf16"], what="xl2_2048")
    g = gla_backward(case, f)
    _check_bwd(case, g, TOL["bf16"], what="xl2_2048")


# Seed sweep of the bf16 backward.  Where the first tokens of a sequence give an o_t that
# cancels to a short vector, rstd_t is large and the RMSNorm gradient magnifies the relative
# error of o_t (saved by the forward) by rstd_t; a dozen seeds per head shape, through the
# single-launch look-back (seg 0) and through three passes (seg 2).
@pytest.mark.parametrize("name,batch,seq_len", [
    ("dig_s2_256", 4, 256),     # DiG-S/2 head shape (6 heads, 32/64)
    ("dig_xl2_2048", 1, 256),   # DiG-XL/2 head shape (16 heads, 36/72)
    ("tiny_f32", 8, 256),       # (16, 32) heads, in bf16
])
@pytest.mark.parametrize("seg", [0, 2])
def test_bwd_seed_sweep(name, batch, seq_len, seg):
    cfg = W.cfg_replace(W.CONFIGS[name], dtype="bf16")
    worst = {}
    for seed in range(100, 112):
        announce("bwd seed sweep %s B=%d L=%d seg=%d seed=%d" % (name, batch, seq_len, seg, seed))
        case = W.make_gla_case(cfg, seed=seed, batch=batch, seq_len=seq_len, random_gamma=True)
        f = gla_forward(case, 64, seg_chunks=seg, want_saved=True)
        _check_fwd(case, f, TOL["bf16"], what="seed %d" % seed)
        errs = _check_bwd(case, gla_backward(case, f), TOL["bf16"], what="seed %d" % seed)
        for n, e in errs.items():
            worst[n] = max(worst.get(n, 0.0), e)
    print("  worst over seeds: " + " ".join("%s=%.2e" % kv for kv in worst.items()), flush=True)


def test_lookback_expired_wait_is_reported():
    """A look-back wait that gives up leaves NaN where the values it waited for would have gone
    and makes dig_lookback_status report DIG_ERR_DEVICE.  Forced from the host: the waits look
    for a flag value no workgroup raises and give up after a few polls, so every kernel still
    ends.  Afterwards normal calls are correct and the status is clean again."""
    import torch
    import diffusion_backbone_amd as dig
    announce("look-back expired wait: forward, then backward")
    case = _case("dig_s2_256", batch=2, seq_len=256, random_gamma=True)   # 4 chunks
    dig.dig_lookback_status()  # nothing pending from earlier tests
    f_ok = gla_forward(case, 64, want_saved=True)
    torch.cuda.synchronize()
    try:
        dig.dig_debug_lookback(8, True)
        f = gla_forward(case, 64, want_saved=False)
        torch.cuda.synchronize()
        with pytest.raises(dig.DigError) as ei:
            dig.dig_lookback_status()
        assert ei.value.status == dig.DIG_ERR_DEVICE
        y = to_f64(f["y"])
        assert np.isfinite(y[:, :64]).all()      # the first chunk waits for nothing
        assert np.isnan(y[:, 64:]).all()         # every later chunk's state never arrived
        g = gla_backward(case, f_ok)
        torch.cuda.synchronize()
        with pytest.raises(dig.DigError):
            dig.dig_lookback_status()
        dk = to_f64(g["dk"])
        assert np.isfinite(dk[:, 192:]).all()    # the last chunk waits for nothing
        assert np.isnan(dk[:, :192]).all()
        assert np.isnan(g["dgamma"].cpu().numpy()).all()
    finally:
        dig.dig_debug_lookback(0, False)
    dig.dig_lookback_status()  # cleared by the query above
    f2 = gla_forward(case, 64, want_saved=True)
    _check_fwd(case, f2, TOL["bf16"], what="after")
    _check_bwd(case, gla_backward(case, f2), TOL["bf16"], what="after")
    dig.dig_lookback_status()
