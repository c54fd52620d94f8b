"""GPU parity of the DiG block forward (slides Figure 4; write-up section 3 "DiG Block")
against the fp64 oracle: the adaptive RMSNorm (dig_rmsnorm_modulate), dig_linear's GELU and
gated-residual epilogues, the conditioning regression (dig_block_cond), one block
(dig_block_fwd) on every scan-direction step, head shapes S and XL, a ragged grid and chunk 16,
and block stacks run free (GPU and oracle each from their own previous block, the block
boundary holding bf16 on both sides).  Normwise max relative error <= 2e-2 per output
(elementwise statistics are logged)."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import TOL, announce, empty, has_gpu, maxrel, nbytes_buf, to_dev, to_f64

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not has_gpu(), reason="needs a GPU")]


def _f32(a):
    import torch
    return None if a is None else torch.from_numpy(np.asarray(a, dtype=np.float32)).cuda()


def _diag(got, ref):
    d = np.abs(got - ref)
    big = np.abs(ref) > 1e-3 * np.max(np.abs(ref))
    ew = float(np.max(d[big] / np.abs(ref[big]))) if np.any(big) else 0.0
    return "ew%.1e" % ew


# ------------------------------------------------------------------ adaptive RMSNorm
@pytest.mark.parametrize("B,L,D", [(2, 37, 384), (3, 8, 1152), (1, 5, 8), (2, 3, 2048),
                                   (3, 100, 1160)])
def test_rmsnorm_modulate_parity(B, L, D):
    import torch
    import diffusion_backbone_amd as dig
    announce("rmsnorm_modulate B=%d L=%d D=%d" % (B, L, D))
    rng = np.random.default_rng(B * 1000 + D)
    x = W.quantize(rng.standard_normal((B, L, D)) * 3.0, "bf16")
    mod = W.quantize(rng.standard_normal((B, 6 * D)), "bf16")
    h = empty((B, L, D), "bf16")
    md = to_dev(mod, "bf16")
    dig.dig_rmsnorm_modulate(B * L, D, L, 1e-5, to_dev(x, "bf16"), md[:, 3 * D:],
                             md[:, 4 * D:], 6 * D, h)
    torch.cuda.synchronize()
    ref = oracle.rmsnorm_modulate(x, mod[:, 3 * D:4 * D], mod[:, 4 * D:5 * D], 1e-5)
    e = maxrel(to_f64(h), ref)
    print("  err %.2e %s" % (e, _diag(to_f64(h), ref)), flush=True)
    assert e <= TOL["bf16"]


# --------------------------------------------------------------- linear epilogues
@pytest.mark.parametrize("m,k,n,rpg,inplace", [(300, 200, 136, 100, False),
                                               (2048, 384, 1536, 256, True),
                                               (33000, 64, 264, 16384, True)])
def test_linear_gelu_and_gated_residual(m, k, n, rpg, inplace):
    import torch
    import diffusion_backbone_amd as dig
    announce("linear epilogues m=%d k=%d n=%d rows_per_gate=%d inplace=%d" % (m, k, n, rpg,
                                                                             inplace))
    rng = np.random.default_rng(m + n)
    a = W.quantize(rng.standard_normal((m, k)), "bf16")
    w = W.quantize(rng.standard_normal((n, k)) / np.sqrt(k), "bf16")
    b = W.f32_round(rng.standard_normal(n) * 0.5)
    res = W.quantize(rng.standard_normal((m, n)), "bf16")
    groups = (m + rpg - 1) // rpg
    gate_ld = n + 8
    gate = W.quantize(rng.standard_normal((groups, gate_ld)), "bf16")
    ad, wd, bd = to_dev(a, "bf16"), to_dev(w, "bf16"), _f32(b)
    c_gelu = empty((m, n), "bf16")
    resd = to_dev(res, "bf16")
    c_res = resd if inplace else empty((m, n), "bf16")
    gd = to_dev(gate, "bf16")
    dig.dig_linear(m, k, ad, [dig.linear_out(c_gelu, wd, bd, act=dig.DIG_ACT_GELU),
                              dig.linear_out(c_res, wd, bd, res=resd, gate=gd, gate_ld=gate_ld,
                                             rows_per_gate=rpg)])
    torch.cuda.synchronize()
    t = oracle.linear(a, w, b)
    ref_gelu = oracle.gelu(t)
    g_rows = gate[np.arange(m) // rpg, :n]
    ref_res = res + g_rows * t
    e1 = maxrel(to_f64(c_gelu), ref_gelu)
    e2 = maxrel(to_f64(c_res), ref_res)
    print("  gelu %.2e %s  gated residual %.2e %s" % (e1, _diag(to_f64(c_gelu), ref_gelu), e2,
                                                      _diag(to_f64(c_res), ref_res)), flush=True)
    assert e1 <= TOL["bf16"] and e2 <= TOL["bf16"], (e1, e2)


def test_linear_residual_alias_rules():
    import torch
    import diffusion_backbone_amd as dig
    a = torch.zeros(64, 8, dtype=torch.bfloat16, device="cuda")
    w = torch.zeros(16, 8, dtype=torch.bfloat16, device="cuda")
    c = torch.zeros(64, 16, dtype=torch.bfloat16, device="cuda")
    g = torch.zeros(1, 16, dtype=torch.bfloat16, device="cuda")
    big = torch.zeros(64 * 16 + 8, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(dig.DigError) as ei:      # residual overlapping c without being c
        dig.dig_linear(64, 8, a, [dig.linear_out(big[:64 * 16].view(64, 16), w,
                                                 res=big[8:].view(64, 16), gate=g, gate_ld=16,
                                                 rows_per_gate=64)])
    assert ei.value.status == dig.DIG_ERR_ALIAS
    with pytest.raises(dig.DigError) as ei:      # gate_ld below n
        dig.dig_linear(64, 8, a, [dig.linear_out(c, w, res=c, gate=g, gate_ld=8,
                                                 rows_per_gate=64)])
    assert ei.value.status == dig.DIG_ERR_SHAPE


# ------------------------------------------------------------------- conditioning
def test_block_cond_parity():
    import torch
    import diffusion_backbone_amd as dig
    cfg = W.CONFIGS["dig_s2_256"]
    announce("block_cond B=%d D=%d blocks=3" % (cfg.batch, cfg.d_model))
    cond = W.make_block_cond(cfg, 3, np.random.default_rng(21))
    mod = empty((cfg.batch, 18 * cfg.d_model), "bf16")
    ws = nbytes_buf(dig.dig_block_cond_workspace_bytes(cfg.batch, cfg.d_model))
    dig.dig_block_cond(cfg.batch, cfg.d_model, 3, to_dev(cond["c"], "bf16"),
                       to_dev(cond["w_ada"], "bf16"), _f32(cond["b_ada"]), mod, ws)
    torch.cuda.synchronize()
    ref = oracle.block_cond(cond["c"], cond["w_ada"], cond["b_ada"])
    e = maxrel(to_f64(mod), ref)
    print("  err %.2e" % e, flush=True)
    assert e <= TOL["bf16"]


# ---------------------------------------------------------------------- one block
def _dev_weights(wts):
    import diffusion_backbone_amd as dig
    dev = {}
    for k, v in wts.items():
        dev[k] = to_dev(v, "bf16") if k.startswith("w_") else _f32(v)
    return dev, dig.make_block_weights(**dev)


def _block_case(cfg, seed, ffn_mult=4):
    rng = np.random.default_rng(seed)
    wts = W.make_dig_block_weights(cfg, rng, ffn_mult)
    cond = W.make_block_cond(cfg, 1, rng)
    mod = W.quantize(oracle.block_cond(cond["c"], cond["w_ada"], cond["b_ada"]), "bf16")
    x = W.quantize(rng.standard_normal((cfg.batch, cfg.seq_len, cfg.d_model)), "bf16")
    return x, mod, wts


def _gpu_block(cfg, desc, wdev, wstruct, x_dev, mod_dev, mod_ld, d, dn, ws):
    import diffusion_backbone_amd as dig
    out = empty(tuple(x_dev.shape), "bf16")
    dig.dig_block_fwd(desc, wstruct, mod_dev, mod_ld, d, dn, x_dev, out, ws)
    return out


def _desc(cfg, ffn_mult=4):
    import diffusion_backbone_amd as dig
    return dig.make_block_desc(cfg.batch, cfg.grid_h, cfg.grid_w, cfg.d_model, cfg.heads,
                               cfg.d_k, cfg.d_v, cfg.rank, ffn_mult * cfg.d_model, cfg.chunk,
                               cfg.tau, 1e-5)


S16 = W.cfg_replace(W.CONFIGS["dig_s2_256"], batch=2)
XL16 = W.cfg_replace(W.CONFIGS["dig_xl2_1024"], batch=1, grid_h=16, grid_w=16)


@pytest.mark.parametrize("cfg,d,dn", [
    (S16, W.ROW, W.ROW_REV), (S16, W.ROW_REV, W.COL), (S16, W.COL, W.COL_REV),
    (S16, W.COL_REV, W.ROW),
    (XL16, W.ROW, W.ROW_REV), (XL16, W.COL, W.COL_REV),
    (W.cfg_replace(S16, grid_h=9, grid_w=7), W.COL, W.COL_REV),       # ragged chunk, odd grid
    (W.cfg_replace(S16, chunk=16, grid_h=12, grid_w=20), W.ROW_REV, W.COL),
    (W.cfg_replace(S16, rank=8), W.ROW, W.COL),   # rank 8: the logits through a projection
], ids=["s_row", "s_rowrev", "s_col", "s_colrev", "xl_row", "xl_col", "s_ragged", "s_chunk16",
        "s_rank8"])
def test_block_fwd_parity(cfg, d, dn):
    import torch
    import diffusion_backbone_amd as dig
    announce("block_fwd %s B=%d %dx%d D=%d H=%d dk=%d dv=%d C=%d %s->%s" % (
        cfg.name, cfg.batch, cfg.grid_h, cfg.grid_w, cfg.d_model, cfg.heads, cfg.d_k, cfg.d_v,
        cfg.chunk, W.SCAN_NAMES[d], W.SCAN_NAMES[dn]))
    x, mod, wts = _block_case(cfg, 31 + d * 4 + dn)
    desc = _desc(cfg)
    wdev, ws_struct = _dev_weights(wts)
    ws = nbytes_buf(dig.dig_block_fwd_workspace_bytes(desc))
    out = _gpu_block(cfg, desc, wdev, ws_struct, to_dev(x, "bf16"), to_dev(mod, "bf16"),
                     6 * cfg.d_model, d, dn, ws)
    torch.cuda.synchronize()
    ref = oracle.block_forward(x, mod, wts, cfg.grid_h, cfg.grid_w, cfg.heads, cfg.d_k, cfg.d_v,
                               d, dn, tau=cfg.tau)
    got = to_f64(out)
    e = maxrel(got, ref)
    print("  err %.2e %s" % (e, _diag(got, ref)), flush=True)
    assert e <= TOL["bf16"]


def test_block_fwd_rejects_bad_arguments():
    import torch
    import diffusion_backbone_amd as dig
    cfg = S16
    desc = _desc(cfg)
    need = dig.dig_block_fwd_workspace_bytes(desc)
    assert need > 0
    x = torch.zeros(cfg.batch, cfg.seq_len, cfg.d_model, dtype=torch.bfloat16, device="cuda")
    mod = torch.zeros(cfg.batch, 6 * cfg.d_model, dtype=torch.bfloat16, device="cuda")
    wkeep, wts = _dev_weights(W.make_dig_block_weights(cfg, np.random.default_rng(1)))
    ws = nbytes_buf(need)
    with pytest.raises(dig.DigError) as ei:             # output aliasing the input
        dig.dig_block_fwd(desc, wts, mod, 6 * cfg.d_model, 0, 1, x, x, ws)
    assert ei.value.status == dig.DIG_ERR_ALIAS
    with pytest.raises(dig.DigError) as ei:             # workspace too small
        dig.dig_block_fwd(desc, wts, mod, 6 * cfg.d_model, 0, 1, x, torch.empty_like(x), ws,
                          workspace_bytes=need - 256)
    assert ei.value.status == dig.DIG_ERR_WORKSPACE
    bad = dig.make_block_desc(cfg.batch, cfg.grid_h, cfg.grid_w, 100, cfg.heads, cfg.d_k, cfg.d_v)
    assert dig.dig_block_fwd_workspace_bytes(bad) == 0   # dim not a multiple of 8


# ------------------------------------------------------------------- block stacks
@pytest.mark.parametrize("cfg,n_blocks", [(S16, 12), (XL16, 4)], ids=["s2_12", "xl2_4"])
def test_block_stack_free_running(cfg, n_blocks):
    """The conditioning regression and n_blocks blocks cycling the four scan directions.  The
    oracle's stack runs free (each block's output held in bf16, the boundary's element type);
    the GPU runs every block on the oracle's input to it (with its own adaLN parameters from
    dig_block_cond), so no oracle input comes from the GPU; the GPU's own free-running stack
    is run beside it and its drift logged."""
    import torch
    import diffusion_backbone_amd as dig
    rng = np.random.default_rng(41 + n_blocks)
    D = cfg.d_model
    blocks = [W.make_dig_block_weights(cfg, rng) for _ in range(n_blocks)]
    cond = W.make_block_cond(cfg, n_blocks, rng)
    x0 = W.quantize(rng.standard_normal((cfg.batch, cfg.seq_len, D)), "bf16")
    desc = _desc(cfg)
    ws = nbytes_buf(max(dig.dig_block_fwd_workspace_bytes(desc),
                        dig.dig_block_cond_workspace_bytes(cfg.batch, D)))
    mod = empty((cfg.batch, n_blocks * 6 * D), "bf16")
    dig.dig_block_cond(cfg.batch, D, n_blocks, to_dev(cond["c"], "bf16"),
                       to_dev(cond["w_ada"], "bf16"), _f32(cond["b_ada"]), mod, ws)
    mod_ref = W.quantize(oracle.block_cond(cond["c"], cond["w_ada"], cond["b_ada"]), "bf16")
    devs = [_dev_weights(b) for b in blocks]
    x_free, x_ref = to_dev(x0, "bf16"), x0
    for l in range(n_blocks):
        d, dn = W.SCHEDULE[l % 4], W.SCHEDULE[(l + 1) % 4]
        announce("stack %s block %d: %s -> %s" % (cfg.name, l, W.SCAN_NAMES[d],
                                                  W.SCAN_NAMES[dn]))
        x_dev = _gpu_block(cfg, desc, devs[l][0], devs[l][1], to_dev(x_ref, "bf16"),
                           mod[:, 6 * D * l:], n_blocks * 6 * D, d, dn, ws)
        x_free = _gpu_block(cfg, desc, devs[l][0], devs[l][1], x_free, mod[:, 6 * D * l:],
                            n_blocks * 6 * D, d, dn, ws)
        torch.cuda.synchronize()
        x_ref = W.quantize(oracle.block_forward(x_ref, mod_ref[:, 6 * D * l:6 * D * (l + 1)],
                                                blocks[l], cfg.grid_h, cfg.grid_w, cfg.heads,
                                                cfg.d_k, cfg.d_v, d, dn, tau=cfg.tau), "bf16")
        got = to_f64(x_dev)
        e = maxrel(got, x_ref)
        print("  block %2d err %.2e %s  GPU's own stack drift %.2e"
              % (l, e, _diag(got, x_ref), maxrel(to_f64(x_free), x_ref)), flush=True)
        assert e <= TOL["bf16"], (l, e)


def test_block_stack_graph_replay():
    """dig_block_cond + four dig_block_fwd calls captured once in a HIP graph and replayed over
    new inputs, with eager work and synchronisation between replays: every replay must give the
    eager calls' bits for the same inputs."""
    import torch
    import diffusion_backbone_amd as dig
    cfg, nb = S16, 4
    D = cfg.d_model
    announce("block stack graph replay, %d blocks" % nb)
    rng = np.random.default_rng(51)
    devs = [_dev_weights(W.make_dig_block_weights(cfg, rng)) for _ in range(nb)]
    cond = W.make_block_cond(cfg, nb, rng)
    c = to_dev(cond["c"], "bf16")
    w_ada, b_ada = to_dev(cond["w_ada"], "bf16"), _f32(cond["b_ada"])
    desc = _desc(cfg)
    ws = nbytes_buf(max(dig.dig_block_fwd_workspace_bytes(desc),
                        dig.dig_block_cond_workspace_bytes(cfg.batch, D)))
    mod = torch.empty(cfg.batch, nb * 6 * D, dtype=torch.bfloat16, device="cuda")
    x0 = torch.empty(cfg.batch, cfg.seq_len, D, dtype=torch.bfloat16, device="cuda")
    bufs = [torch.empty_like(x0) for _ in range(2)]

    def forward():
        dig.dig_block_cond(cfg.batch, D, nb, c, w_ada, b_ada, mod, ws)
        src = x0
        for l in range(nb):
            dst = bufs[l % 2]
            dig.dig_block_fwd(desc, devs[l][1], mod[:, 6 * D * l:], nb * 6 * D, W.SCHEDULE[l % 4],
                              W.SCHEDULE[(l + 1) % 4], src, dst, ws)
            src = dst
        return src

    x0.copy_(to_dev(W.quantize(rng.standard_normal(tuple(x0.shape)), "bf16"), "bf16"))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        forward()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = forward()
    torch.cuda.synchronize()
    for i in range(3):
        x0.copy_(to_dev(W.quantize(rng.standard_normal(tuple(x0.shape)), "bf16"), "bf16"))
        c.copy_(to_dev(W.quantize(rng.standard_normal(tuple(c.shape)), "bf16"), "bf16"))
        want = to_f64(forward())
        torch.cuda.synchronize()
        for b in bufs:
            b.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_f64(out), want), "replay %d differs from the eager calls" % i


def test_block_fwd_full_xl2_2048():
    """One DiG-XL/2 block at the full 2048-px size (128 x 128 tokens, the launch configuration
    the bench times), every output element against the oracle."""
    import torch
    import diffusion_backbone_amd as dig
    cfg = W.CONFIGS["dig_xl2_2048"]
    announce("block_fwd full dig_xl2_2048 col -> col_rev")
    x, mod, wts = _block_case(cfg, 61)
    desc = _desc(cfg)
    wdev, ws_struct = _dev_weights(wts)   # wdev keeps the weights alive
    ws = nbytes_buf(dig.dig_block_fwd_workspace_bytes(desc))
    out = _gpu_block(cfg, desc, wdev, ws_struct, to_dev(x, "bf16"), to_dev(mod, "bf16"),
                     6 * cfg.d_model, W.COL, W.COL_REV, ws)
    torch.cuda.synchronize()
    got = to_f64(out)
    announce("  oracle (fp64, about 20 s)")
    ref = oracle.block_forward(x, mod, wts, cfg.grid_h, cfg.grid_w, cfg.heads, cfg.d_k, cfg.d_v,
                               W.COL, W.COL_REV, tau=cfg.tau)
    e = maxrel(got, ref)
    print("  err %.2e %s" % (e, _diag(got, ref)), flush=True)
    assert e <= TOL["bf16"]
