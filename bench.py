#!/usr/bin/env python3
"""Throughput of the DiG hot path on one MI355X: GLA token mixer + SREM, forward and backward.

Headline (``value``): the DiG-XL/2 2048-px training step (batch 1, 128 x 128 tokens, 16 heads,
d_k 36, d_v 72, chunk 64).  One step = four blocks in the four scan directions (row, row_rev,
col, col_rev), each ``dig_gla_fwd`` (saving what the backward needs) -> ``dig_dwconv3x3``
(fused reorient to the next direction), then, blocks in reverse, ``dig_dwconv3x3_bwd`` ->
``dig_gla_bwd``.  Inputs are generated on the GPU before timing (seeded; x ~ N(0,1), weights
~ N(0, 1/D), upstream gradients ~ N(0,1)) and are resident in HBM.  The metric is GLA-layer
tokens/s: batch * tokens * blocks / step time.

Beside it, in the same JSON line: the other configurations (DiG-S/2 256 px, 12 blocks,
forward and forward+backward; S/2 1792 px; XL/2 1024 px over the four directions), the
roofline of the dominant call, an LDS-resident contraction microbenchmark (MFMA fraction of
the contraction phases), steady-state and cold-cache probes against a measured streaming-copy
ceiling, and the fp64 oracle timed on the host (single thread and all cores).

Prints ONE JSON line.  --gpus N with N > 1 exits: the library measures one GPU.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix peak
HEADLINE = "dig_xl2_2048"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=HEADLINE, choices=sorted(W.CONFIGS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probes", action="store_true",
                    help="skip everything outside the headline step (other configs, probes, "
                         "microbenchmark)")
    ap.add_argument("--seg-chunks", type=int, default=0)
    # profiling helpers (rocprofv3 counter runs): run only one library call of the step, or a
    # plain device copy of known size that calibrates the byte counters
    ap.add_argument("--pmc-target", choices=["gla_fwd", "gla_bwd", "srem_fwd", "srem_bwd"],
                    default=None)
    ap.add_argument("--copy-probe-mib", type=int, default=0)
    ap.add_argument("--copy-probe-width", type=int, default=16, choices=[4, 8, 16])
    ap.add_argument("--value-gate", action="store_true",
                    help="time only the value-gate calls (dig_gla_*_beta) at --workload")
    ap.add_argument("--stack", default=None,
                    choices=["dig_s2_256_stack", "dig_xl2_256_stack", "dig_xl2_2048_stack"],
                    help="time only this DiG block stack forward (for kernel traces)")
    ap.add_argument("--oracle-leg", default=None, help=argparse.SUPPRESS)  # child process
    return ap.parse_args()


def n_blocks(cfg):
    """Blocks per step: the configuration's own count (12 for DiG-S/2 256 px), else one block
    per scan direction."""
    return cfg.blocks if cfg.blocks > 1 else 4


def gen_blocks(cfg, nblocks, seed):
    """Per-block bf16 operands on the GPU: projections of x ~ N(0,1) by weights ~ N(0,1/D)."""
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    B, L, D, H, dk, dv = cfg.batch, cfg.seq_len, cfg.d_model, cfg.heads, cfg.d_k, cfg.d_v
    s = 1.0 / np.sqrt(D)
    blocks = []
    for _ in range(nblocks):
        x = torch.randn(B * L, D, device="cuda", generator=g)
        w = lambda n, m: torch.randn(n, m, device="cuda", generator=g) * s
        q = (x @ w(D, H * dk)).view(B, L, H, dk)
        k = (x @ w(D, H * dk)).view(B, L, H, dk)
        v = (x @ w(D, H * dv)).view(B, L, H, dv)
        u = x @ w(D, cfg.rank)          # the low-rank gate's factor x W_a1
        wa2 = w(cfg.rank, H * dk)
        z = (u @ wa2).view(B, L, H, dk)
        r = (x @ w(D, H * dv)).view(B, L, H, dv)
        cw = torch.randn(D, 3, 3, device="cuda", generator=g) / 3.0
        dy = torch.randn(B, L, H, dv, device="cuda", generator=g)
        dys = torch.randn(B, L, D, device="cuda", generator=g)
        bf = lambda t: t.to(torch.bfloat16).contiguous()
        blocks.append(dict(q=bf(q), k=bf(k), v=bf(v), z=bf(z), r=bf(r), x=bf(x.view(B, L, D)),
                           cw=cw.contiguous(), dy=bf(dy), dys=bf(dys),
                           gamma=torch.ones(dv, device="cuda"), u=bf(u.view(B, L, cfg.rank)),
                           wa2=bf(wa2.t()), ba=torch.zeros(H * dk, device="cuda")))
        del x, q, k, v, z, r, dy, dys, u
    return blocks


class Path:
    """Buffers and the library calls of one step."""

    def __init__(self, cfg, blocks, seg_chunks, lowrank=False):
        import torch
        import diffusion_backbone_amd as dig
        self.dig, self.cfg, self.blocks = dig, cfg, blocks
        self.lowrank = lowrank  # the gate formed in the chunk kernels from x W_a1 and W_a2
        B, L, H, dk, dv, D = cfg.batch, cfg.seq_len, cfg.heads, cfg.d_k, cfg.d_v, cfg.d_model
        self.desc = dig.make_desc(B, L, H, dk, dv, cfg.chunk, cfg.tau, 1.0, 1e-5, dig.DIG_BF16,
                                  seg_chunks)
        bt = lambda *s: torch.empty(*s, dtype=torch.bfloat16, device="cuda")
        by = lambda n: torch.empty(max(int(n), 16), dtype=torch.uint8, device="cuda")
        self.fws_b = dig.dig_gla_fwd_workspace_bytes(self.desc)
        self.bws_b = dig.dig_gla_bwd_workspace_bytes(self.desc)
        self.cws_b = dig.dig_dwconv3x3_bwd_workspace_bytes(B, cfg.grid_h, cfg.grid_w, D)
        self.fws, self.bws, self.cws = by(self.fws_b), by(self.bws_b), by(self.cws_b)
        n = len(blocks)
        self.saved = [by(dig.dig_gla_saved_bytes(self.desc)) for _ in range(n)]
        self.y = [bt(B, L, H, dv) for _ in range(n)]
        self.xs = [bt(B, L, D) for _ in range(n)]
        self.g = {k: bt(B, L, H, dk) for k in ("dq", "dk", "dz")}
        self.g.update({k: bt(B, L, H, dv) for k in ("dv", "dr")})
        self.dgamma = torch.empty(dv, device="cuda")
        self.dxs = bt(B, L, D)
        self.dw = torch.empty(D, 3, 3, device="cuda")
        self.db = torch.empty(D, device="cuda")
        self.sched = [W.SCHEDULE[l % 4] for l in range(n + 1)]

    def gla_fwd(self, l):
        b = self.blocks[l]
        if self.lowrank:
            self.dig.dig_gla_fwd_lowrank(self.desc, b["q"], b["k"], b["v"], b["u"], b["wa2"],
                                         b["ba"], b["r"], b["gamma"], self.y[l], None,
                                         self.saved[l], self.fws, self.fws_b)
            return
        self.dig.dig_gla_fwd(self.desc, b["q"], b["k"], b["v"], b["z"], b["r"], b["gamma"],
                             self.y[l], None, self.saved[l], self.fws, self.fws_b)

    def srem_fwd(self, l):
        c, b = self.cfg, self.blocks[l]
        self.dig.dig_dwconv3x3(c.batch, c.grid_h, c.grid_w, c.d_model, self.dig.DIG_BF16,
                               self.sched[l], self.sched[l + 1], b["x"], b["cw"], None, self.xs[l])

    def srem_bwd(self, l):
        c, b = self.cfg, self.blocks[l]
        self.dig.dig_dwconv3x3_bwd(c.batch, c.grid_h, c.grid_w, c.d_model, self.dig.DIG_BF16,
                                   self.sched[l], self.sched[l + 1], b["x"], b["cw"], b["dys"],
                                   self.dxs, self.dw, self.db, self.cws, self.cws_b)

    def gla_bwd(self, l):
        b, g = self.blocks[l], self.g
        if self.lowrank:
            self.dig.dig_gla_bwd_lowrank(self.desc, b["q"], b["k"], b["v"], b["u"], b["wa2"],
                                         b["ba"], b["r"], b["gamma"], b["dy"], self.saved[l],
                                         g["dq"], g["dk"], g["dv"], g["dz"], g["dr"], self.dgamma,
                                         self.bws, self.bws_b)
            return
        self.dig.dig_gla_bwd(self.desc, b["q"], b["k"], b["v"], b["z"], b["r"], b["gamma"],
                             b["dy"], self.saved[l], g["dq"], g["dk"], g["dv"], g["dz"], g["dr"],
                             self.dgamma, self.bws, self.bws_b)

    def step(self, ev=None):
        n = len(self.blocks)
        for l in range(n):
            if ev is not None:
                ev.record_pair("gla_fwd", lambda: self.gla_fwd(l))
            else:
                self.gla_fwd(l)
            self.srem_fwd(l)
        for l in reversed(range(n)):
            self.srem_bwd(l)
            if ev is not None:
                ev.record_pair("gla_bwd", lambda: self.gla_bwd(l))
            else:
                self.gla_bwd(l)

    def step_fwd(self):
        for l in range(len(self.blocks)):
            self.gla_fwd(l)
            self.srem_fwd(l)


class EventTimer:
    """HIP events around chosen calls on torch's current stream (the stream the library calls
    run on).  Created up front so that recording them adds no allocation to the timed region."""

    def __init__(self, n):
        import torch
        self.free = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                     for _ in range(n)]
        self.pairs = {}

    def record_pair(self, name, fn):
        a, b = self.free.pop()
        a.record()
        fn()
        b.record()
        self.pairs.setdefault(name, []).append((a, b))

    def avg_ms(self, name):
        ps = self.pairs.get(name, [])
        return sum(a.elapsed_time(b) for a, b in ps) / max(len(ps), 1)


def timed_graph(fn, steps, reps=10):
    """ms per call of fn with the host out of the way: `reps` calls captured once in a HIP
    graph, the graph replayed `steps` times (one warm-up replay)."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(reps):
            fn()
    ms = timed(graph.replay, steps, 1) / reps
    del graph
    return ms


def timed(fn, steps, warmup):
    """ms per call of fn over exactly `steps` calls after `warmup` untimed ones, with a device
    synchronisation on both sides of the timed region."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


# HBM traffic of one GLA call on the headline workload, from rocprofv3 FETCH_SIZE and
# WRITE_SIZE runs (summed over the call's kernels) divided by the counters' reading per byte
# of a plain copy; valid only for the kernel sources it was measured on (sha256 below).
TRAFFIC = {
    "workload": "dig_xl2_2048",
    "bytes": {
        # pass A 115319.7 KiB / 0.500076 + 91413.1 KiB / 1.0, segment scan 1695.6 + 2594.2,
        # final pass 95167.8 + 92273.1 (FETCH_SIZE, WRITE_SIZE; copy: 131091.8 KiB read per
        # 262144 KiB moved, 262144 KiB written per 262144 KiB moved)
        "dig_gla_bwd": 625236564,
        # pass A 36420.3 + 5093.8, state scan 2864.6 + 5184.0, output pass 68264.5 + 157063.7
        "dig_gla_fwd": 391585479,
    },
    "sources_sha256": "cd034969375aacdffccbc2e98c79b112e10608749f42542ca169771c4c8f2843",
}
TRAFFIC_SOURCES = ("diffusion_backbone_amd/csrc/gla_bwd_kernel.h",
                   "diffusion_backbone_amd/csrc/gla_bwd.hip",
                   "diffusion_backbone_amd/csrc/gla_fwd_kernel.h",
                   "diffusion_backbone_amd/csrc/gla_fwd.hip",
                   "diffusion_backbone_amd/csrc/dig_device.h")


def sources_sha256():
    import hashlib
    h = hashlib.sha256()
    for rel in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload, call):
    """Counter-derived bytes per call, or None when the kernels changed since the run."""
    byts = TRAFFIC["bytes"].get(call)
    if byts is None or workload != TRAFFIC["workload"]:
        return None
    return byts if TRAFFIC["sources_sha256"] == sources_sha256() else None


def probe_lib():
    """libdig_probe.so: measurement kernels (contraction microbenchmark, streaming copy)."""
    import ctypes
    path = os.path.join(ROOT, "diffusion_backbone_amd", "libdig_probe.so")
    if not os.path.exists(path):
        raise RuntimeError("libdig_probe.so is not built (run __graft_entry__.build())")
    L = ctypes.CDLL(path)
    P, I = ctypes.c_void_p, ctypes.c_int
    L.digp_contraction.argtypes = [I, I, I, P, P]
    L.digp_contraction.restype = I
    L.digp_contraction_waves.argtypes = [I]
    L.digp_contraction_waves.restype = I
    L.digp_contraction_flops.argtypes = [I, ctypes.POINTER(ctypes.c_double),
                                         ctypes.POINTER(ctypes.c_double)]
    L.digp_copy.argtypes = [P, P, ctypes.c_size_t, P]
    L.digp_copy.restype = I
    L.digp_copy_w.argtypes = [P, P, ctypes.c_size_t, I, P]
    L.digp_copy_w.restype = I
    L.digp_mfma_rate.argtypes = [I, I, I, P, P]
    L.digp_mfma_rate.restype = I
    L.digp_mfma_rate_flops.argtypes = [I, I, I]
    L.digp_mfma_rate_flops.restype = ctypes.c_double
    return L


def _stream():
    import torch
    return torch.cuda.current_stream().cuda_stream


def device_copy(L, src, dst):
    err = L.digp_copy(src.data_ptr(), dst.data_ptr(), src.numel() * src.element_size(), _stream())
    if err:
        raise RuntimeError("digp_copy failed: %d" % err)


def copy_probe(mib, reps, width=16):
    """A plain streaming copy of known size with `width`-byte lanes: the reference for scaling
    FETCH_SIZE / WRITE_SIZE counter readings to bytes."""
    import torch
    L = probe_lib()
    x = torch.ones(mib * 1024 * 1024 // 2, dtype=torch.bfloat16, device="cuda")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(reps):
        err = L.digp_copy_w(x.data_ptr(), y.data_ptr(), x.numel() * 2, width, _stream())
        if err:
            raise RuntimeError("digp_copy_w failed: %d" % err)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_each_way": x.numel() * 2, "reps": reps,
                      "lane_bytes": width}), flush=True)


def gla_bytes_per_token_head(cfg, which):
    """Algorithmic HBM bytes per (token, head) of one mixer call (bf16 I/O)."""
    dk, dv = cfg.d_k, cfg.d_v
    if which == "fwd":   # read q, k, z, v, r; write y
        return 2 * (3 * dk + 3 * dv)
    # bwd: read q, k, z, v, r, dy; write dq, dk, dz, dv, dr
    return 2 * (6 * dk + 5 * dv)


def srem_bytes_per_token(cfg, which):
    """Algorithmic bytes per token of the conv with fused reorient: read x, write y (fwd); read
    x and dy, write dx (bwd)."""
    return (2 if which == "fwd" else 3) * cfg.d_model * 2


def run_config(cfg, steps, warmup, seg_chunks=0, fwd_only=False, events=False, lowrank=False):
    """Times the step of one configuration; returns a dict (and the Path when events=True).
    lowrank: the mixer calls take the gate as x W_a1 and W_a2 (dig_gla_*_lowrank)."""
    import torch
    nb = n_blocks(cfg)
    blocks = gen_blocks(cfg, nb, cfg.seed)
    path = Path(cfg, blocks, seg_chunks, lowrank)
    torch.cuda.synchronize()
    tokens = cfg.batch * cfg.seq_len * nb
    out = {"workload": cfg.name, "batch": cfg.batch, "grid": [cfg.grid_h, cfg.grid_w],
           "heads": cfg.heads, "d_k": cfg.d_k, "d_v": cfg.d_v, "d_model": cfg.d_model,
           "chunk": cfg.chunk, "blocks": nb,
           "directions": [W.SCAN_NAMES[d] for d in path.sched[:nb]]}
    ms_fwd = timed(path.step_fwd, steps, warmup)
    out["fwd"] = {"tokens_per_s": round(tokens / (ms_fwd / 1e3), 1), "ms_per_step": round(ms_fwd, 4)}
    # the same step captured once in a HIP graph and replayed: the GPU's own time where the
    # host's launches (tens of calls of a few us each) would otherwise set the pace
    ms_g = timed_graph(path.step_fwd, steps, reps=1)
    out["fwd"]["graph_replay"] = {"tokens_per_s": round(tokens / (ms_g / 1e3), 1),
                                  "ms_per_step": round(ms_g, 4)}
    if not fwd_only:
        ms = timed(path.step, steps, warmup)
        out["fwd_bwd"] = {"tokens_per_s": round(tokens / (ms / 1e3), 1), "ms_per_step": round(ms, 4)}
        ms_g = timed_graph(path.step, steps, reps=1)
        out["fwd_bwd"]["graph_replay"] = {"tokens_per_s": round(tokens / (ms_g / 1e3), 1),
                                          "ms_per_step": round(ms_g, 4)}
    if not events:
        del path, blocks
        torch.cuda.empty_cache()
        return out, None
    return out, path


def lowrank_gate(cfg, steps):
    """The headline step with the key gate given as x W_a1 (16 per token) and W_a2, the logits
    formed inside the chunk kernels (dig_gla_fwd_lowrank / dig_gla_bwd_lowrank), and one
    block's calls of both gate forms timed back to back."""
    import torch
    res, path = run_config(cfg, steps, 3, events=True, lowrank=True)
    calls = {}
    for lr in (False, True):
        path.lowrank = lr
        key = "lowrank" if lr else "logits"
        calls[key] = {"gla_fwd_us": round(_time_us(lambda: path.gla_fwd(0), reps=20), 2),
                      "gla_bwd_us": round(_time_us(lambda: path.gla_bwd(0), reps=20), 2)}
    res["calls"] = calls
    res["gate_bytes_per_token"] = {"logits": 2 * cfg.heads * cfg.d_k, "lowrank": 2 * cfg.rank}
    del path
    torch.cuda.empty_cache()
    return res


def value_gate(cfg):
    """The mixer with the general gate of eq. (5), G_t = alpha_t^T beta_t (dig_gla_fwd_beta /
    dig_gla_bwd_beta), at the headline shape: one block's calls, timed per call (HIP events on
    the stream), against the bytes their bf16 inputs and outputs must move."""
    import torch
    import diffusion_backbone_amd as dig
    B, L, H, dk, dv = cfg.batch, cfg.seq_len, cfg.heads, cfg.d_k, cfg.d_v
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    bf = lambda d, s=1.0: (torch.randn(B, L, H, d, device="cuda", generator=g) * s).to(torch.bfloat16)
    q, k, z, v, w, r, dy = bf(dk, 0.5), bf(dk, 0.5), bf(dk), bf(dv), bf(dv), bf(dv), bf(dv)
    nw = torch.ones(dv, device="cuda")
    desc = dig.make_desc(B, L, H, dk, dv, 64, 16.0, 1.0, 1e-5, "bf16", 0)
    saved = torch.empty(dig.dig_gla_beta_saved_bytes(desc), dtype=torch.uint8, device="cuda")
    fwb, bwb = dig.dig_gla_beta_fwd_workspace_bytes(desc), dig.dig_gla_beta_bwd_workspace_bytes(desc)
    fws = torch.empty(fwb, dtype=torch.uint8, device="cuda")
    bws = torch.empty(bwb, dtype=torch.uint8, device="cuda")
    y = torch.empty_like(r)
    grads = [torch.empty_like(t) for t in (q, k, v, z, w, r)]
    dnw = torch.empty(dv, device="cuda")
    fwd = lambda: dig.dig_gla_fwd_beta(desc, q, k, v, z, w, r, nw, y, None, saved, fws, fwb)
    bwd = lambda: dig.dig_gla_bwd_beta(desc, q, k, v, z, w, r, nw, dy, saved, grads[0], grads[1],
                                       grads[2], grads[3], grads[4], grads[5], dnw, bws, bwb)
    fwd()
    fu, bu = _time_us(fwd, reps=20), _time_us(bwd, reps=20)
    tok = B * L * H
    fb, bb = 2 * (3 * dk + 4 * dv) * tok, 2 * (6 * dk + 7 * dv) * tok
    res = {"shape": {"batch": B, "seq_len": L, "heads": H, "d_k": dk, "d_v": dv, "chunk": 64},
           "gla_fwd_beta_us": round(fu, 2), "gla_bwd_beta_us": round(bu, 2),
           "fwd_algorithmic_bytes": fb, "bwd_algorithmic_bytes": bb,
           "fwd_frac_of_hbm_peak": round(fb / (fu * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
           "bwd_frac_of_hbm_peak": round(bb / (bu * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
           "layer_tokens_per_s_fwd_bwd": round(B * L / ((fu + bu) * 1e-6), 1)}
    del saved, fws, bws
    torch.cuda.empty_cache()
    return res


def contraction_microbench():
    """The chunk kernel's contraction phases with operands resident in LDS (no global
    traffic): how busy they can keep the matrix cores.  A microbenchmark, not the step."""
    import ctypes
    import torch
    L = probe_lib()
    res = {}
    for shape, label in ((0, "s_heads_32_64"), (1, "xl_heads_36_72")):
        nwg, iters = 256 * 4, 400
        waves = L.digp_contraction_waves(shape)
        sink = torch.empty(nwg * 64 * waves, device="cuda")
        run = lambda: L.digp_contraction(shape, nwg, iters, sink.data_ptr(), _stream())
        ms = timed(run, 5, 2)
        alg, iss = ctypes.c_double(), ctypes.c_double()
        L.digp_contraction_flops(shape, ctypes.byref(alg), ctypes.byref(iss))
        chunks = nwg * iters
        t_alg = alg.value * chunks / (ms / 1e3) / 1e12
        t_iss = iss.value * chunks / (ms / 1e3) / 1e12
        res[label] = {
            "what": "gated Q K^T (split hi/lo), P V, (q e^b) S0 and the state update of one "
                    "64-token chunk per workgroup iteration, operands in LDS; %d workgroups x "
                    "%d iterations" % (nwg, iters),
            "ms": round(ms, 4),
            "mfma_issued_tflops": round(t_iss, 1),
            "mfma_frac_of_bf16_peak": round(t_iss / BF16_PEAK_TFLOPS, 4),
            "algorithmic_tflops": round(t_alg, 1),
            "algorithmic_frac_of_bf16_peak": round(t_alg / BF16_PEAK_TFLOPS, 4),
            "issued_flops_per_chunk": iss.value, "algorithmic_flops_per_chunk": alg.value}
        del sink
    # the instructions' own ceilings: operands and accumulators in registers, no memory
    nwg, iters = 2048, 1000
    sink = torch.empty(nwg * 256, device="cuda")
    for wide, label in ((0, "mfma_16x16x32_bf16"), (1, "mfma_32x32x16_bf16")):
        ms = timed(lambda: L.digp_mfma_rate(wide, nwg, iters, sink.data_ptr(), _stream()), 3, 1)
        tf = L.digp_mfma_rate_flops(wide, nwg, iters) / (ms / 1e3) / 1e12
        res["register_only_" + label] = {"tflops": round(tf, 1),
                                         "frac_of_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4)}
    res["note"] = ("the contraction phases use the 16x16x32 instruction; its register-only rate "
                   "is the ceiling for them on this part")
    return res


def projections(cfg, steps):
    """The projections around the mixer (dig_linear, bf16 matrix cores) at one configuration's
    size, timed alone (MFMA-bound: flops against the 2.5 PFLOP/s bf16 peak), and one layer's
    forward with them: x -> q, k, v, rank-16 gate factor, r (one launch) -> gate logits
    (rank 16 -> H d_k, + bias) -> dig_gla_fwd -> output projection -> dig_dwconv3x3 (fused
    reorient).  Random-init weights of the layer's shapes."""
    import torch
    import diffusion_backbone_amd as dig
    B, L, D, H, dk, dv = cfg.batch, cfg.seq_len, cfg.d_model, cfg.heads, cfg.d_k, cfg.d_v
    M = B * L
    g = torch.Generator(device="cuda")
    g.manual_seed(cfg.seed + 5)
    bf = lambda *sh, s=1.0: (torch.randn(*sh, device="cuda", generator=g) * s).to(torch.bfloat16)
    x = bf(B, L, D)
    s = 1.0 / np.sqrt(D)
    wq, wk, wv, wr = bf(H * dk, D, s=s), bf(H * dk, D, s=s), bf(H * dv, D, s=s), bf(H * dv, D, s=s)
    wa1, wa2 = bf(cfg.rank, D, s=s), bf(H * dk, cfg.rank, s=s)
    wo = bf(D, H * dv, s=s)
    b_alpha = torch.zeros(H * dk, device="cuda")
    q, k, z = bf(B, L, H, dk), bf(B, L, H, dk), bf(B, L, H, dk)
    v, r, y = bf(B, L, H, dv), bf(B, L, H, dv), bf(B, L, H, dv)
    zl = bf(B, L, cfg.rank)
    yo, xs = bf(B, L, D), bf(B, L, D)
    cw = torch.randn(D, 3, 3, device="cuda", generator=g) / 3.0
    gamma = torch.ones(dv, device="cuda")
    desc = dig.make_desc(B, L, H, dk, dv, cfg.chunk, cfg.tau, 1.0, 1e-5, dig.DIG_BF16, 0)
    fwb = dig.dig_gla_fwd_workspace_bytes(desc)
    fws = torch.empty(max(fwb, 16), dtype=torch.uint8, device="cuda")
    proj_in = lambda: dig.dig_linear(M, D, x, [(q, wq, None), (k, wk, None), (v, wv, None),
                                               (zl, wa1, None), (r, wr, None)])
    gate_up = lambda: dig.dig_linear(M, cfg.rank, zl, [(z, wa2, b_alpha)])
    proj_out = lambda: dig.dig_linear(M, H * dv, y, [(yo, wo, None)])
    n_in = 2 * H * dk + 2 * H * dv + cfg.rank
    # the same products through torch's library GEMM (hipBLASLt), as a reference point only
    w_cat = torch.cat([wq, wk, wv, wa1, wr], dim=0).contiguous()
    x2, y2 = x.view(M, D), y.view(M, H * dv)
    lib_in = lambda: torch.nn.functional.linear(x2, w_cat)
    lib_out = lambda: torch.nn.functional.linear(y2, wo)
    res = {}
    for name, fn, flops, ref in (("in_projection", proj_in, 2.0 * M * D * n_in, lib_in),
                                 ("gate_up_projection", gate_up, 2.0 * M * cfg.rank * H * dk, None),
                                 ("out_projection", proj_out, 2.0 * M * H * dv * D, lib_out)):
        ms = timed(fn, steps, 3)
        tf = flops / (ms / 1e3) / 1e12
        res[name] = {"us": round(ms * 1e3, 1), "tflops": round(tf, 1),
                     "frac_of_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4), "flops": flops}
        if ref is not None:
            ms_ref = timed(ref, steps, 3)
            res[name]["torch_linear_reference_us"] = round(ms_ref * 1e3, 1)
            res[name]["torch_linear_reference_tflops"] = round(flops / (ms_ref / 1e3) / 1e12, 1)

    def layer():
        proj_in()
        gate_up()
        dig.dig_gla_fwd(desc, q, k, v, z, r, gamma, y, None, None, fws, fwb)
        proj_out()
        dig.dig_dwconv3x3(B, cfg.grid_h, cfg.grid_w, D, dig.DIG_BF16, W.ROW, W.ROW_REV, yo, cw,
                          None, xs)
    def layer_lowrank():
        proj_in()
        dig.dig_gla_fwd_lowrank(desc, q, k, v, zl, wa2, b_alpha, r, gamma, y, None, None, fws, fwb)
        proj_out()
        dig.dig_dwconv3x3(B, cfg.grid_h, cfg.grid_w, D, dig.DIG_BF16, W.ROW, W.ROW_REV, yo, cw,
                          None, xs)
    ms = timed(layer, steps, 3)
    res["layer_fwd_with_projections"] = {
        "what": "in-projection, gate up-projection, dig_gla_fwd, out-projection, dig_dwconv3x3 "
                "(fused reorient), one block", "ms": round(ms, 4),
        "tokens_per_s": round(M / (ms / 1e3), 1)}
    ms = timed(layer_lowrank, steps, 3)
    res["layer_fwd_with_projections_lowrank_gate"] = {
        "what": "in-projection, dig_gla_fwd_lowrank (gate logits formed in the chunk kernels), "
                "out-projection, dig_dwconv3x3 (fused reorient), one block", "ms": round(ms, 4),
        "tokens_per_s": round(M / (ms / 1e3), 1)}
    res["workload"] = cfg.name
    return res


def block_stack(name, steps, warmup=2):
    """The DiG block stack forward (slides Figure 4, Table 1): the conditioning regression of
    every block (dig_block_cond), then n blocks of dig_block_fwd cycling the four scan
    directions, on random-init weights of the model's shapes (projections ~ N(0, 1/fan_in),
    DWConv identity + noise, adaLN gamma ~ 1, alpha ~ 0.5) and x ~ N(0, 1).  Reported: images/s
    and tokens/s of the whole forward, the dense-matmul share against the bf16 peak, and one
    block's steps timed one by one through the public calls the block composes (each replayed
    from a captured graph, so the host's launch cost does not hide the small kernels)."""
    import torch
    import diffusion_backbone_amd as dig
    if name in W.STACKS:
        cfg, nb = W.STACKS[name]
    else:  # the headline image size with the XL/2 stack
        cfg, nb = W.CONFIGS["dig_xl2_2048"], 28
    B, L, D, H, dk, dv, R = cfg.batch, cfg.seq_len, cfg.d_model, cfg.heads, cfg.d_k, cfg.d_v, cfg.rank
    F, M = 4 * D, cfg.batch * cfg.seq_len
    HK, HV = H * dk, H * dv
    nin = 2 * HK + 2 * HV + R
    g = torch.Generator(device="cuda")
    g.manual_seed(cfg.seed + 9)
    bf = lambda *sh, s=1.0: (torch.randn(*sh, device="cuda", generator=g) * s).to(torch.bfloat16)
    f32 = lambda n, s=0.1: torch.randn(n, device="cuda", generator=g) * s
    keep, structs = [], []
    for _ in range(nb):
        cw = torch.randn(D, 3, 3, device="cuda", generator=g) / 6.0
        cw[:, 1, 1] += 1.0
        t = dict(w_in=bf(nin, D, s=D ** -0.5), b_in=f32(nin), w_gate=bf(HK, R, s=R ** -0.5),
                 b_gate=f32(HK, 1.0), gla_norm_w=1.0 + f32(dv), w_out=bf(D, HV, s=HV ** -0.5),
                 b_out=f32(D), w_ffn1=bf(F, D, s=D ** -0.5), b_ffn1=f32(F),
                 w_ffn2=bf(D, F, s=F ** -0.5), b_ffn2=f32(D), conv_w=cw, conv_b=f32(D))
        keep.append(t)
        structs.append(dig.make_block_weights(**t))
    part = torch.cat([torch.full((D,), v, device="cuda") for v in (1.0, 0.0, 0.5, 1.0, 0.0, 0.5)])
    c = bf(B, D)
    w_ada = bf(nb * 6 * D, D, s=0.1 * D ** -0.5)
    b_ada = part.repeat(nb).contiguous()
    mod = torch.empty(B, nb * 6 * D, dtype=torch.bfloat16, device="cuda")
    desc = dig.make_block_desc(B, cfg.grid_h, cfg.grid_w, D, H, dk, dv, R, F, cfg.chunk, cfg.tau)
    wsb = max(dig.dig_block_fwd_workspace_bytes(desc), dig.dig_block_cond_workspace_bytes(B, D))
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    x0 = bf(B, L, D)
    xa, xb = torch.empty_like(x0), torch.empty_like(x0)
    mld = nb * 6 * D

    def forward():
        dig.dig_block_cond(B, D, nb, c, w_ada, b_ada, mod, ws)
        src, dst = x0, xa
        for l in range(nb):
            d, dn = W.SCHEDULE[l % 4], W.SCHEDULE[(l + 1) % 4]
            dig.dig_block_fwd(desc, structs[l], mod[:, 6 * D * l:], mld, d, dn, src, dst, ws)
            src, dst = dst, (xb if dst is xa else xa)
    ms = timed(forward, steps, warmup)
    # the same forward captured once in a HIP graph and replayed (no host launch overhead)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        forward()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        forward()
    ms_graph = timed(graph.replay, steps, warmup)
    del graph
    fused = R == dig.DIG_GATE_RANK  # dig_block_fwd forms the gate logits in the mixer
    gemm = 2.0 * M * (D * nin + (0 if fused else R * HK) + HV * D + 2 * D * F)
    out = {"what": "dig_block_cond + %d x dig_block_fwd (four scan directions cycling)" % nb,
           "batch": B, "grid": [cfg.grid_h, cfg.grid_w], "d_model": D, "heads": H, "d_k": dk,
           "d_v": dv, "ffn_dim": F, "blocks": nb, "ms_per_forward": round(ms, 4),
           "images_per_s": round(B / (ms / 1e3), 2),
           "tokens_per_s": round(M / (ms / 1e3), 1),
           "matmul_flops_per_forward": gemm * nb,
           "matmul_tflops_over_whole_forward": round(gemm * nb / (ms / 1e3) / 1e12, 1),
           "graph_replay": {"ms_per_forward": round(ms_graph, 4),
                            "images_per_s": round(B / (ms_graph / 1e3), 2),
                            "tokens_per_s": round(M / (ms_graph / 1e3), 1)}}
    # one block's steps, each timed alone through the public calls dig_block_fwd composes
    t = keep[0]
    h, x1 = torch.empty_like(x0), torch.empty_like(x0)
    q, k, z = (torch.empty(M, HK, dtype=torch.bfloat16, device="cuda") for _ in range(3))
    v, r, y = (torch.empty(M, HV, dtype=torch.bfloat16, device="cuda") for _ in range(3))
    u = torch.empty(M, R, dtype=torch.bfloat16, device="cuda")
    hid = torch.empty(M, F, dtype=torch.bfloat16, device="cuda")
    gdesc = dig.make_desc(B, L, H, dk, dv, cfg.chunk, cfg.tau, 1.0, 1e-5, dig.DIG_BF16, 0)
    gwb = dig.dig_gla_fwd_workspace_bytes(gdesc)
    gws = torch.empty(max(gwb, 16), dtype=torch.uint8, device="cuda")
    rows = [0, HK, 2 * HK, 2 * HK + HV, 2 * HK + HV + R, nin]
    outs_in = [(o, t["w_in"][rows[i]:rows[i + 1]], t["b_in"][rows[i]:rows[i + 1]])
               for i, o in enumerate((q, k, v, u, r))]
    steps_ = (
        ("rmsnorm_modulate", lambda: dig.dig_rmsnorm_modulate(M, D, L, 1e-5, x0, mod, mod[:, D:],
                                                              mld, h), 0.0),
        ("in_projection", lambda: dig.dig_linear(M, D, h, outs_in), 2.0 * M * D * nin),
        ("gate_up_projection", lambda: dig.dig_linear(M, R, u, [(z, t["w_gate"], t["b_gate"])]),
         2.0 * M * R * HK),
        ("gla_fwd", lambda: dig.dig_gla_fwd(gdesc, q, k, v, z, r, t["gla_norm_w"], y, None, None,
                                            gws, gwb), 0.0),
        ("gla_fwd_lowrank", lambda: dig.dig_gla_fwd_lowrank(
            gdesc, q, k, v, u, t["w_gate"], t["b_gate"], r, t["gla_norm_w"], y, None, None, gws,
            gwb), 0.0),
        ("out_projection_gated_residual", lambda: dig.dig_linear(M, HV, y, [dig.linear_out(
            x1, t["w_out"], t["b_out"], res=x0, gate=mod[:, 2 * D:], gate_ld=mld,
            rows_per_gate=L)]), 2.0 * M * HV * D),
        ("ffn1_gelu", lambda: dig.dig_linear(M, D, h, [dig.linear_out(
            hid, t["w_ffn1"], t["b_ffn1"], act=dig.DIG_ACT_GELU)]), 2.0 * M * D * F),
        ("ffn2_gated_residual", lambda: dig.dig_linear(M, F, hid, [dig.linear_out(
            x1, t["w_ffn2"], t["b_ffn2"], res=x1, gate=mod[:, 5 * D:], gate_ld=mld,
            rows_per_gate=L)]), 2.0 * M * F * D),
        ("dwconv3x3_reorient", lambda: dig.dig_dwconv3x3(B, cfg.grid_h, cfg.grid_w, D,
                                                         dig.DIG_BF16, W.ROW, W.ROW_REV, x1,
                                                         t["conv_w"], t["conv_b"], xa), 0.0),
    )
    # the one-output products as dig_block_fwd issues them: K split over a workspace where the
    # grid of tiles would not fill the GPU
    lws = torch.empty(max(dig.dig_block_fwd_workspace_bytes(desc), 16), dtype=torch.uint8,
                      device="cuda")
    split = {
        "out_projection_gated_residual": lambda: dig.dig_linear_ws(M, HV, y, [dig.linear_out(
            x1, t["w_out"], t["b_out"], res=x0, gate=mod[:, 2 * D:], gate_ld=mld,
            rows_per_gate=L)], lws),
        "ffn1_gelu": lambda: dig.dig_linear_ws(M, D, h, [dig.linear_out(
            hid, t["w_ffn1"], t["b_ffn1"], act=dig.DIG_ACT_GELU)], lws),
        "ffn2_gated_residual": lambda: dig.dig_linear_ws(M, F, hid, [dig.linear_out(
            x1, t["w_ffn2"], t["b_ffn2"], res=x1, gate=mod[:, 5 * D:], gate_ld=mld,
            rows_per_gate=L)], lws),
    }
    # the steps dig_block_fwd runs: rank 16 forms the gate logits inside the mixer
    skip = ("gate_up_projection", "gla_fwd") if fused else ("gla_fwd_lowrank",)
    steps_ = tuple((n, split.get(n, fn), fl) for n, fn, fl in steps_ if n not in skip)
    parts = {}
    for pname, fn, flops in steps_:
        pm = timed_graph(fn, max(5, steps))
        e = {"us": round(pm * 1e3, 1)}
        if flops:
            tf = flops / (pm / 1e3) / 1e12
            e.update(tflops=round(tf, 1), frac_of_bf16_peak=round(tf / BF16_PEAK_TFLOPS, 4))
        else:
            e["gbs_in_out"] = round(2 * M * D * 2 / (pm / 1e3) / 1e9, 1) \
                if not pname.startswith("gla_fwd") \
                else round(gla_bytes_per_token_head(cfg, "fwd") * M * H / (pm / 1e3) / 1e9, 1)
        parts[pname] = e
    out["one_block_parts"] = parts
    out["one_block_us"] = round(ms * 1e3 / nb, 1)
    return out


def _median(xs):
    xs = sorted(xs)
    return xs[len(xs) // 2]


def _time_us(fn, reps=10, cold=None):
    """Average µs per call back to back (warm), or with `cold` given: the median of single
    calls, each after `cold()` (a 1 GiB write, outside the events) has flushed the caches."""
    import torch
    for _ in range(2):
        fn()
    torch.cuda.synchronize()
    if cold is None:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps * 1e3
    ts = []
    for _ in range(reps):
        cold()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) * 1e3)
    return _median(ts)


def probes():
    """Probes outside the timed step, labelled as such: single library calls on larger inputs
    (warm: back to back; cold: after a 1 GiB write), and the streaming-copy ceiling of the same
    bytes (this repository's own copy kernel)."""
    import torch
    import diffusion_backbone_amd as dig
    PL = probe_lib()
    flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")   # 1 GiB
    cold = lambda: flush.fill_(1.0)
    out = {}

    def rec(key, call, shape, us, byts, **kw):
        gbs = byts / (us / 1e6) / 1e9
        out[key] = dict(call=call, shape=shape, us=round(us, 1), achieved_gbs=round(gbs, 1),
                        frac=round(gbs / HBM_PEAK_GBS, 4), **kw)

    def gla(label, B, L, H, dk, dv, chunk=64):
        bt = lambda *sh: torch.randn(*sh, device="cuda").to(torch.bfloat16)
        q, k, v, r = bt(B, L, H, dk), bt(B, L, H, dk), bt(B, L, H, dv), bt(B, L, H, dv)
        z = (torch.randn(B, L, H, dk, device="cuda") * 0.2).to(torch.bfloat16)
        dy = bt(B, L, H, dv)
        desc = dig.make_desc(B, L, H, dk, dv, chunk, 16.0, 1.0, 1e-5, dig.DIG_BF16, 0)
        by = lambda n: torch.empty(max(int(n), 16), dtype=torch.uint8, device="cuda")
        fwb, bwb = dig.dig_gla_fwd_workspace_bytes(desc), dig.dig_gla_bwd_workspace_bytes(desc)
        fws, bws, saved = by(fwb), by(bwb), by(dig.dig_gla_saved_bytes(desc))
        y = torch.empty_like(r)
        g = [torch.empty_like(q), torch.empty_like(k), torch.empty_like(v), torch.empty_like(z),
             torch.empty_like(r)]
        dgam = torch.empty(dv, device="cuda")
        f = lambda: dig.dig_gla_fwd(desc, q, k, v, z, r, None, y, None, saved, fws, fwb)
        bw = lambda: dig.dig_gla_bwd(desc, q, k, v, z, r, None, dy, saved, *g, dgam, bws, bwb)
        th = B * L * H
        for name, fn, byts in (("fwd", f, 2 * (3 * dk + 3 * dv) * th),
                               ("bwd", bw, 2 * (6 * dk + 5 * dv) * th)):
            for mode in ("warm", "cold"):
                us = _time_us(fn, cold=cold if mode == "cold" else None)
                rec("%s_%s_%s" % (label, name, mode), "dig_gla_" + name, [B, L, H, dk, dv], us,
                    byts, tokens_per_s=round(B * L / (us / 1e6), 1))
        del q, k, v, r, z, dy, y, g, fws, bws, saved

    def srem(label, B, gh, gw, D):
        x = torch.randn(B, gh * gw, D, device="cuda").to(torch.bfloat16)
        dy = torch.randn_like(x)
        y, dx = torch.empty_like(x), torch.empty_like(x)
        w = torch.randn(D, 3, 3, device="cuda") / 3.0
        dw, db = torch.empty_like(w), torch.empty(D, device="cuda")
        wsb = dig.dig_dwconv3x3_bwd_workspace_bytes(B, gh, gw, D)
        ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda")
        nb = x.numel() * 2
        R, C = dig.DIG_SCAN_ROW, dig.DIG_SCAN_COL
        cases = (
            ("reorient", "dig_srem_reorient",
             lambda: dig.dig_srem_reorient(B, gh, gw, D, dig.DIG_BF16, R, C, x, y), 2 * nb),
            ("dwconv3x3", "dig_dwconv3x3",
             lambda: dig.dig_dwconv3x3(B, gh, gw, D, dig.DIG_BF16, R, C, x, w, None, y), 2 * nb),
            ("dwconv3x3_bwd", "dig_dwconv3x3_bwd",
             lambda: dig.dig_dwconv3x3_bwd(B, gh, gw, D, dig.DIG_BF16, R, C, x, w, dy, dx, dw, db,
                                           ws, wsb), 3 * nb),
            ("copy_ceiling", "streaming copy (probe kernel, not the library)",
             lambda: device_copy(PL, x, y), 2 * nb))
        for mode in ("warm", "cold"):
            for name, call, fn, byts in cases:
                us = _time_us(fn, cold=cold if mode == "cold" else None)
                rec("%s_%s_%s" % (label, name, mode), call, [B, gh, gw, D], us, byts)
            ceil = out["%s_copy_ceiling_%s" % (label, mode)]["achieved_gbs"]
            for name, *_ in cases[:3]:
                e = out["%s_%s_%s" % (label, name, mode)]
                e["frac_of_copy_ceiling"] = round(e["achieved_gbs"] / ceil, 4)
        del x, dy, y, dx, ws

    gla("s2_b256", 256, 256, 6, 32, 64)
    c5 = W.CONFIGS["dig_xl2_2048"]
    srem("xl2_2048", c5.batch, c5.grid_h, c5.grid_w, c5.d_model)
    # 16 images: 604 MB per tensor, past the 256 MB Infinity Cache (HBM streaming regime)
    srem("xl2_2048_b16", 16, c5.grid_h, c5.grid_w, c5.d_model)
    del flush
    torch.cuda.empty_cache()
    return out


# ------------------------------------------------------------------ CPU baseline
def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_leg(spec):
    """Child process (no GPU): times the fp64 oracle on a bounded sample of one
    configuration's step and prints one JSON line.  spec = "<workload>:<blocks>:<div>:<min_s>":
    `blocks` blocks, each over heads / div of the heads and d_model / div of the channels."""
    import oracle
    name, nblk, div, min_s = spec.split(":")
    cfg, nblk, div, min_s = W.CONFIGS[name], int(nblk), int(div), float(min_s)
    cfg = W.cfg_replace(cfg, heads=cfg.heads // div, d_model=cfg.d_model // div)
    case = W.make_gla_case(cfg)
    srem = W.make_srem_case(cfg)
    gh, gw = cfg.grid_h, cfg.grid_w
    best, reps, t_all = None, 0, time.perf_counter()
    while True:
        t0 = time.perf_counter()
        for l in range(nblk):
            d0, d1 = W.SCHEDULE[l % 4], W.SCHEDULE[(l + 1) % 4]
            oracle.gla_fwd(case.q, case.k, case.v, case.z, case.r, case.gamma)
            oracle.dwconv3x3(srem.x, srem.w, gh, gw, d0, d1)
        for l in reversed(range(nblk)):
            d0, d1 = W.SCHEDULE[l % 4], W.SCHEDULE[(l + 1) % 4]
            oracle.dwconv3x3_bwd(srem.x, srem.w, srem.dy, gh, gw, d0, d1)
            oracle.gla_bwd(case.q, case.k, case.v, case.z, case.r, case.dy, case.gamma)
        t = time.perf_counter() - t0
        best = t if best is None else min(best, t)
        reps += 1
        if (reps >= 3 and time.perf_counter() - t_all > min_s) or time.perf_counter() - t_all > 3 * min_s:
            break
    print(json.dumps({"seconds_best": best, "reps": reps, "threads": oracle.num_threads(),
                      "wall": time.perf_counter() - t_all}), flush=True)


def cpu_baseline(cfg):
    """The oracle (untuned) on this host: a bounded sample of the headline step (one block in
    its first scan direction; a quarter of the heads and channels for the single-thread leg),
    best of at least three repetitions, single-threaded and on every thread OpenMP is given
    (each leg in a child process); the oracle's work is linear in heads, channels and blocks,
    so the sample's time is scaled to GLA-layer tokens/s of the full step."""
    import subprocess
    nb = n_blocks(cfg)
    res, divs = {}, {}
    # the oracle runs its (image, head) units in parallel: the all-threads leg keeps every head
    for leg, threads, div in (("single_thread", "1", 4), ("all_threads", None, 1)):
        divs[leg] = div
        env = dict(os.environ)
        if threads:
            env["OMP_NUM_THREADS"] = threads
        cmd = [sys.executable, os.path.abspath(__file__), "--oracle-leg",
               "%s:1:%d:4.0" % (cfg.name, div)]
        p = subprocess.run(cmd, env=env, capture_output=True, text=True, timeout=600)
        if p.returncode != 0:
            raise RuntimeError("oracle leg failed: %s" % p.stderr[-2000:])
        r = json.loads(p.stdout.strip().splitlines()[-1])
        step_s = r["seconds_best"] * div * nb          # the full step's time at this rate
        res[leg] = {"value": round(cfg.batch * cfg.seq_len * nb / step_s, 1),
                    "cores": r["threads"], "sample_seconds_best": round(r["seconds_best"], 3),
                    "reps": r["reps"]}
    allc = res["all_threads"]
    return {"value": allc["value"], "unit": "GLA-layer tokens/s (fwd+bwd)", "cores": allc["cores"],
            "kind": "oracle",
            "sample": "fp64 oracle fwd+bwd (GLA mixer + conv/reorient) of one %s block, best "
                      "of >= 3 repetitions, scaled to the %d-block step: all threads over all "
                      "%d heads and %d channels, single thread over %d heads and %d channels"
                      % (cfg.name, nb, cfg.heads, cfg.d_model, cfg.heads // divs["single_thread"],
                         cfg.d_model // divs["single_thread"]),
            "host_cpu": _cpu_model(), "single_thread": res["single_thread"],
            "all_threads": allc}


def main():
    args = parse()
    if args.oracle_leg:
        oracle_leg(args.oracle_leg)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the hot path here has no multi-GPU leg "
              "(data-parallel sharding is a design note, not built). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if args.copy_probe_mib:
        copy_probe(args.copy_probe_mib, max(1, args.steps), args.copy_probe_width)
        return
    if args.stack:
        print(json.dumps({args.stack: block_stack(args.stack, max(1, args.steps))}), flush=True)
        return
    if args.value_gate:
        print(json.dumps({"value_gate": value_gate(W.CONFIGS[args.workload])}), flush=True)
        return
    cfg = W.CONFIGS[args.workload]
    nblocks = n_blocks(cfg)
    if args.pmc_target:  # one library call per block, `steps` times (for counter runs)
        path = Path(cfg, gen_blocks(cfg, nblocks, cfg.seed), args.seg_chunks)
        for l in range(nblocks):  # the forward's saved buffers feed the backward
            path.gla_fwd(l)
        torch.cuda.synchronize()
        fn = getattr(path, args.pmc_target)
        for _ in range(args.steps):
            for l in range(nblocks):
                fn(l)
        torch.cuda.synchronize()
        print(json.dumps({"pmc_target": args.pmc_target, "calls": args.steps * nblocks}),
              flush=True)
        return

    blocks = gen_blocks(cfg, nblocks, cfg.seed)
    path = Path(cfg, blocks, args.seg_chunks)
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        path.step()
    torch.cuda.synchronize()

    # timed region: exactly K steps, the library calls back to back on the stream
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(args.steps):
        path.step()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    tokens = cfg.batch * cfg.seq_len * nblocks
    value = tokens / (ms / 1e3)

    # second timed pass of K steps with HIP events around every GLA call (kept out of the
    # first: recording events between calls adds host work and stream markers)
    ev = EventTimer(2 * nblocks * args.steps)
    torch.cuda.synchronize()
    s1, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s1.record()
    for _ in range(args.steps):
        path.step(ev)
    e1.record()
    torch.cuda.synchronize()
    ms_ev = s1.elapsed_time(e1) / args.steps
    ms_fwd = timed(path.step_fwd, args.steps, 3)
    ms_graph = timed_graph(path.step, args.steps, reps=1)  # the same step replayed from a graph

    th = cfg.batch * cfg.seq_len * cfg.heads
    rl = {}
    for name, which in (("gla_fwd", "fwd"), ("gla_bwd", "bwd")):
        t = ev.avg_ms(name)
        byts = gla_bytes_per_token_head(cfg, which) * th
        rl[name] = {"ms": t, "bytes": byts, "gbs": byts / (t / 1e3) / 1e9}
    dom = max(rl, key=lambda n: rl[n]["ms"])
    other = [n for n in rl if n != dom][0]
    roof = {"bound": "hbm", "achieved": round(rl[dom]["gbs"], 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(rl[dom]["gbs"] / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(cfg.name, "dig_" + dom),
            "call": "dig_" + dom, "avg_call_us": round(rl[dom]["ms"] * 1e3, 2),
            "algorithmic_bytes_per_launch": rl[dom]["bytes"],
            "bytes_per_token_head": gla_bytes_per_token_head(cfg, dom[4:]),
            "source": "HIP events around each dig_%s call on the stream its kernels run on, in a "
                      "second timed pass of the same K steps (%.4f ms/step with the events); the "
                      "rocprofv3 kernel-trace summary of this command gives the call's kernel "
                      "durations" % (dom, ms_ev)}
    del path, blocks
    torch.cuda.empty_cache()
    out = {
        "metric": "GLA-layer tokens/s (fwd+bwd)",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "batch": cfg.batch, "grid": [cfg.grid_h, cfg.grid_w],
                   "seq_len": cfg.seq_len, "d_model": cfg.d_model, "heads": cfg.heads,
                   "d_k": cfg.d_k, "d_v": cfg.d_v, "chunk": cfg.chunk, "blocks": nblocks,
                   "step": "%d x (gla_fwd + dwconv3x3 reorient) + %d x (dwconv3x3_bwd + gla_bwd), "
                           "scan directions cycling row, row_rev, col, col_rev"
                           % (nblocks, nblocks)},
        "fwd_only": {"value": round(tokens / (ms_fwd / 1e3), 1), "unit": "tokens/s",
                     "ms_per_step": round(ms_fwd, 4)},
        "graph_replay": {"value": round(tokens / (ms_graph / 1e3), 1), "unit": "tokens/s",
                         "ms_per_step": round(ms_graph, 4),
                         "what": "the same K steps, each replayed from one captured HIP graph"},
        "roofline": roof,
        "roofline_other_call": {"call": "dig_" + other, "avg_call_us": round(rl[other]["ms"] * 1e3, 2),
                                "achieved_gbs": round(rl[other]["gbs"], 1),
                                "frac": round(rl[other]["gbs"] / HBM_PEAK_GBS, 4),
                                "traffic": measured_traffic(cfg.name, "dig_" + other)},
    }
    if not args.no_probes:
        configs = {}
        for name in ("dig_s2_256", "dig_s2_1792", "dig_xl2_1024"):
            if name == cfg.name:
                continue
            c = W.CONFIGS[name]
            configs[name], _ = run_config(c, max(10, args.steps // 2), 3,
                                          fwd_only=(name == "dig_xl2_1024"))
            print("[bench] %s done" % name, file=sys.stderr, flush=True)
        out["configs"] = configs
        out["lowrank_gate"] = lowrank_gate(cfg, max(10, args.steps // 2))
        print("[bench] lowrank_gate done", file=sys.stderr, flush=True)
        out["value_gate"] = value_gate(cfg)
        print("[bench] value_gate done", file=sys.stderr, flush=True)
        out["projections"] = projections(cfg, max(10, args.steps // 2))
        stacks = {}
        for sname in ("dig_s2_256_stack", "dig_xl2_256_stack", "dig_xl2_2048_stack"):
            stacks[sname] = block_stack(sname, max(5, args.steps // 10))
            print("[bench] %s done" % sname, file=sys.stderr, flush=True)
        out["block_stack_fwd"] = stacks
        out["mfma_microbench"] = contraction_microbench()
        out["probes"] = probes()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
