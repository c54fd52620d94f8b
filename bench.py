#!/usr/bin/env python3
"""Throughput of the DiG hot path on one MI355X: GLA token mixer + SREM, forward and backward.

One step = one pass of the whole path over one batch of synthetic DiG-S/2 256-px input:
for each of the 12 blocks (scan directions cycling row, row_rev, col, col_rev)
    dig_gla_fwd (saving chunk states) -> dig_dwconv3x3 (fused reorient to the next direction)
then, blocks in reverse,
    dig_dwconv3x3_bwd -> dig_gla_bwd.
Inputs are generated on the GPU before timing (seeded, x ~ N(0,1), weights ~ N(0, 1/D)).
The metric is GLA-layer tokens/s: batch * tokens * blocks / step time.

Prints ONE JSON line.  --gpus N with N > 1 exits: this build runs on one GPU.
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
BF16_PEAK_TFLOPS = 2500.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="dig_s2_256", choices=sorted(W.CONFIGS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probes", action="store_true",
                    help="skip the steady-state probes (larger shapes, outside the timed step)")
    ap.add_argument("--seg-chunks", type=int, default=0)
    ap.add_argument("--quiet", action="store_true")
    # profiling helpers (rocprofv3 counter runs): run only one library call of the step, or a
    # plain device copy of known size that calibrates the byte counters
    ap.add_argument("--pmc-target", choices=["gla_fwd", "gla_bwd", "srem_fwd", "srem_bwd"],
                    default=None)
    ap.add_argument("--copy-probe-mib", type=int, default=0)
    return ap.parse_args()


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
        z = ((x @ w(D, cfg.rank)) @ w(cfg.rank, H * dk)).view(B, L, H, dk)
        r = (x @ w(D, H * dv)).view(B, L, H, dv)
        cw = torch.randn(D, 3, 3, device="cuda", generator=g) / 3.0
        dy = torch.randn(B, L, H, dv, device="cuda", generator=g)
        dys = torch.randn(B, L, D, device="cuda", generator=g)
        bf = lambda t: t.to(torch.bfloat16).contiguous()
        blocks.append(dict(q=bf(q), k=bf(k), v=bf(v), z=bf(z), r=bf(r), x=bf(x.view(B, L, D)),
                           cw=cw.contiguous(), dy=bf(dy), dys=bf(dys),
                           gamma=torch.ones(dv, device="cuda")))
    return blocks


class Path:
    """Buffers and the library calls of one step."""

    def __init__(self, cfg, blocks, seg_chunks):
        import torch
        import diffusion_backbone_amd as dig
        self.dig, self.cfg, self.blocks = dig, cfg, blocks
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
    """HIP events around chosen calls on torch's current stream (the stream they run on).
    The events are created up front so that recording them adds no allocation to the
    timed region."""

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


# HBM traffic of one GLA call on the default workload, from rocprofv3 FETCH_SIZE and
# WRITE_SIZE runs (summed over the call's kernels) divided by the counters' reading per byte
# of a plain copy; valid only for the kernel sources it was measured on (sha256 below).
TRAFFIC = {
    "workload": "dig_s2_256",
    "bytes": {
        # FETCH_SIZE 8886.1 KiB / 0.50006 (copy: 131088.0 KiB read per 262144 KiB moved) +
        # WRITE_SIZE 6997.8 KiB / 1.0 (copy: 262144 KiB written per 262144 KiB moved)
        "dig_gla_bwd": 25362253,
        # FETCH_SIZE 5145.2 KiB / 0.50006 + WRITE_SIZE 7765.5 KiB / 1.0
        "dig_gla_fwd": 18487983,
    },
    "sources_sha256": "834f09c8cae3003b695a888b3be3d3f76831e6e85b8238bc8e8beeea36dc9391",
}
TRAFFIC_SOURCES = ("diffusion_backbone_amd/csrc/gla_bwd_kernel.h",
                   "diffusion_backbone_amd/csrc/gla_bwd.hip",
                   "diffusion_backbone_amd/csrc/gla_fwd_kernel.h",
                   "diffusion_backbone_amd/csrc/gla_fwd.hip",
                   "diffusion_backbone_amd/csrc/dig_device.h")


# The kernels one call runs on the default workload (B=8, 16x16 grid, 6 heads: 4 chunks of 64
# tokens per image and head).
KERNEL_OF_CALL = {
    "gla_bwd": "gla_bwd_kernel, look-back (one chunk per workgroup, one launch)",
    "gla_fwd": "gla_fwd_kernel, look-back (one chunk per workgroup, one launch)",
}


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


def copy_probe(mib, reps):
    """A plain copy of known size through dig_srem_reorient (identity order): the reference
    for scaling FETCH_SIZE / WRITE_SIZE counter readings to bytes."""
    import torch
    import diffusion_backbone_amd as dig
    n = mib * 1024 * 1024 // 2
    D = 1024
    rows = n // D
    x = torch.ones(rows * D, dtype=torch.bfloat16, device="cuda")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(reps):
        dig.dig_srem_reorient(1, 1, rows, D, dig.DIG_BF16, dig.DIG_SCAN_ROW, dig.DIG_SCAN_ROW, x, y)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_each_way": rows * D * 2, "reps": reps}), flush=True)


def gla_bytes_per_token_head(cfg, which):
    """Algorithmic HBM bytes per (token, head) of one mixer call (bf16 I/O)."""
    dk, dv = cfg.d_k, cfg.d_v
    if which == "fwd":   # read q, k, z, v, r; write y
        return 2 * (3 * dk + 3 * dv)
    # bwd: read q, k, z, v, r, dy; write dq, dk, dz, dv, dr
    return 2 * (6 * dk + 5 * dv)


def cpu_baseline(cfg, nblocks):
    """The fp64 oracle on the host: one full step (fwd + bwd of every block) of a bounded
    sample of the batch, scaled to GLA-layer tokens/s."""
    import oracle
    sample_batch = max(1, min(cfg.batch, 2))
    scfg = W.cfg_replace(cfg, batch=sample_batch)
    case = W.make_gla_case(scfg)
    srem = W.make_srem_case(scfg)
    gh, gw = cfg.grid_h, cfg.grid_w
    t0 = time.perf_counter()
    reps = 0
    while True:
        for l in range(nblocks):
            d0, d1 = W.SCHEDULE[l % 4], W.SCHEDULE[(l + 1) % 4]
            oracle.gla_fwd(case.q, case.k, case.v, case.z, case.r, case.gamma)
            oracle.dwconv3x3(srem.x, srem.w, gh, gw, d0, d1)
        for l in reversed(range(nblocks)):
            d0, d1 = W.SCHEDULE[l % 4], W.SCHEDULE[(l + 1) % 4]
            oracle.dwconv3x3_bwd(srem.x, srem.w, srem.dy, gh, gw, d0, d1)
            oracle.gla_bwd(case.q, case.k, case.v, case.z, case.r, case.dy, case.gamma)
        reps += 1
        el = time.perf_counter() - t0
        if el > 10.0 or reps >= 200:
            break
    tokens = sample_batch * cfg.seq_len * nblocks * reps
    return {"value": tokens / el, "unit": "GLA-layer tokens/s (fwd+bwd)",
            "cores": oracle.num_threads(), "kind": "oracle",
            "sample": "%d full fwd+bwd step(s) of %d of %d images (%d blocks, %d tokens each), %.1f s"
                      % (reps, sample_batch, cfg.batch, nblocks, cfg.seq_len, el)}


def _time_us(fn, reps=10):
    import torch
    for _ in range(2):
        fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps * 1e3


def probes():
    """Steady-state probes, outside the timed step: one library call at a time, back to back,
    on inputs large enough that launch latency does not dominate.  Labelled as probes: they
    are not the step's workload."""
    import torch
    import diffusion_backbone_amd as dig
    out = {}

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
        tf = _time_us(lambda: dig.dig_gla_fwd(desc, q, k, v, z, r, None, y, None, saved, fws, fwb))
        tb = _time_us(lambda: dig.dig_gla_bwd(desc, q, k, v, z, r, None, dy, saved, *g, dgam,
                                              bws, bwb))
        th = B * L * H
        for name, t, byts in (("fwd", tf, 2 * (3 * dk + 3 * dv) * th),
                              ("bwd", tb, 2 * (6 * dk + 5 * dv) * th)):
            gbs = byts / (t / 1e6) / 1e9
            out["%s_%s" % (label, name)] = {
                "call": "dig_gla_" + name, "shape": [B, L, H, dk, dv], "us": round(t, 1),
                "tokens_per_s": round(B * L / (t / 1e6), 1), "achieved_gbs": round(gbs, 1),
                "frac": round(gbs / HBM_PEAK_GBS, 4)}
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
            ("reorient", lambda: dig.dig_srem_reorient(B, gh, gw, D, dig.DIG_BF16, R, C, x, y), 2 * nb),
            ("dwconv3x3", lambda: dig.dig_dwconv3x3(B, gh, gw, D, dig.DIG_BF16, R, C, x, w, None, y),
             2 * nb),
            ("dwconv3x3_bwd", lambda: dig.dig_dwconv3x3_bwd(B, gh, gw, D, dig.DIG_BF16, R, C, x, w, dy,
                                                           dx, dw, db, ws, wsb), 3 * nb))
        for name, fn, byts in cases:
            t = _time_us(fn)
            gbs = byts / (t / 1e6) / 1e9
            out["%s_%s" % (label, name)] = {
                "call": "dig_" + ("srem_" + name if name == "reorient" else name),
                "shape": [B, gh, gw, D], "us": round(t, 1), "achieved_gbs": round(gbs, 1),
                "frac": round(gbs / HBM_PEAK_GBS, 4)}
        # reference ceiling: the runtime's own device copy of the same bytes (torch copy_)
        t = _time_us(lambda: y.copy_(x))
        gbs = 2 * nb / (t / 1e6) / 1e9
        out["%s_copy_ref" % label] = {
            "call": "torch copy_ (reference, not the library)", "shape": [B, gh, gw, D],
            "us": round(t, 1), "achieved_gbs": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4)}
        del x, dy, y, dx, ws

    gla("s2_b256", 256, 256, 6, 32, 64)
    c5 = W.CONFIGS["dig_xl2_2048"]
    gla("xl2_2048", c5.batch, c5.seq_len, c5.heads, c5.d_k, c5.d_v)
    srem("xl2_2048", c5.batch, c5.grid_h, c5.grid_w, c5.d_model)
    # 16 images: 604 MB per tensor, past the 256 MB Infinity Cache (HBM streaming regime)
    srem("xl2_2048_b16", 16, c5.grid_h, c5.grid_w, c5.d_model)
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the hot path here has no multi-GPU leg "
              "(data-parallel sharding is a design note, not built). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if args.copy_probe_mib:
        copy_probe(args.copy_probe_mib, max(1, args.steps))
        return
    cfg = W.CONFIGS[args.workload]
    nblocks = cfg.blocks
    blocks = gen_blocks(cfg, nblocks, cfg.seed)
    path = Path(cfg, blocks, args.seg_chunks)
    torch.cuda.synchronize()
    if args.pmc_target:  # one library call per block, `steps` times (for counter runs)
        fn = getattr(path, args.pmc_target)
        for _ in range(args.steps):
            for l in range(nblocks):
                fn(l)
        torch.cuda.synchronize()
        print(json.dumps({"pmc_target": args.pmc_target, "calls": args.steps * nblocks}),
              flush=True)
        return

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
    tokens = cfg.batch * cfg.seq_len * nblocks
    value = tokens / (ms / 1e3)

    # forward-only figure (same calls without the backward), reported beside the main value
    for _ in range(3):
        path.step_fwd()
    torch.cuda.synchronize()
    s2, e2 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s2.record()
    for _ in range(args.steps):
        path.step_fwd()
    e2.record()
    torch.cuda.synchronize()
    ms_fwd = s2.elapsed_time(e2) / args.steps

    th = cfg.batch * cfg.seq_len * cfg.heads
    rl = {}
    for name, which in (("gla_fwd", "fwd"), ("gla_bwd", "bwd")):
        t = ev.avg_ms(name)
        byts = gla_bytes_per_token_head(cfg, which) * th
        rl[name] = {"ms": t, "bytes": byts, "gbs": byts / (t / 1e3) / 1e9}
    dom = max(rl, key=lambda n: rl[n]["ms"])
    traffic = measured_traffic(cfg.name, "dig_" + dom)
    roof = {"bound": "hbm", "achieved": round(rl[dom]["gbs"], 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(rl[dom]["gbs"] / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel": KERNEL_OF_CALL[dom],
            "call": "dig_" + dom, "avg_call_us": round(rl[dom]["ms"] * 1e3, 2),
            "algorithmic_bytes_per_launch": rl[dom]["bytes"],
            "note": "per library call: HIP events bracket the whole call on its stream, "
                    "in a second timed pass of the same K steps (%.4f ms/step with the events)"
                    % ms_ev}
    other = [n for n in rl if n != dom][0]
    traffic_other = measured_traffic(cfg.name, "dig_" + other)
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
                   "step": "12 x (gla_fwd + dwconv3x3 reorient) + 12 x (dwconv3x3_bwd + gla_bwd)"},
        "fwd_only": {"value": round(tokens / (ms_fwd / 1e3), 1), "unit": "tokens/s",
                     "ms_per_step": round(ms_fwd, 4)},
        "roofline": roof,
        "roofline_other_call": {"call": "dig_" + other, "avg_call_us": round(rl[other]["ms"] * 1e3, 2),
                                "achieved_gbs": round(rl[other]["gbs"], 1),
                                "frac": round(rl[other]["gbs"] / HBM_PEAK_GBS, 4),
                                "kernel": KERNEL_OF_CALL[other], "traffic": traffic_other},
    }
    if not args.no_probes:
        out["probes"] = probes()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, nblocks)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
