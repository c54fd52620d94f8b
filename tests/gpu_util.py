"""Helpers for the GPU parity tests: upload/download of quantised arrays, error metric, and
thin drivers that run one library call on torch-allocated buffers."""
from __future__ import annotations

import sys

import numpy as np

import workloads as W


def has_gpu() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def announce(msg: str):
    print("[case] " + msg, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray, dtype: str):
    import torch
    raw = W.storage(a, dtype)
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(raw).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(raw))
    return t.cuda()


def to_f64(t) -> np.ndarray:
    import torch
    t = t.detach()
    if t.dtype == torch.bfloat16:
        bits = t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        return W.bf16_to_f64(bits)
    return t.cpu().numpy().astype(np.float64)


def empty(shape, dtype: str, fill_nan: bool = True):
    """Output buffer, NaN-poisoned so that unwritten elements show up."""
    import torch
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    t = torch.empty(shape, dtype=td, device="cuda")
    if fill_nan:
        t.fill_(float("nan"))
    return t


def nbytes_buf(n: int):
    """Workspace / saved buffer, every byte 0xFF (NaN in fp32 and bf16), so that a read of
    an element nothing wrote shows up."""
    import torch
    return torch.full((max(int(n), 16),), 255, dtype=torch.uint8, device="cuda")


def maxrel(got: np.ndarray, ref: np.ndarray) -> float:
    """max_i |got_i - ref_i| / max_i |ref_i| (normwise by the reference's max)."""
    denom = float(np.max(np.abs(ref))) if ref.size else 0.0
    if ref.size == 0:
        return 0.0
    diff = np.abs(got - ref)
    if not np.all(np.isfinite(got)):
        return float("inf")
    return float(np.max(diff)) / (denom if denom > 0 else 1.0)


TOL = {"bf16": 2e-2, "f32": 1e-4}


def elementwise_diag(got: np.ndarray, ref: np.ndarray) -> str:
    """Elementwise diagnostics of a [B, L, H, d] tensor (logged, not asserted): where the
    normwise error peaks (token, head) and the largest elementwise relative error over the
    elements whose reference exceeds 1e-3 of the tensor's max."""
    d = np.abs(got - ref)
    at = np.unravel_index(int(np.argmax(d)), d.shape)
    big = np.abs(ref) > 1e-3 * np.max(np.abs(ref))
    ew = float(np.max(d[big] / np.abs(ref[big]))) if np.any(big) else 0.0
    return "t%d/h%d ew%.1e" % (at[1], at[2], ew)


def gla_forward(case: W.GLACase, chunk: int, *, seg_chunks: int = 0, want_saved: bool = False,
                want_opre: bool = True, gamma=True, tau: float = 16.0, q_scale: float = 1.0,
                eps: float = 1e-5, ws=None, lowrank: W.LowRankGate | None = None):
    """Runs dig_gla_fwd (dig_gla_fwd_lowrank with `lowrank`: the gate from its factor, W_a2
    and bias instead of case.z) on the case; returns dict of device tensors."""
    import torch
    import diffusion_backbone_amd as dig
    cfg = case.cfg
    B, L, H, dk = case.q.shape
    dv = case.v.shape[-1]
    dt = cfg.dtype
    desc = dig.make_desc(B, L, H, dk, dv, chunk, tau, q_scale, eps, dt, seg_chunks)
    d = {n: to_dev(getattr(case, n), dt) for n in ("q", "k", "v", "r")}
    if lowrank is None:
        d["z"] = to_dev(case.z, dt)
    else:
        d["z"] = to_dev(lowrank.factor, "bf16")
        d["zw"] = to_dev(lowrank.w, "bf16")
        d["zb"] = torch.from_numpy(lowrank.bias.astype(np.float32)).cuda()
    d["lowrank"] = lowrank is not None
    d["gamma"] = torch.from_numpy(case.gamma.astype(np.float32)).cuda() if gamma else None
    d["y"] = empty((B, L, H, dv), dt)
    d["o_pre"] = empty((B, L, H, dv), dt) if want_opre else None
    d["saved"] = nbytes_buf(dig.dig_gla_saved_bytes(desc)) if want_saved else None
    wsb = dig.dig_gla_fwd_workspace_bytes(desc)
    d["ws"] = (nbytes_buf(wsb) if wsb else None) if ws is None else ws  # may be reused
    assert d["ws"] is None or d["ws"].numel() >= wsb
    if lowrank is None:
        dig.dig_gla_fwd(desc, d["q"], d["k"], d["v"], d["z"], d["r"], d["gamma"], d["y"],
                        d["o_pre"], d["saved"], d["ws"], wsb)
    else:
        dig.dig_gla_fwd_lowrank(desc, d["q"], d["k"], d["v"], d["z"], d["zw"], d["zb"], d["r"],
                                d["gamma"], d["y"], d["o_pre"], d["saved"], d["ws"], wsb)
    d["desc"] = desc
    return d


def gla_backward(case: W.GLACase, fwd: dict, *, dgamma: bool = True, ws=None):
    import torch
    import diffusion_backbone_amd as dig
    dt = case.cfg.dtype
    desc = fwd["desc"]
    B, L, H, dk = case.q.shape
    dv = case.v.shape[-1]
    g = {"dy": to_dev(case.dy, dt)}
    for n, d in (("dq", dk), ("dk", dk), ("dz", dk), ("dv", dv), ("dr", dv)):
        g[n] = empty((B, L, H, d), dt)
    g["dgamma"] = torch.full((dv,), float("nan"), dtype=torch.float32, device="cuda") if dgamma else None
    wsb = dig.dig_gla_bwd_workspace_bytes(desc)
    g["ws"] = nbytes_buf(wsb) if ws is None else ws   # a caller's workspace may be reused
    assert g["ws"].numel() >= wsb
    if not fwd.get("lowrank"):
        dig.dig_gla_bwd(desc, fwd["q"], fwd["k"], fwd["v"], fwd["z"], fwd["r"], fwd["gamma"],
                        g["dy"], fwd["saved"], g["dq"], g["dk"], g["dv"], g["dz"], g["dr"],
                        g["dgamma"], g["ws"], wsb)
    else:
        dig.dig_gla_bwd_lowrank(desc, fwd["q"], fwd["k"], fwd["v"], fwd["z"], fwd["zw"],
                                fwd["zb"], fwd["r"], fwd["gamma"], g["dy"], fwd["saved"], g["dq"],
                                g["dk"], g["dv"], g["dz"], g["dr"], g["dgamma"], g["ws"], wsb)
    return g
