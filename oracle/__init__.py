"""fp64 CPU oracle for the DiG GLA token mixer and SREM step (ctypes over dig_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py``.  The product library never imports it.

What each function computes, and the passages it follows, is documented in
``dig_oracle.c``.  Arrays are float64 numpy arrays in the layouts stated there:
GLA tensors ``[B, L, H, d]``, SREM tensors ``[B, L, D]``, conv weights ``[D, 3, 3]``.

Functions with no pin of their own besides the tests in ``tests/test_oracle_*.py``:
none -- every entry point is pinned there (brute force, closed forms, finite
differences, library convolution, explicit transposes).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dig_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

ROW, ROW_REV, COL, COL_REV = 0, 1, 2, 3


def build(force: bool = False) -> str:
    """Compile dig_oracle.c with gcc (-O2, no fast-math, OpenMP over independent units)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp",
                               "-fno-fast-math", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        D = ctypes.POINTER(ctypes.c_double)
        I64 = ctypes.POINTER(ctypes.c_int64)
        i, d, v, i64 = ctypes.c_int, ctypes.c_double, ctypes.c_void_p, ctypes.c_int64
        lib.oref_logsigmoid.argtypes = [d]
        lib.oref_logsigmoid.restype = d
        lib.oref_sigmoid.argtypes = [d]
        lib.oref_sigmoid.restype = d
        lib.oref_gate_logalpha.argtypes = [ctypes.c_size_t, D, d, D]
        lib.oref_gla_recurrence.argtypes = [i, i, i, i, i, D, D, D, D, d, D]
        lib.oref_output_stage.argtypes = [i, i, i, i, D, D, D, d, D, D]
        lib.oref_gla_fwd.argtypes = [i, i, i, i, i, D, D, D, D, D, D, d, d, d, D, D, D]
        lib.oref_gla_bwd_logalpha.argtypes = [i, i, i, i, i, D, D, D, D, D, D, d, d, D,
                                              D, D, D, D, D, D]
        lib.oref_gla_bwd.argtypes = [i, i, i, i, i, D, D, D, D, D, D, d, d, d, D,
                                     D, D, D, D, D, D]
        lib.oref_gla_fwd_beta.argtypes = [i, i, i, i, i, D, D, D, D, D, D, D, d, d, d, D, D, D]
        lib.oref_gla_bwd_beta.argtypes = [i, i, i, i, i, D, D, D, D, D, D, D, d, d, d, D,
                                          D, D, D, D, D, D, D]
        lib.oref_scan_canonical.argtypes = [i, i64, i64, i64]
        lib.oref_scan_canonical.restype = i64
        lib.oref_scan_perm.argtypes = [i, i64, i64, I64, I64]
        lib.oref_reorient.argtypes = [i, i64, i64, i64, i, i, v, v]
        lib.oref_dwconv3x3.argtypes = [i, i64, i64, i, i, i, D, D, D, D]
        lib.oref_dwconv3x3_bwd.argtypes = [i, i64, i64, i, i, i, D, D, D, D, D, D]
        lib.oref_num_threads.restype = i
        lib.oref_linear.argtypes = [i64, i64, i64, D, D, D, D]
        lib.oref_rmsnorm_modulate.argtypes = [i64, i64, i64, D, D, D, i64, d, D]
        lib.oref_gelu.argtypes = [i64, D, D]
        lib.oref_silu.argtypes = [i64, D, D]
        _lib = lib
    return _lib


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _p(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def num_threads() -> int:
    return int(_load().oref_num_threads())


# ----------------------------------------------------------------------------- gate
def logsigmoid(z: float) -> float:
    return float(_load().oref_logsigmoid(float(z)))


def gate_logalpha(z, tau: float):
    z = _f64(z)
    out = np.empty_like(z)
    _load().oref_gate_logalpha(z.size, _p(z), float(tau), _p(out))
    return out


# ----------------------------------------------------------------------- forward
def gla_recurrence(q, k, v, loga, q_scale: float = 1.0):
    """o_pre from the token-by-token recurrence, gate given as log(alpha) ([B,L,H,d_k])."""
    q, k, v, loga = map(_f64, (q, k, v, loga))
    B, L, H, dk = q.shape
    dv = v.shape[-1]
    o = np.empty((B, L, H, dv))
    _load().oref_gla_recurrence(B, L, H, dk, dv, _p(q), _p(k), _p(v), _p(loga),
                                float(q_scale), _p(o))
    return o


def output_stage(o_pre, r, gamma=None, eps: float = 1e-5):
    """(y, rstd): head-wise RMSNorm x gamma x Swish(r)."""
    o_pre, r = _f64(o_pre), _f64(r)
    B, L, H, dv = o_pre.shape
    g = None if gamma is None else _f64(gamma)
    y = np.empty_like(o_pre)
    rstd = np.empty((B, L, H))
    _load().oref_output_stage(B, L, H, dv, _p(o_pre), _p(r), _p(g), float(eps), _p(y), _p(rstd))
    return y, rstd


def gla_fwd(q, k, v, z, r, gamma=None, tau: float = 16.0, q_scale: float = 1.0,
            eps: float = 1e-5):
    """(y, o_pre, rstd) of the whole mixer forward with gate logits z."""
    q, k, v, z, r = map(_f64, (q, k, v, z, r))
    B, L, H, dk = q.shape
    dv = v.shape[-1]
    g = None if gamma is None else _f64(gamma)
    y = np.empty((B, L, H, dv))
    o = np.empty((B, L, H, dv))
    rstd = np.empty((B, L, H))
    _load().oref_gla_fwd(B, L, H, dk, dv, _p(q), _p(k), _p(v), _p(z), _p(r), _p(g),
                         float(tau), float(q_scale), float(eps), _p(y), _p(o), _p(rstd))
    return y, o, rstd


# ---------------------------------------------------------------------- backward
def gla_bwd_logalpha(q, k, v, loga, r, dy, gamma=None, q_scale: float = 1.0,
                     eps: float = 1e-5):
    """dict of dq, dk, dv, dloga, dr, dgamma for L = <dy, y>, gate given as log(alpha)."""
    q, k, v, loga, r, dy = map(_f64, (q, k, v, loga, r, dy))
    B, L, H, dk = q.shape
    dv = v.shape[-1]
    g = None if gamma is None else _f64(gamma)
    out = {n: np.empty_like(a) for n, a in (("dq", q), ("dk", k), ("dv", v), ("dloga", loga),
                                            ("dr", r))}
    out["dgamma"] = np.empty(dv)
    _load().oref_gla_bwd_logalpha(B, L, H, dk, dv, _p(q), _p(k), _p(v), _p(loga), _p(r), _p(g),
                                  float(q_scale), float(eps), _p(dy), _p(out["dq"]),
                                  _p(out["dk"]), _p(out["dv"]), _p(out["dloga"]), _p(out["dr"]),
                                  _p(out["dgamma"]))
    return out


def gla_bwd(q, k, v, z, r, dy, gamma=None, tau: float = 16.0, q_scale: float = 1.0,
            eps: float = 1e-5):
    """dict of dq, dk, dv, dz, dr, dgamma for L = <dy, y> with gate logits z."""
    q, k, v, z, r, dy = map(_f64, (q, k, v, z, r, dy))
    B, L, H, dk = q.shape
    dv = v.shape[-1]
    g = None if gamma is None else _f64(gamma)
    out = {n: np.empty_like(a) for n, a in (("dq", q), ("dk", k), ("dv", v), ("dz", z),
                                            ("dr", r))}
    out["dgamma"] = np.empty(dv)
    _load().oref_gla_bwd(B, L, H, dk, dv, _p(q), _p(k), _p(v), _p(z), _p(r), _p(g), float(tau),
                         float(q_scale), float(eps), _p(dy), _p(out["dq"]), _p(out["dk"]),
                         _p(out["dv"]), _p(out["dz"]), _p(out["dr"]), _p(out["dgamma"]))
    return out


# ---------------------------------------------------- value-side gate beta (eq. 5)
def gla_fwd_beta(q, k, v, z, w, r, gamma=None, tau: float = 16.0, q_scale: float = 1.0,
                 eps: float = 1e-5):
    """(y, o_pre, rstd) of the mixer forward with the outer-product gate G_t = alpha_t^T beta_t:
    key-gate logits z [B,L,H,d_k], value-gate logits w [B,L,H,d_v]."""
    q, k, v, z, w, r = map(_f64, (q, k, v, z, w, r))
    B, L, H, dk = q.shape
    dv = v.shape[-1]
    g = None if gamma is None else _f64(gamma)
    y = np.empty((B, L, H, dv))
    o = np.empty((B, L, H, dv))
    rstd = np.empty((B, L, H))
    _load().oref_gla_fwd_beta(B, L, H, dk, dv, _p(q), _p(k), _p(v), _p(z), _p(w), _p(r), _p(g),
                              float(tau), float(q_scale), float(eps), _p(y), _p(o), _p(rstd))
    return y, o, rstd


def gla_bwd_beta(q, k, v, z, w, r, dy, gamma=None, tau: float = 16.0, q_scale: float = 1.0,
                 eps: float = 1e-5):
    """dict of dq, dk, dv, dz, dw, dr, dgamma for L = <dy, y> of gla_fwd_beta."""
    q, k, v, z, w, r, dy = map(_f64, (q, k, v, z, w, r, dy))
    B, L, H, dk = q.shape
    dv = v.shape[-1]
    g = None if gamma is None else _f64(gamma)
    out = {n: np.empty_like(a) for n, a in (("dq", q), ("dk", k), ("dv", v), ("dz", z),
                                            ("dw", w), ("dr", r))}
    out["dgamma"] = np.empty(dv)
    _load().oref_gla_bwd_beta(B, L, H, dk, dv, _p(q), _p(k), _p(v), _p(z), _p(w), _p(r), _p(g),
                              float(tau), float(q_scale), float(eps), _p(dy), _p(out["dq"]),
                              _p(out["dk"]), _p(out["dv"]), _p(out["dz"]), _p(out["dw"]),
                              _p(out["dr"]), _p(out["dgamma"]))
    return out


# ------------------------------------------------------------------------- SREM
def scan_canonical(d: int, gh: int, gw: int, p: int) -> int:
    return int(_load().oref_scan_canonical(int(d), int(gh), int(gw), int(p)))


def scan_perm(d: int, gh: int, gw: int):
    """(perm, inv): perm[p] = canonical id at position p in order d; inv is its inverse."""
    L = gh * gw
    perm = np.empty(L, dtype=np.int64)
    inv = np.empty(L, dtype=np.int64)
    P = ctypes.POINTER(ctypes.c_int64)
    _load().oref_scan_perm(int(d), int(gh), int(gw), perm.ctypes.data_as(P), inv.ctypes.data_as(P))
    return perm, inv


def reorient(x: np.ndarray, gh: int, gw: int, frm: int, to: int) -> np.ndarray:
    """Exact byte gather of token rows; x is [B, L, D] of any fixed-size dtype."""
    x = np.ascontiguousarray(x)
    B, L, D = x.shape
    assert L == gh * gw
    y = np.empty_like(x)
    _load().oref_reorient(B, gh, gw, D * x.itemsize, int(frm), int(to),
                          x.ctypes.data_as(ctypes.c_void_p), y.ctypes.data_as(ctypes.c_void_p))
    return y


def dwconv3x3(x, w, gh: int, gw: int, layout: int, out_layout: int, bias=None):
    x, w = _f64(x), _f64(w)
    B, L, D = x.shape
    b = None if bias is None else _f64(bias)
    y = np.empty_like(x)
    _load().oref_dwconv3x3(B, gh, gw, D, int(layout), int(out_layout), _p(x), _p(w), _p(b), _p(y))
    return y


def dwconv3x3_bwd(x, w, dy, gh: int, gw: int, layout: int, out_layout: int):
    """(dx, dw, dbias) for L = <dy, dwconv3x3(x, w, bias)>."""
    x, w, dy = _f64(x), _f64(w), _f64(dy)
    B, L, D = x.shape
    dx = np.empty_like(x)
    dw = np.empty((D, 3, 3))
    db = np.empty(D)
    _load().oref_dwconv3x3_bwd(B, gh, gw, D, int(layout), int(out_layout), _p(x), _p(w), _p(dy),
                               _p(dx), _p(dw), _p(db))
    return dx, dw, db


# ------------------------------------------------------------------- projections
def linear(a, w, bias=None):
    """c = a w^T (+ bias): a [..., k], w [n, k] (out x in features), bias [n] or None."""
    a, w = _f64(a), _f64(w)
    k = a.shape[-1]
    m = a.size // k if k else 0
    n = w.shape[0]
    b = None if bias is None else _f64(bias)
    c = np.empty(a.shape[:-1] + (n,))
    _load().oref_linear(m, k, n, _p(a), _p(w), _p(b), _p(c))
    return c


def lowrank_gate_logits(factor, w, bias, heads: int, d_k: int):
    """Gate logits of the low-rank key gate (slides eq. (5): (x W_a1) W_a2 + b_alpha):
    z[b, t, h, c] = bias[h d_k + c] + sum_r factor[b, t, r] w[h d_k + c, r];
    factor [B, L, R], w [H d_k, R] (out x in features), bias [H d_k] or None -> [B, L, H, d_k]."""
    z = linear(factor, w, bias)
    return z.reshape(z.shape[:-1] + (heads, d_k))


# --------------------------------------------------------------------- DiG block
def rmsnorm_modulate(x, scale, shift, eps: float = 1e-5):
    """h = RMSNorm(x) * scale + shift over the last axis; x [B, L, D], scale/shift [B, D]."""
    x, scale, shift = _f64(x), _f64(scale), _f64(shift)
    B, L, D = x.shape
    h = np.empty_like(x)
    _load().oref_rmsnorm_modulate(B * L, D, max(L, 1), _p(x), _p(scale), _p(shift), D,
                                  float(eps), _p(h))
    return h


def gelu(x):
    x = _f64(x)
    y = np.empty_like(x)
    _load().oref_gelu(x.size, _p(x), _p(y))
    return y


def silu(x):
    x = _f64(x)
    y = np.empty_like(x)
    _load().oref_silu(x.size, _p(x), _p(y))
    return y


def block_cond(c, w_ada, b_ada=None):
    """adaLN parameters of every block: SiLU(c) W_ada^T + b_ada, c [B, D] -> [B, 6 D n]."""
    return linear(silu(c), w_ada, b_ada)


def block_forward(x, mod, wts: dict, gh: int, gw: int, heads: int, d_k: int, d_v: int,
                  layout: int, out_layout: int, tau: float = 16.0, eps: float = 1e-5,
                  intermediates: bool = False):
    """One DiG block forward (slides Figure 4; write-up section 3 "DiG Block"):
        x1 = x  + a1 * (GLA(RMSNorm(x) g1 + b1) W_out + b_out)
        x2 = x1 + a2 * (GELU((RMSNorm(x1) g2 + b2) W_ffn1 + b_ffn1) W_ffn2 + b_ffn2)
        x_out = DWConv3x3(x2) in scan order layout, written in out_layout (SREM)
    x [B, L, D] in scan order `layout`; mod [B, 6 D] = g1 | b1 | a1 | g2 | b2 | a2; wts holds
    the fields of dig_block_weights as float64 arrays (None for an absent bias).  The GLA
    layer: [q | k | v | u | r] = h W_in^T + b_in, z = u W_gate^T + b_gate, then gla_fwd."""
    x, mod = _f64(x), _f64(mod)
    B, L, D = x.shape
    HK, HV = heads * d_k, heads * d_v
    g1, b1, a1, g2, b2, a2 = (mod[:, i * D:(i + 1) * D] for i in range(6))
    h = rmsnorm_modulate(x, g1, b1, eps)
    proj = linear(h, wts["w_in"], wts.get("b_in"))
    cuts = np.cumsum([HK, HK, HV, proj.shape[-1] - 2 * HK - 2 * HV])
    q, k, v, u, r = np.split(proj, cuts, axis=-1)
    z = linear(u, wts["w_gate"], wts.get("b_gate"))
    shp = lambda t, d: t.reshape(B, L, heads, d)
    y, _, _ = gla_fwd(shp(q, d_k), shp(k, d_k), shp(v, d_v), shp(z, d_k), shp(r, d_v),
                      wts.get("gla_norm_w"), tau=tau, eps=eps)
    x1 = x + a1[:, None, :] * linear(y.reshape(B, L, HV), wts["w_out"], wts.get("b_out"))
    h2 = rmsnorm_modulate(x1, g2, b2, eps)
    f = linear(gelu(linear(h2, wts["w_ffn1"], wts.get("b_ffn1"))), wts["w_ffn2"],
               wts.get("b_ffn2"))
    x2 = x1 + a2[:, None, :] * f
    out = dwconv3x3(x2, wts["conv_w"], gh, gw, layout, out_layout, wts.get("conv_b"))
    if intermediates:
        return out, dict(h=h, q=q, k=k, v=v, u=u, r=r, z=z, y=y.reshape(B, L, HV), x1=x1, h2=h2,
                         x2=x2)
    return out
