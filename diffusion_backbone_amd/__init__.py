"""Python binding of libdig: the DiG gated-linear-attention mixer and SREM step on MI355X.

Argument marshalling only: every function forwards to the C entry point of the same name in
``libdig.so`` (declared in ``include/dig.h``), turning tensors into device pointers and the
current torch stream into a ``hipStream_t``.  All computation happens in the HIP kernels.
There is no fallback: if the library is missing, every call raises.

Tensors are torch tensors on the GPU (or raw integer device addresses); the caller allocates
every output and workspace buffer (the ``*_bytes`` queries give the sizes).
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdig.so")

DIG_OK, DIG_ERR_NULL, DIG_ERR_SHAPE, DIG_ERR_UNSUPPORTED = 0, 1, 2, 3
DIG_ERR_WORKSPACE, DIG_ERR_ALIAS, DIG_ERR_DEVICE, DIG_ERR_ALIGN = 4, 5, 6, 7
DIG_F32, DIG_BF16 = 0, 1
DIG_SCAN_ROW, DIG_SCAN_ROW_REV, DIG_SCAN_COL, DIG_SCAN_COL_REV = 0, 1, 2, 3

# Every symbol the header declares (checked by the CPU tests).
EXPORTS = (
    "dig_gla_saved_bytes", "dig_gla_fwd_workspace_bytes", "dig_gla_fwd",
    "dig_gla_bwd_workspace_bytes", "dig_gla_bwd", "dig_srem_reorient", "dig_dwconv3x3",
    "dig_dwconv3x3_bwd_workspace_bytes", "dig_dwconv3x3_bwd", "dig_status_str",
    "dig_last_error", "dig_abi_version", "dig_lookback_status", "dig_debug_lookback",
    "dig_dwconv3x3_bwd_noalloc", "dig_dwconv3x3_bwd_noalloc_max_bytes", "dig_linear",
    "dig_rmsnorm_modulate", "dig_block_cond_workspace_bytes", "dig_block_cond",
    "dig_block_fwd_workspace_bytes", "dig_block_fwd", "dig_linear_workspace_bytes",
    "dig_linear_ws", "dig_gla_fwd_lowrank", "dig_gla_bwd_lowrank", "dig_gla_beta_saved_bytes",
    "dig_gla_beta_fwd_workspace_bytes", "dig_gla_beta_bwd_workspace_bytes", "dig_gla_fwd_beta",
    "dig_gla_bwd_beta",
)
DIG_GATE_RANK = 16  # the rank of the low-rank key gate the chunk kernels form
DIG_LINEAR_MAX_OUT = 6
DIG_ACT_NONE, DIG_ACT_GELU = 0, 1


class DigError(RuntimeError):
    def __init__(self, status: int, func: str, detail: str):
        self.status = status
        super().__init__("%s failed: %s (%s)" % (func, _status_name(status), detail))


class dig_linear_out(ctypes.Structure):
    _fields_ = [("c", ctypes.c_void_p), ("w", ctypes.c_void_p), ("bias", ctypes.c_void_p),
                ("n", ctypes.c_int32), ("act", ctypes.c_int32), ("res", ctypes.c_void_p),
                ("gate", ctypes.c_void_p), ("gate_ld", ctypes.c_int64),
                ("rows_per_gate", ctypes.c_int64)]


class dig_block_desc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("grid_h", ctypes.c_int32), ("grid_w", ctypes.c_int32),
                ("dim", ctypes.c_int32), ("heads", ctypes.c_int32), ("d_k", ctypes.c_int32),
                ("d_v", ctypes.c_int32), ("gate_rank", ctypes.c_int32),
                ("ffn_dim", ctypes.c_int32), ("chunk", ctypes.c_int32), ("tau", ctypes.c_float),
                ("norm_eps", ctypes.c_float)]


class dig_block_weights(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in (
        "w_in", "b_in", "w_gate", "b_gate", "gla_norm_w", "w_out", "b_out", "w_ffn1", "b_ffn1",
        "w_ffn2", "b_ffn2", "conv_w", "conv_b")]


class dig_gla_desc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seq_len", ctypes.c_int32),
                ("heads", ctypes.c_int32), ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("chunk", ctypes.c_int32), ("tau", ctypes.c_float), ("q_scale", ctypes.c_float),
                ("norm_eps", ctypes.c_float), ("dtype", ctypes.c_int32),
                ("seg_chunks", ctypes.c_int32)]


def make_desc(batch, seq_len, heads, d_k, d_v, chunk=64, tau=16.0, q_scale=1.0,
              norm_eps=1e-5, dtype=DIG_BF16, seg_chunks=0) -> dig_gla_desc:
    if isinstance(dtype, str):
        dtype = {"bf16": DIG_BF16, "f32": DIG_F32}[dtype]
    return dig_gla_desc(batch, seq_len, heads, d_k, d_v, chunk, tau, q_scale, norm_eps, dtype,
                        seg_chunks)


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libdig.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libdig.so is not built (run `python -m diffusion_backbone_amd.build`)")
        L = ctypes.CDLL(LIB_PATH)
        P, S, I = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32
        D = ctypes.POINTER(dig_gla_desc)
        L.dig_gla_saved_bytes.argtypes = [D]
        L.dig_gla_saved_bytes.restype = S
        L.dig_gla_fwd_workspace_bytes.argtypes = [D]
        L.dig_gla_fwd_workspace_bytes.restype = S
        L.dig_gla_bwd_workspace_bytes.argtypes = [D]
        L.dig_gla_bwd_workspace_bytes.restype = S
        L.dig_gla_fwd.argtypes = [D, P, P, P, P, P, P, P, P, P, P, S, P]
        L.dig_gla_fwd.restype = ctypes.c_int
        L.dig_gla_bwd.argtypes = [D, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, S, P]
        L.dig_gla_bwd.restype = ctypes.c_int
        L.dig_gla_fwd_lowrank.argtypes = [D, P, P, P, P, P, P, I, P, P, P, P, P, P, S, P]
        L.dig_gla_fwd_lowrank.restype = ctypes.c_int
        L.dig_gla_bwd_lowrank.argtypes = [D, P, P, P, P, P, P, I, P, P, P, P, P, P, P, P, P, P,
                                          P, S, P]
        L.dig_gla_bwd_lowrank.restype = ctypes.c_int
        for n in ("dig_gla_beta_saved_bytes", "dig_gla_beta_fwd_workspace_bytes",
                  "dig_gla_beta_bwd_workspace_bytes"):
            getattr(L, n).argtypes = [D]
            getattr(L, n).restype = S
        L.dig_gla_fwd_beta.argtypes = [D, P, P, P, P, P, P, P, P, P, P, P, S, P]
        L.dig_gla_fwd_beta.restype = ctypes.c_int
        L.dig_gla_bwd_beta.argtypes = [D, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, S, P]
        L.dig_gla_bwd_beta.restype = ctypes.c_int
        L.dig_srem_reorient.argtypes = [I, I, I, I, I, I, I, P, P, P]
        L.dig_srem_reorient.restype = ctypes.c_int
        L.dig_dwconv3x3.argtypes = [I, I, I, I, I, I, I, P, P, P, P, P]
        L.dig_dwconv3x3.restype = ctypes.c_int
        L.dig_dwconv3x3_bwd_workspace_bytes.argtypes = [I, I, I, I]
        L.dig_dwconv3x3_bwd_workspace_bytes.restype = S
        L.dig_dwconv3x3_bwd.argtypes = [I, I, I, I, I, I, I, P, P, P, P, P, P, P, S, P]
        L.dig_dwconv3x3_bwd.restype = ctypes.c_int
        L.dig_status_str.argtypes = [ctypes.c_int]
        L.dig_status_str.restype = ctypes.c_char_p
        L.dig_last_error.argtypes = []
        L.dig_last_error.restype = ctypes.c_char_p
        L.dig_abi_version.restype = I
        L.dig_lookback_status.argtypes = [P]
        L.dig_lookback_status.restype = ctypes.c_int
        L.dig_debug_lookback.argtypes = [ctypes.c_uint32, I]
        L.dig_debug_lookback.restype = None
        L.dig_dwconv3x3_bwd_noalloc.argtypes = [I, I, I, I, I, I, I, P, P, P, P, P, P, P]
        L.dig_dwconv3x3_bwd_noalloc.restype = ctypes.c_int
        L.dig_dwconv3x3_bwd_noalloc_max_bytes.argtypes = []
        L.dig_dwconv3x3_bwd_noalloc_max_bytes.restype = S
        L.dig_linear.argtypes = [I, I, I, P, I, ctypes.POINTER(dig_linear_out), P]
        L.dig_linear.restype = ctypes.c_int
        L.dig_linear_workspace_bytes.argtypes = [I, I, I, ctypes.POINTER(dig_linear_out)]
        L.dig_linear_workspace_bytes.restype = S
        L.dig_linear_ws.argtypes = [I, I, I, P, I, ctypes.POINTER(dig_linear_out), P, S, P]
        L.dig_linear_ws.restype = ctypes.c_int
        I64, F = ctypes.c_int64, ctypes.c_float
        L.dig_rmsnorm_modulate.argtypes = [I64, I, I64, F, P, P, P, I64, P, P]
        L.dig_rmsnorm_modulate.restype = ctypes.c_int
        L.dig_block_cond_workspace_bytes.argtypes = [I, I]
        L.dig_block_cond_workspace_bytes.restype = S
        L.dig_block_cond.argtypes = [I, I, I, P, P, P, P, P, S, P]
        L.dig_block_cond.restype = ctypes.c_int
        BD = ctypes.POINTER(dig_block_desc)
        L.dig_block_fwd_workspace_bytes.argtypes = [BD]
        L.dig_block_fwd_workspace_bytes.restype = S
        L.dig_block_fwd.argtypes = [BD, ctypes.POINTER(dig_block_weights), P, I64, I, I, P, P, P,
                                    S, P]
        L.dig_block_fwd.restype = ctypes.c_int
        _lib = L
    return _lib


def _status_name(s: int) -> str:
    try:
        return lib().dig_status_str(s).decode()
    except Exception:  # library unavailable while formatting an error
        return str(s)


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("tensors passed to libdig must be contiguous")
    return t.data_ptr()


def _addr(t):
    """Device address of a tensor or view (no contiguity needed: strided-row arguments)."""
    if t is None or isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, func: str):
    if status != DIG_OK:
        raise DigError(status, func, lib().dig_last_error().decode())


def _nbytes(t, given):
    if given is not None:
        return given
    if t is None or isinstance(t, int):
        return 0
    return t.numel() * t.element_size()


# ------------------------------------------------------------------- queries
def dig_gla_saved_bytes(desc: dig_gla_desc) -> int:
    return lib().dig_gla_saved_bytes(ctypes.byref(desc))


def dig_gla_fwd_workspace_bytes(desc: dig_gla_desc) -> int:
    return lib().dig_gla_fwd_workspace_bytes(ctypes.byref(desc))


def dig_gla_bwd_workspace_bytes(desc: dig_gla_desc) -> int:
    return lib().dig_gla_bwd_workspace_bytes(ctypes.byref(desc))


def dig_dwconv3x3_bwd_workspace_bytes(batch, grid_h, grid_w, channels) -> int:
    return lib().dig_dwconv3x3_bwd_workspace_bytes(batch, grid_h, grid_w, channels)


# ------------------------------------------------------------------ compute
def dig_gla_fwd(desc, q, k, v, gate_logit, r, norm_w, y, o_pre=None, saved=None,
                workspace=None, workspace_bytes=None, stream=None):
    st = lib().dig_gla_fwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(gate_logit),
                           _ptr(r), _ptr(norm_w), _ptr(y), _ptr(o_pre), _ptr(saved),
                           _ptr(workspace), _nbytes(workspace, workspace_bytes), _stream(stream))
    _check(st, "dig_gla_fwd")


def dig_gla_bwd(desc, q, k, v, gate_logit, r, norm_w, dy, saved, dq, dk, dv, d_gate_logit, dr,
                d_norm_w=None, workspace=None, workspace_bytes=None, stream=None):
    st = lib().dig_gla_bwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(gate_logit),
                           _ptr(r), _ptr(norm_w), _ptr(dy), _ptr(saved), _ptr(dq), _ptr(dk),
                           _ptr(dv), _ptr(d_gate_logit), _ptr(dr), _ptr(d_norm_w),
                           _ptr(workspace), _nbytes(workspace, workspace_bytes), _stream(stream))
    _check(st, "dig_gla_bwd")


def dig_gla_fwd_lowrank(desc, q, k, v, gate_factor, gate_w, gate_bias, r, norm_w, y, o_pre=None,
                        saved=None, workspace=None, workspace_bytes=None, stream=None,
                        gate_rank=DIG_GATE_RANK):
    st = lib().dig_gla_fwd_lowrank(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v),
                                   _ptr(gate_factor), _ptr(gate_w), _ptr(gate_bias), gate_rank,
                                   _ptr(r), _ptr(norm_w), _ptr(y), _ptr(o_pre), _ptr(saved),
                                   _ptr(workspace), _nbytes(workspace, workspace_bytes),
                                   _stream(stream))
    _check(st, "dig_gla_fwd_lowrank")


def dig_gla_bwd_lowrank(desc, q, k, v, gate_factor, gate_w, gate_bias, r, norm_w, dy, saved, dq,
                        dk, dv, d_gate_logit, dr, d_norm_w=None, workspace=None,
                        workspace_bytes=None, stream=None, gate_rank=DIG_GATE_RANK):
    st = lib().dig_gla_bwd_lowrank(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v),
                                   _ptr(gate_factor), _ptr(gate_w), _ptr(gate_bias), gate_rank,
                                   _ptr(r), _ptr(norm_w), _ptr(dy), _ptr(saved), _ptr(dq),
                                   _ptr(dk), _ptr(dv), _ptr(d_gate_logit), _ptr(dr),
                                   _ptr(d_norm_w), _ptr(workspace),
                                   _nbytes(workspace, workspace_bytes), _stream(stream))
    _check(st, "dig_gla_bwd_lowrank")


def dig_gla_beta_saved_bytes(desc: dig_gla_desc) -> int:
    return lib().dig_gla_beta_saved_bytes(ctypes.byref(desc))


def dig_gla_beta_fwd_workspace_bytes(desc: dig_gla_desc) -> int:
    return lib().dig_gla_beta_fwd_workspace_bytes(ctypes.byref(desc))


def dig_gla_beta_bwd_workspace_bytes(desc: dig_gla_desc) -> int:
    return lib().dig_gla_beta_bwd_workspace_bytes(ctypes.byref(desc))


def dig_gla_fwd_beta(desc, q, k, v, gate_logit, value_gate_logit, r, norm_w, y, o_pre=None,
                     saved=None, workspace=None, workspace_bytes=None, stream=None):
    st = lib().dig_gla_fwd_beta(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(gate_logit),
                                _ptr(value_gate_logit), _ptr(r), _ptr(norm_w), _ptr(y),
                                _ptr(o_pre), _ptr(saved), _ptr(workspace),
                                _nbytes(workspace, workspace_bytes), _stream(stream))
    _check(st, "dig_gla_fwd_beta")


def dig_gla_bwd_beta(desc, q, k, v, gate_logit, value_gate_logit, r, norm_w, dy, saved, dq, dk,
                     dv, d_gate_logit, d_value_gate_logit, dr, d_norm_w=None, workspace=None,
                     workspace_bytes=None, stream=None):
    st = lib().dig_gla_bwd_beta(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(gate_logit),
                                _ptr(value_gate_logit), _ptr(r), _ptr(norm_w), _ptr(dy),
                                _ptr(saved), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(d_gate_logit),
                                _ptr(d_value_gate_logit), _ptr(dr), _ptr(d_norm_w),
                                _ptr(workspace), _nbytes(workspace, workspace_bytes),
                                _stream(stream))
    _check(st, "dig_gla_bwd_beta")


def dig_srem_reorient(batch, grid_h, grid_w, channels, dtype, frm, to, x, y, stream=None):
    st = lib().dig_srem_reorient(batch, grid_h, grid_w, channels, dtype, frm, to, _ptr(x), _ptr(y),
                                 _stream(stream))
    _check(st, "dig_srem_reorient")


def dig_dwconv3x3(batch, grid_h, grid_w, channels, dtype, layout, out_layout, x, w, bias, y,
                  stream=None):
    st = lib().dig_dwconv3x3(batch, grid_h, grid_w, channels, dtype, layout, out_layout, _ptr(x),
                             _ptr(w), _ptr(bias), _ptr(y), _stream(stream))
    _check(st, "dig_dwconv3x3")


def dig_dwconv3x3_bwd(batch, grid_h, grid_w, channels, dtype, layout, out_layout, x, w, dy, dx,
                      dw, dbias=None, workspace=None, workspace_bytes=None, stream=None):
    st = lib().dig_dwconv3x3_bwd(batch, grid_h, grid_w, channels, dtype, layout, out_layout,
                                 _ptr(x), _ptr(w), _ptr(dy), _ptr(dx), _ptr(dw), _ptr(dbias),
                                 _ptr(workspace), _nbytes(workspace, workspace_bytes),
                                 _stream(stream))
    _check(st, "dig_dwconv3x3_bwd")


def dig_abi_version() -> int:
    return lib().dig_abi_version()


def dig_lookback_status(stream=None):
    """Raises DigError(DIG_ERR_DEVICE) if a look-back wait gave up since the last query."""
    _check(lib().dig_lookback_status(_stream(stream)), "dig_lookback_status")


def dig_debug_lookback(spins: int, never_match: bool):
    lib().dig_debug_lookback(int(spins), 1 if never_match else 0)


def dig_dwconv3x3_bwd_noalloc(batch, grid_h, grid_w, channels, dtype, layout, out_layout, x, w,
                              dy, dx, dw, dbias=None, stream=None):
    st = lib().dig_dwconv3x3_bwd_noalloc(batch, grid_h, grid_w, channels, dtype, layout,
                                         out_layout, _ptr(x), _ptr(w), _ptr(dy), _ptr(dx),
                                         _ptr(dw), _ptr(dbias), _stream(stream))
    _check(st, "dig_dwconv3x3_bwd_noalloc")


def dig_dwconv3x3_bwd_noalloc_max_bytes() -> int:
    return lib().dig_dwconv3x3_bwd_noalloc_max_bytes()



def linear_out(c, w, bias=None, act=DIG_ACT_NONE, res=None, gate=None, gate_ld=0,
               rows_per_gate=1, n=None) -> dict:
    """One output of dig_linear.  gate: tensor view or address of gate row 0."""
    return dict(c=c, w=w, bias=bias, act=act, res=res, gate=gate, gate_ld=gate_ld,
                rows_per_gate=rows_per_gate, n=n)


def _linear_outs(outs):
    arr = (dig_linear_out * max(len(outs), 1))()
    for i, o in enumerate(outs):
        if not isinstance(o, dict):
            o = linear_out(*o)
        n = o["n"] if o["n"] is not None else int(o["w"].shape[0])
        arr[i] = dig_linear_out(_ptr(o["c"]), _ptr(o["w"]), _ptr(o["bias"]), n, int(o["act"]),
                                _ptr(o["res"]), _addr(o["gate"]), int(o["gate_ld"]),
                                int(o["rows_per_gate"]))
    return arr


def dig_linear(m, k, a, outs, stream=None):
    """outs: sequence of (c, w, bias_or_None) tuples or linear_out(...) dicts;
    c [m, n] bf16, w [n, k] bf16."""
    st = lib().dig_linear(int(m), int(k), DIG_BF16, _ptr(a), len(outs), _linear_outs(outs),
                          _stream(stream))
    _check(st, "dig_linear")


def dig_linear_workspace_bytes(m, k, outs) -> int:
    return lib().dig_linear_workspace_bytes(int(m), int(k), len(outs), _linear_outs(outs))


def dig_linear_ws(m, k, a, outs, workspace, workspace_bytes=None, stream=None):
    st = lib().dig_linear_ws(int(m), int(k), DIG_BF16, _ptr(a), len(outs), _linear_outs(outs),
                             _ptr(workspace), _nbytes(workspace, workspace_bytes),
                             _stream(stream))
    _check(st, "dig_linear_ws")


# ---------------------------------------------------------------- DiG block
def dig_rmsnorm_modulate(rows, dim, rows_per_group, eps, x, scale, shift, mod_ld, h,
                         stream=None):
    """scale, shift: tensor views or addresses of row 0 (rows mod_ld elements apart)."""
    st = lib().dig_rmsnorm_modulate(int(rows), int(dim), int(rows_per_group), float(eps), _ptr(x),
                                    _addr(scale), _addr(shift), int(mod_ld), _ptr(h),
                                    _stream(stream))
    _check(st, "dig_rmsnorm_modulate")


def make_block_desc(batch, grid_h, grid_w, dim, heads, d_k, d_v, gate_rank=16, ffn_dim=None,
                    chunk=64, tau=16.0, norm_eps=1e-5) -> dig_block_desc:
    return dig_block_desc(batch, grid_h, grid_w, dim, heads, d_k, d_v, gate_rank,
                          4 * dim if ffn_dim is None else ffn_dim, chunk, tau, norm_eps)


def make_block_weights(**tensors) -> dig_block_weights:
    """Keyword arguments named as the fields of dig_block_weights (tensors or None)."""
    unknown = set(tensors) - {f for f, _ in dig_block_weights._fields_}
    if unknown:
        raise ValueError("unknown block weights: %s" % sorted(unknown))
    return dig_block_weights(*[_ptr(tensors.get(f)) for f, _ in dig_block_weights._fields_])


def dig_block_cond_workspace_bytes(batch, dim) -> int:
    return lib().dig_block_cond_workspace_bytes(int(batch), int(dim))


def dig_block_cond(batch, dim, n_blocks, c, w_ada, b_ada, mod, workspace, workspace_bytes=None,
                   stream=None):
    st = lib().dig_block_cond(int(batch), int(dim), int(n_blocks), _ptr(c), _ptr(w_ada),
                              _ptr(b_ada), _ptr(mod), _ptr(workspace),
                              _nbytes(workspace, workspace_bytes), _stream(stream))
    _check(st, "dig_block_cond")


def dig_block_fwd_workspace_bytes(desc: dig_block_desc) -> int:
    return lib().dig_block_fwd_workspace_bytes(ctypes.byref(desc))


def dig_block_fwd(desc, weights, mod, mod_ld, layout, out_layout, x, x_out, workspace,
                  workspace_bytes=None, stream=None):
    """mod: tensor view or address of this block's parameters for image 0."""
    st = lib().dig_block_fwd(ctypes.byref(desc), ctypes.byref(weights), _addr(mod), int(mod_ld),
                             int(layout), int(out_layout), _ptr(x), _ptr(x_out), _ptr(workspace),
                             _nbytes(workspace, workspace_bytes), _stream(stream))
    _check(st, "dig_block_fwd")
