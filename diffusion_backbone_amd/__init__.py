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
    "dig_last_error", "dig_abi_version",
)


class DigError(RuntimeError):
    def __init__(self, status: int, func: str, detail: str):
        self.status = status
        super().__init__("%s failed: %s (%s)" % (func, _status_name(status), detail))


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
