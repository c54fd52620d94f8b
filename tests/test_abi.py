"""The C-ABI library loads, exports every symbol include/dig.h declares, and rejects bad
arguments on the host before touching the GPU (no compute calls here: CPU only)."""
import ctypes
import os
import re

import pytest

import diffusion_backbone_amd as dig

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dig.h")
BAD_PTR = 0x1000  # never dereferenced: every case below fails validation first


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dig_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    lib = dig.lib()
    declared = _declared()
    assert len(declared) >= 12
    for name in declared:
        assert hasattr(lib, name), name
    assert sorted(dig.EXPORTS) == declared
    assert dig.dig_abi_version() == 105


def test_status_strings():
    lib = dig.lib()
    for code, name in [(0, "DIG_OK"), (1, "DIG_ERR_NULL"), (2, "DIG_ERR_SHAPE"),
                       (3, "DIG_ERR_UNSUPPORTED"), (4, "DIG_ERR_WORKSPACE"), (5, "DIG_ERR_ALIAS"),
                       (6, "DIG_ERR_DEVICE"), (7, "DIG_ERR_ALIGN")]:
        assert lib.dig_status_str(code).decode() == name


def _desc(**kw):
    base = dict(batch=2, seq_len=256, heads=6, d_k=32, d_v=64, chunk=64)
    base.update(kw)
    return dig.make_desc(**base)


def _fwd(desc, q=BAD_PTR, ws=None, wsb=0, y=BAD_PTR + 0x100000000, saved=None):
    lib = dig.lib()
    P = BAD_PTR
    return lib.dig_gla_fwd(ctypes.byref(desc), q, P + 0x10000000, P + 0x20000000, P + 0x30000000,
                           P + 0x40000000, None, y, None, saved, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(batch=-1), dig.DIG_ERR_SHAPE),
    (dict(heads=0), dig.DIG_ERR_SHAPE),
    (dict(d_k=0), dig.DIG_ERR_SHAPE),
    (dict(d_k=65), dig.DIG_ERR_UNSUPPORTED),
    (dict(d_v=200), dig.DIG_ERR_UNSUPPORTED),
    (dict(chunk=48), dig.DIG_ERR_UNSUPPORTED),
    (dict(dtype=7), dig.DIG_ERR_UNSUPPORTED),
    (dict(tau=0.0), dig.DIG_ERR_SHAPE),
    (dict(tau=float("inf")), dig.DIG_ERR_SHAPE),
    (dict(norm_eps=-1.0), dig.DIG_ERR_SHAPE),
    (dict(seg_chunks=-2), dig.DIG_ERR_SHAPE),
])
def test_fwd_descriptor_errors(kw, code):
    d = _desc(**kw)
    assert _fwd(d) == code
    assert dig.lib().dig_last_error().decode() != ""
    assert dig.dig_gla_saved_bytes(d) == 0


def test_fwd_null_alias_align_workspace():
    d = _desc()
    assert _fwd(d, q=None) == dig.DIG_ERR_NULL
    assert _fwd(d, q=BAD_PTR + 8) == dig.DIG_ERR_ALIGN
    # y overlapping q (with the workspace this short sequence's look-back needs)
    nd = dig.dig_gla_fwd_workspace_bytes(d)
    assert nd > 0
    assert _fwd(d, y=BAD_PTR + 64, ws=BAD_PTR + 0x200000000, wsb=nd) == dig.DIG_ERR_ALIAS
    assert _fwd(d, ws=None) == dig.DIG_ERR_WORKSPACE
    # a long sequence needs a workspace for the cross-segment scan
    dl = _desc(batch=1, heads=6, seq_len=12544)
    need = dig.dig_gla_fwd_workspace_bytes(dl)
    assert need > 0
    assert _fwd(dl, ws=None) == dig.DIG_ERR_WORKSPACE
    assert _fwd(dl, ws=BAD_PTR + 0x200000000, wsb=need - 1) == dig.DIG_ERR_WORKSPACE
    # empty problems succeed without touching anything
    assert _fwd(_desc(batch=0), q=None) == dig.DIG_OK
    assert _fwd(_desc(seq_len=0), q=None) == dig.DIG_OK


def test_sizes_match_layout():
    d = _desc(batch=1, seq_len=1000, heads=16, d_k=36, d_v=72, chunk=64)
    nchunks = (1000 + 63) // 64
    a256 = lambda x: (x + 255) // 256 * 256
    states = 1 * 16 * nchunks * 36 * 72 * 4             # fp32 state entering each chunk
    obar = 1 * 16 * nchunks * 64 * 80 * 4               # normalised output (fp32), 16-wide d_v tiles
    rstd = 1 * 16 * nchunks * 64 * 4                    # per-row rsqrt(mean o^2 + eps)
    assert dig.dig_gla_saved_bytes(d) == a256(states) + a256(obar) + a256(rstd)
    assert dig.dig_gla_bwd_workspace_bytes(d) > 0


def test_bwd_errors():
    lib = dig.lib()
    d = _desc()
    P = BAD_PTR
    args = [P + i * 0x10000000 for i in range(13)]
    st = lib.dig_gla_bwd(ctypes.byref(d), *args[:7], None, *args[8:13], None, None, 0, None)
    assert st == dig.DIG_ERR_NULL  # saved missing
    st = lib.dig_gla_bwd(ctypes.byref(d), *args[:13], None, None, 0, None)
    assert st == dig.DIG_ERR_WORKSPACE


def test_srem_errors():
    lib = dig.lib()
    P = BAD_PTR
    assert lib.dig_srem_reorient(1, 4, 4, 8, 1, 0, 5, P, P + 0x100000, None) == dig.DIG_ERR_SHAPE
    assert lib.dig_srem_reorient(1, 4, 4, 8, 3, 0, 1, P, P + 0x100000, None) == dig.DIG_ERR_UNSUPPORTED
    assert lib.dig_srem_reorient(1, 4, 4, 8, 1, 0, 1, P, P + 64, None) == dig.DIG_ERR_ALIAS
    assert lib.dig_srem_reorient(1, 4, 4, 8, 1, 0, 1, None, P, None) == dig.DIG_ERR_NULL
    assert lib.dig_srem_reorient(1, 4, 4, 0, 1, 0, 1, P, P + 0x100000, None) == dig.DIG_ERR_SHAPE
    assert lib.dig_srem_reorient(0, 4, 4, 8, 1, 0, 1, None, None, None) == dig.DIG_OK
    assert lib.dig_dwconv3x3(1, 4, 4, 8, 1, 0, 1, P, None, None, P + 0x100000, None) == dig.DIG_ERR_NULL
    assert lib.dig_dwconv3x3(1, 4, 4, 8, 1, 0, 1, P + 2, P + 0x200000, None, P + 0x100000,
                             None) == dig.DIG_ERR_ALIGN
    need = dig.dig_dwconv3x3_bwd_workspace_bytes(1, 16, 16, 384)
    assert need > 0
    st = lib.dig_dwconv3x3_bwd(1, 16, 16, 384, 1, 0, 1, P, P + 0x1000000, P + 0x2000000,
                               P + 0x3000000, P + 0x4000000, None, None, 0, None)
    assert st == dig.DIG_ERR_WORKSPACE
