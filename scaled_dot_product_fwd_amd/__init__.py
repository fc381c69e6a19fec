"""Fused masked multi-head attention forward for AMD Instinct MI355X (gfx950).

A thin ctypes binding over ``libattn.so`` (C ABI declared in ``include/attn.h``). Every step of
the computation runs in the library's HIP kernels; this module only marshals arguments. There is
no fallback: if the library is missing, calls raise ``ImportError``.

Raw entry points (same names and argument order as the C ABI; pointers are integers, stride
arguments are 3-sequences of element strides or None):
    attn_fwd, attn_fwd_validate, attn_fwd_strided, attn_fwd_strided_validate,
    attn_fwd_masked, attn_fwd_masked_validate, attn_bwd, attn_bwd_validate, attn_bwd_strided,
    attn_bwd_strided_validate, attn_bwd_masked, attn_bwd_masked_validate,
    attn_status_string, attn_version
Convenience for torch tensors (device memory and streams only):
    forward(q, k, v, causal=..., valid_len=None, scale=None, out=None, lse=None, layout="bhnd",
            attn_mask=None)
    backward(q, k, v, out, dout, lse, causal=..., valid_len=None, scale=None)
    attention(q, k, v, causal=..., valid_len=None, scale=None)   # torch autograd Function
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

__all__ = ["ATTN_F16", "ATTN_BF16", "ATTN_F32", "AttnError", "attn_fwd", "attn_fwd_validate",
           "attn_fwd_strided", "attn_fwd_strided_validate", "attn_fwd_masked",
           "attn_fwd_masked_validate", "attn_fwd_ws", "attn_fwd_ws_validate",
           "attn_fwd_workspace_floats", "attn_bwd", "attn_bwd_validate", "attn_bwd_strided",
           "attn_bwd_strided_validate", "attn_bwd_masked", "attn_bwd_masked_validate",
           "attn_bwd_ws", "attn_bwd_ws_validate", "attn_bwd_workspace_floats",
           "attn_bwd_scratch", "ATTN_SCRATCH_FLOATS", "attention",
           "backward", "attn_status_string",
           "attn_version", "forward", "library_path", "load_library"]

ATTN_F16 = 0
ATTN_BF16 = 1
ATTN_F32 = 2

ATTN_OK = 0
ATTN_ERR_NULL = -1
ATTN_ERR_SHAPE = -2
ATTN_ERR_HEAD_DIM = -3
ATTN_ERR_DTYPE = -4
ATTN_ERR_SCALE = -5
ATTN_ERR_LAUNCH = -6
ATTN_ERR_ALIAS = -7
ATTN_ERR_LAYOUT = -8
ATTN_ERR_MASK = -9
ATTN_ERR_WORKSPACE = -10
ATTN_ERR_SCRATCH = -11

ATTN_SCRATCH_FLOATS = 1 << 23   # float32 values of attn_bwd_scratch's static device workspace

ATTN_MASK_NONE = 0
ATTN_MASK_KEEP_U8 = 1
ATTN_MASK_ADD = 2

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libattn.so")
_lib: Optional[ctypes.CDLL] = None

_c_int, _c_float, _vp = ctypes.c_int, ctypes.c_float, ctypes.c_void_p
_i64p = ctypes.POINTER(ctypes.c_int64)


class AttnError(RuntimeError):
    def __init__(self, status: int, where: str = "attn_fwd"):
        self.status = status
        super().__init__("%s failed with status %d: %s" % (where, status,
                                                          attn_status_string(status)))


def library_path() -> str:
    return _LIB_PATH


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libattn.so (once). Raises ImportError if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or _LIB_PATH
    if not os.path.exists(p):
        raise ImportError("libattn.so not found at %s; build it with "
                          "`python -m scaled_dot_product_fwd_amd.build`" % p)
    lib = ctypes.CDLL(p)
    lib.attn_fwd.restype = _c_int
    lib.attn_fwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int,
                             _c_float, _c_int, _vp, _c_int, _vp]
    lib.attn_fwd_validate.restype = _c_int
    lib.attn_fwd_validate.argtypes = [_vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int,
                                      _c_int, _c_float, _c_int, _vp, _c_int]
    lib.attn_fwd_strided.restype = _c_int
    lib.attn_fwd_strided.argtypes = [_vp, _i64p, _vp, _i64p, _vp, _i64p, _vp, _i64p, _vp, _c_int,
                                     _c_int, _c_int, _c_int, _c_int, _c_float, _c_int, _vp,
                                     _c_int, _vp]
    lib.attn_fwd_strided_validate.restype = _c_int
    lib.attn_fwd_strided_validate.argtypes = [_vp, _i64p, _vp, _i64p, _vp, _i64p, _vp, _i64p,
                                              _vp, _c_int, _c_int, _c_int, _c_int, _c_int,
                                              _c_float, _c_int, _vp, _c_int]
    lib.attn_fwd_masked.restype = _c_int
    lib.attn_fwd_masked.argtypes = [_vp, _i64p, _vp, _i64p, _vp, _i64p, _vp, _i64p, _vp, _c_int,
                                    _c_int, _c_int, _c_int, _c_int, _c_float, _c_int, _vp, _vp,
                                    _c_int, _i64p, _c_int, _vp]
    lib.attn_fwd_masked_validate.restype = _c_int
    lib.attn_fwd_masked_validate.argtypes = [_vp, _i64p, _vp, _i64p, _vp, _i64p, _vp, _i64p,
                                             _vp, _c_int, _c_int, _c_int, _c_int, _c_int,
                                             _c_float, _c_int, _vp, _vp, _c_int, _i64p, _c_int]
    lib.attn_fwd_ws.restype = _c_int
    lib.attn_fwd_ws.argtypes = ([_vp, _i64p] * 4 + [_vp, _vp, ctypes.c_int64] + [_c_int] * 5 +
                                [_c_float, _c_int, _vp, _c_int, _vp])
    lib.attn_fwd_ws_validate.restype = _c_int
    lib.attn_fwd_ws_validate.argtypes = ([_vp, _i64p] * 4 + [_vp, _vp, ctypes.c_int64] +
                                         [_c_int] * 5 + [_c_float, _c_int, _vp, _c_int])
    lib.attn_fwd_workspace_floats.restype = ctypes.c_int64
    lib.attn_fwd_workspace_floats.argtypes = [_c_int] * 6
    lib.attn_bwd.restype = _c_int
    lib.attn_bwd.argtypes = [_vp] * 10 + [_c_int] * 5 + [_c_float, _c_int, _vp, _c_int, _vp]
    lib.attn_bwd_validate.restype = _c_int
    lib.attn_bwd_validate.argtypes = [_vp] * 10 + [_c_int] * 5 + [_c_float, _c_int, _vp, _c_int]
    lib.attn_bwd_strided.restype = _c_int
    lib.attn_bwd_strided.argtypes = ([_vp, _i64p] * 5 + [_vp] + [_vp, _i64p] * 3 + [_vp] +
                                     [_c_int] * 5 + [_c_float, _c_int, _vp, _c_int, _vp])
    lib.attn_bwd_strided_validate.restype = _c_int
    lib.attn_bwd_strided_validate.argtypes = ([_vp, _i64p] * 5 + [_vp] + [_vp, _i64p] * 3 +
                                              [_vp] + [_c_int] * 5 + [_c_float, _c_int, _vp,
                                                                      _c_int])
    lib.attn_bwd_masked.restype = _c_int
    lib.attn_bwd_masked.argtypes = ([_vp, _i64p] * 5 + [_vp] + [_vp, _i64p] * 3 + [_vp] +
                                    [_c_int] * 5 + [_c_float, _c_int, _vp, _vp, _c_int, _i64p,
                                                    _c_int, _vp])
    lib.attn_bwd_masked_validate.restype = _c_int
    lib.attn_bwd_masked_validate.argtypes = ([_vp, _i64p] * 5 + [_vp] + [_vp, _i64p] * 3 +
                                             [_vp] + [_c_int] * 5 + [_c_float, _c_int, _vp, _vp,
                                                                     _c_int, _i64p, _c_int])
    lib.attn_bwd_ws.restype = _c_int
    lib.attn_bwd_ws.argtypes = ([_vp, _i64p] * 5 + [_vp] + [_vp, _i64p] * 3 + [_vp, ctypes.c_int64]
                                + [_c_int] * 5 + [_c_float, _c_int, _vp, _vp, _c_int, _i64p,
                                                  _c_int, _vp])
    lib.attn_bwd_ws_validate.restype = _c_int
    lib.attn_bwd_ws_validate.argtypes = ([_vp, _i64p] * 5 + [_vp] + [_vp, _i64p] * 3 +
                                         [_vp, ctypes.c_int64] + [_c_int] * 5 +
                                         [_c_float, _c_int, _vp, _vp, _c_int, _i64p, _c_int])
    lib.attn_bwd_scratch.restype = _c_int
    lib.attn_bwd_scratch.argtypes = ([_vp, _i64p] * 5 + [_vp] + [_vp, _i64p] * 3 + [_c_int] * 5
                                     + [_c_float, _c_int, _vp, _vp, _c_int, _i64p, _c_int, _vp])
    lib.attn_bwd_workspace_floats.restype = ctypes.c_int64
    lib.attn_bwd_workspace_floats.argtypes = [_c_int] * 5
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_status_string.argtypes = [_c_int]
    lib.attn_version.restype = _c_int
    lib.attn_version.argtypes = []
    if path is None:
        _lib = lib
    return lib


def attn_fwd(q: int, k: int, v: int, out: int, lse: Optional[int], B: int, Hq: int, Hkv: int,
             N: int, D: int, scale: float, causal: int, valid_len: Optional[int], dtype: int,
             stream: Optional[int]) -> int:
    """C ``attn_fwd``; pointers are device addresses as integers (None for NULL)."""
    return load_library().attn_fwd(q, k, v, out, lse, B, Hq, Hkv, N, D, scale, int(causal),
                                   valid_len, dtype, stream)


def attn_fwd_validate(q: int, k: int, v: int, out: int, lse: Optional[int], B: int, Hq: int,
                      Hkv: int, N: int, D: int, scale: float, causal: int,
                      valid_len: Optional[int], dtype: int) -> int:
    """C ``attn_fwd_validate``: host-only argument check, no HIP call."""
    return load_library().attn_fwd_validate(q, k, v, out, lse, B, Hq, Hkv, N, D, scale,
                                            int(causal), valid_len, dtype)


def _strides(st):
    if st is None:
        return None
    st = tuple(int(x) for x in st)
    if len(st) != 3:
        raise ValueError("a stride argument has three entries (batch, head, row)")
    return (ctypes.c_int64 * 3)(*st)


def attn_fwd_strided(q: int, q_strides, k: int, k_strides, v: int, v_strides, out: int,
                     out_strides, lse: Optional[int], B: int, Hq: int, Hkv: int, N: int, D: int,
                     scale: float, causal: int, valid_len: Optional[int], dtype: int,
                     stream: Optional[int]) -> int:
    """C ``attn_fwd_strided``; strides are (batch, head, row) element strides or None."""
    return load_library().attn_fwd_strided(q, _strides(q_strides), k, _strides(k_strides), v,
                                           _strides(v_strides), out, _strides(out_strides), lse,
                                           B, Hq, Hkv, N, D, scale, int(causal), valid_len,
                                           dtype, stream)


def attn_fwd_strided_validate(q: int, q_strides, k: int, k_strides, v: int, v_strides, out: int,
                              out_strides, lse: Optional[int], B: int, Hq: int, Hkv: int,
                              N: int, D: int, scale: float, causal: int,
                              valid_len: Optional[int], dtype: int) -> int:
    """C ``attn_fwd_strided_validate``: host-only argument check, no HIP call."""
    return load_library().attn_fwd_strided_validate(
        q, _strides(q_strides), k, _strides(k_strides), v, _strides(v_strides), out,
        _strides(out_strides), lse, B, Hq, Hkv, N, D, scale, int(causal), valid_len, dtype)


def attn_fwd_masked(q: int, q_strides, k: int, k_strides, v: int, v_strides, out: int,
                    out_strides, lse: Optional[int], B: int, Hq: int, Hkv: int, N: int, D: int,
                    scale: float, causal: int, valid_len: Optional[int], mask: Optional[int],
                    mask_type: int, mask_strides, dtype: int, stream: Optional[int]) -> int:
    """C ``attn_fwd_masked``; mask_strides are (batch, head, row) element strides or None."""
    return load_library().attn_fwd_masked(
        q, _strides(q_strides), k, _strides(k_strides), v, _strides(v_strides), out,
        _strides(out_strides), lse, B, Hq, Hkv, N, D, scale, int(causal), valid_len, mask,
        mask_type, _strides(mask_strides), dtype, stream)


def attn_fwd_masked_validate(q: int, q_strides, k: int, k_strides, v: int, v_strides, out: int,
                             out_strides, lse: Optional[int], B: int, Hq: int, Hkv: int, N: int,
                             D: int, scale: float, causal: int, valid_len: Optional[int],
                             mask: Optional[int], mask_type: int, mask_strides,
                             dtype: int) -> int:
    """C ``attn_fwd_masked_validate``: host-only argument check, no HIP call."""
    return load_library().attn_fwd_masked_validate(
        q, _strides(q_strides), k, _strides(k_strides), v, _strides(v_strides), out,
        _strides(out_strides), lse, B, Hq, Hkv, N, D, scale, int(causal), valid_len, mask,
        mask_type, _strides(mask_strides), dtype)


def attn_fwd_ws(q: int, q_strides, k: int, k_strides, v: int, v_strides, out: int, out_strides,
                lse: Optional[int], ws: Optional[int], ws_floats: int, B: int, Hq: int, Hkv: int,
                N: int, D: int, scale: float, causal: bool, valid_len: Optional[int], dtype: int,
                stream: Optional[int]) -> int:
    """C ``attn_fwd_ws``; pointers as integers, strides as 3-sequences or None."""
    return load_library().attn_fwd_ws(
        q, _strides(q_strides), k, _strides(k_strides), v, _strides(v_strides), out,
        _strides(out_strides), lse, ws, ws_floats, B, Hq, Hkv, N, D, scale, int(causal),
        valid_len, dtype, stream)


def attn_fwd_ws_validate(q: int, q_strides, k: int, k_strides, v: int, v_strides, out: int,
                         out_strides, lse: Optional[int], ws: Optional[int], ws_floats: int,
                         B: int, Hq: int, Hkv: int, N: int, D: int, scale: float, causal: bool,
                         valid_len: Optional[int], dtype: int) -> int:
    """C ``attn_fwd_ws_validate``: host-only argument check, no HIP call."""
    return load_library().attn_fwd_ws_validate(
        q, _strides(q_strides), k, _strides(k_strides), v, _strides(v_strides), out,
        _strides(out_strides), lse, ws, ws_floats, B, Hq, Hkv, N, D, scale, int(causal),
        valid_len, dtype)


def attn_fwd_workspace_floats(B: int, Hq: int, Hkv: int, N: int, D: int, causal: bool) -> int:
    """C ``attn_fwd_workspace_floats``: float32 values of the workspace attn_fwd_ws splits with
    (0: these sizes fill the device, no split)."""
    return load_library().attn_fwd_workspace_floats(B, Hq, Hkv, N, D, int(bool(causal)))


def attn_bwd(q: int, k: int, v: int, out: int, dout: int, lse: int, dq: int, dk: int, dv: int,
             ws: int, B: int, Hq: int, Hkv: int, N: int, D: int, scale: float, causal: int,
             valid_len: Optional[int], dtype: int, stream: Optional[int]) -> int:
    """C ``attn_bwd``; pointers are device addresses as integers."""
    return load_library().attn_bwd(q, k, v, out, dout, lse, dq, dk, dv, ws, B, Hq, Hkv, N, D,
                                   scale, int(causal), valid_len, dtype, stream)


def attn_bwd_validate(q: int, k: int, v: int, out: int, dout: int, lse: int, dq: int, dk: int,
                      dv: int, ws: int, B: int, Hq: int, Hkv: int, N: int, D: int,
                      scale: float, causal: int, valid_len: Optional[int], dtype: int) -> int:
    """C ``attn_bwd_validate``: host-only argument check, no HIP call."""
    return load_library().attn_bwd_validate(q, k, v, out, dout, lse, dq, dk, dv, ws, B, Hq,
                                            Hkv, N, D, scale, int(causal), valid_len, dtype)


def attn_bwd_strided(q, q_strides, k, k_strides, v, v_strides, out, out_strides, dout,
                     dout_strides, lse, dq, dq_strides, dk, dk_strides, dv, dv_strides, ws, B, Hq,
                     Hkv, N, D, scale, causal, valid_len, dtype, stream) -> int:
    """C ``attn_bwd_strided``; pointers as integers, strides as 3-sequences or None."""
    return load_library().attn_bwd_strided(
        q, _strides(q_strides), k, _strides(k_strides), v, _strides(v_strides), out,
        _strides(out_strides), dout, _strides(dout_strides), lse, dq, _strides(dq_strides), dk,
        _strides(dk_strides), dv, _strides(dv_strides), ws, B, Hq, Hkv, N, D, scale, int(causal),
        valid_len, dtype, stream)


def attn_bwd_strided_validate(q, q_strides, k, k_strides, v, v_strides, out, out_strides, dout,
                              dout_strides, lse, dq, dq_strides, dk, dk_strides, dv, dv_strides,
                              ws, B, Hq, Hkv, N, D, scale, causal, valid_len, dtype) -> int:
    """C ``attn_bwd_strided_validate``: host-only argument check, no HIP call."""
    return load_library().attn_bwd_strided_validate(
        q, _strides(q_strides), k, _strides(k_strides), v, _strides(v_strides), out,
        _strides(out_strides), dout, _strides(dout_strides), lse, dq, _strides(dq_strides), dk,
        _strides(dk_strides), dv, _strides(dv_strides), ws, B, Hq, Hkv, N, D, scale, int(causal),
        valid_len, dtype)


def attn_bwd_masked(q, q_strides, k, k_strides, v, v_strides, out, out_strides, dout,
                    dout_strides, lse, dq, dq_strides, dk, dk_strides, dv, dv_strides, ws, B, Hq,
                    Hkv, N, D, scale, causal, valid_len, mask, mask_type, mask_strides, dtype,
                    stream) -> int:
    """C ``attn_bwd_masked``; pointers as integers, strides as 3-sequences or None."""
    return load_library().attn_bwd_masked(
        q, _strides(q_strides), k, _strides(k_strides), v, _strides(v_strides), out,
        _strides(out_strides), dout, _strides(dout_strides), lse, dq, _strides(dq_strides), dk,
        _strides(dk_strides), dv, _strides(dv_strides), ws, B, Hq, Hkv, N, D, scale, int(causal),
        valid_len, mask, mask_type, _strides(mask_strides), dtype, stream)


def attn_bwd_masked_validate(q, q_strides, k, k_strides, v, v_strides, out, out_strides, dout,
                             dout_strides, lse, dq, dq_strides, dk, dk_strides, dv, dv_strides,
                             ws, B, Hq, Hkv, N, D, scale, causal, valid_len, mask, mask_type,
                             mask_strides, dtype) -> int:
    """C ``attn_bwd_masked_validate``: host-only argument check, no HIP call."""
    return load_library().attn_bwd_masked_validate(
        q, _strides(q_strides), k, _strides(k_strides), v, _strides(v_strides), out,
        _strides(out_strides), dout, _strides(dout_strides), lse, dq, _strides(dq_strides), dk,
        _strides(dk_strides), dv, _strides(dv_strides), ws, B, Hq, Hkv, N, D, scale, int(causal),
        valid_len, mask, mask_type, _strides(mask_strides), dtype)


def attn_bwd_ws(q, q_strides, k, k_strides, v, v_strides, out, out_strides, dout, dout_strides,
                lse, dq, dq_strides, dk, dk_strides, dv, dv_strides, ws, ws_floats, B, Hq, Hkv, N,
                D, scale, causal, valid_len, mask, mask_type, mask_strides, dtype,
                stream) -> int:
    """C ``attn_bwd_ws``; pointers as integers, strides as 3-sequences or None."""
    return load_library().attn_bwd_ws(
        q, _strides(q_strides), k, _strides(k_strides), v, _strides(v_strides), out,
        _strides(out_strides), dout, _strides(dout_strides), lse, dq, _strides(dq_strides), dk,
        _strides(dk_strides), dv, _strides(dv_strides), ws, ws_floats, B, Hq, Hkv, N, D, scale,
        int(causal), valid_len, mask, mask_type, _strides(mask_strides), dtype, stream)


def attn_bwd_ws_validate(q, q_strides, k, k_strides, v, v_strides, out, out_strides, dout,
                         dout_strides, lse, dq, dq_strides, dk, dk_strides, dv, dv_strides, ws,
                         ws_floats, B, Hq, Hkv, N, D, scale, causal, valid_len, mask, mask_type,
                         mask_strides, dtype) -> int:
    """C ``attn_bwd_ws_validate``: host-only argument check, no HIP call."""
    return load_library().attn_bwd_ws_validate(
        q, _strides(q_strides), k, _strides(k_strides), v, _strides(v_strides), out,
        _strides(out_strides), dout, _strides(dout_strides), lse, dq, _strides(dq_strides), dk,
        _strides(dk_strides), dv, _strides(dv_strides), ws, ws_floats, B, Hq, Hkv, N, D, scale,
        int(causal), valid_len, mask, mask_type, _strides(mask_strides), dtype)


def attn_bwd_scratch(q, q_strides, k, k_strides, v, v_strides, out, out_strides, dout,
                     dout_strides, lse, dq, dq_strides, dk, dk_strides, dv, dv_strides, B, Hq,
                     Hkv, N, D, scale, causal, valid_len, mask, mask_type, mask_strides, dtype,
                     stream) -> int:
    """C ``attn_bwd_scratch``: attn_bwd_ws on the library's static device workspace (no
    allocation); pointers as integers, strides as 3-sequences or None."""
    return load_library().attn_bwd_scratch(
        q, _strides(q_strides), k, _strides(k_strides), v, _strides(v_strides), out,
        _strides(out_strides), dout, _strides(dout_strides), lse, dq, _strides(dq_strides), dk,
        _strides(dk_strides), dv, _strides(dv_strides), B, Hq, Hkv, N, D, scale, int(causal),
        valid_len, mask, mask_type, _strides(mask_strides), dtype, stream)


def attn_bwd_workspace_floats(B: int, Hq: int, Hkv: int, N: int, D: int) -> int:
    """C ``attn_bwd_workspace_floats``: float32 values of the workspace attn_bwd_ws splits with."""
    return load_library().attn_bwd_workspace_floats(B, Hq, Hkv, N, D)


def attn_status_string(status: int) -> str:
    return load_library().attn_status_string(status).decode()


def attn_version() -> int:
    return load_library().attn_version()


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.float16:
        return ATTN_F16
    if t.dtype == torch.float32:
        return ATTN_F32
    raise TypeError("q/k/v must be float16, bfloat16 or float32, got %s" % t.dtype)


def _mask_view(attn_mask, dtype, B, Hq, N):
    """(a [B, Hq, N, N] view of attn_mask, its attn_mask_t): bool / uint8 keep masks, masks of
    the inputs' dtype are additive; 2-D and 3-D masks broadcast over batch and heads."""
    import torch
    m = attn_mask
    if m.dtype == torch.bool:
        m = m.view(torch.uint8)
    if m.dtype == torch.uint8:
        mtype = ATTN_MASK_KEEP_U8
    elif m.dtype == dtype:
        mtype = ATTN_MASK_ADD
    else:
        raise TypeError("attn_mask must be bool, uint8 or q's dtype, got %s" % m.dtype)
    if not m.is_cuda:
        raise ValueError("attn_mask must be a device tensor")
    if m.dim() == 3:
        m = m[:, None]
    elif m.dim() == 2:
        m = m[None, None]
    if m.dim() != 4 or tuple(m.shape[-2:]) != (N, N):
        raise ValueError("attn_mask must be broadcastable to [B, Hq, N, N]")
    m = m.expand(B, Hq, N, N)
    if m.stride(3) != 1:
        raise ValueError("attn_mask: the key dimension must be contiguous")
    return m, mtype


def forward(q, k, v, causal: bool, valid_len=None, scale: Optional[float] = None, out=None,
            lse=None, want_lse: bool = True, stream=None, layout: str = "bhnd",
            attn_mask=None, ws=None, split: bool = True) -> Tuple[object, Optional[object]]:
    """Run the attention forward on torch device tensors on the current (or given) stream.

    ``layout`` names the order of the four dimensions of q, k, v and out: "bhnd" for
    [B, H, N, D] (the default) or "bnhd" for [B, N, H, D]. Any strides are accepted as long as
    the last (D) dimension is contiguous; contiguous [B, H, N, D] tensors take attn_fwd, all
    others attn_fwd_strided (no copies either way).

    ``attn_mask`` is an optional explicit mask over (query, key), broadcastable to
    [B, Hq, N, N] (shapes [N, N], [B, N, N] or [B or 1, Hq or 1, N, N]; query rows and keys are
    in sequence order whatever ``layout`` is): bool or uint8 keeps the key where nonzero, q's
    dtype is added to the scaled score. Its key dimension must be contiguous and its rows
    16-byte aligned (for a ragged N, a [.., N, Npad] view of a padded tensor works). It
    combines with ``causal`` and ``valid_len``; the call then goes to attn_fwd_masked.

    Without a mask, sizes whose query tiles do not fill the device (attn_fwd_workspace_floats
    > 0, 16-bit dtypes) go to attn_fwd_ws, which splits the key ranges; ``ws`` is then its
    float32 workspace (allocated with torch when not given). ``split=False`` keeps them on
    attn_fwd / attn_fwd_strided (one workgroup per query tile).

    Allocates ``out`` (q's shape, layout and dtype, contiguous) and ``lse`` ([B, Hq, N] float32)
    with torch when they are not given. Returns (out, lse); lse is None when want_lse is False
    and none was given.
    """
    import torch
    if layout not in ("bhnd", "bnhd"):
        raise ValueError("layout must be 'bhnd' or 'bnhd'")
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share a dtype")
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k, v must be device tensors")
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    # [B, H, N, D] views of every tensor
    tr = (lambda t: t.transpose(1, 2)) if layout == "bnhd" else (lambda t: t)
    qv, kv, vv, ov = tr(q), tr(k), tr(v), tr(out)
    B, Hq, N, D = qv.shape
    Hkv = kv.shape[1]
    if tuple(kv.shape) != (B, Hkv, N, D) or tuple(vv.shape) != tuple(kv.shape):
        raise ValueError("shape mismatch: q %s k %s v %s" % (tuple(q.shape), tuple(k.shape),
                                                              tuple(v.shape)))
    if tuple(ov.shape) != (B, Hq, N, D) or out.dtype != q.dtype or not out.is_cuda:
        raise ValueError("out must be a device tensor of q's shape and dtype")
    for name, t in (("q", qv), ("k", kv), ("v", vv), ("out", ov)):
        if t.stride(3) != 1:
            raise ValueError("%s: the D dimension must be contiguous" % name)
    if scale is None:
        scale = 1.0 / float(D) ** 0.5
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    if lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, N)
                            or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 [B, Hq, N] tensor")
    vl_ptr = None
    if valid_len is not None:
        if valid_len.dtype != torch.int32 or tuple(valid_len.shape) != (B,) or not valid_len.is_cuda:
            raise ValueError("valid_len must be an int32 device tensor of shape [B]")
        vl_ptr = valid_len.data_ptr()
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    lse_ptr = lse.data_ptr() if lse is not None else None
    if attn_mask is not None:
        m, mtype = _mask_view(attn_mask, q.dtype, B, Hq, N)
        st = attn_fwd_masked(qv.data_ptr(), qv.stride()[:3], kv.data_ptr(), kv.stride()[:3],
                             vv.data_ptr(), vv.stride()[:3], ov.data_ptr(), ov.stride()[:3],
                             lse_ptr, B, Hq, Hkv, N, D, float(scale), int(bool(causal)), vl_ptr,
                             m.data_ptr(), mtype, m.stride()[:3], _dtype_code(q),
                             stream.cuda_stream)
        if st != ATTN_OK:
            raise AttnError(st, "attn_fwd_masked")
        return out, lse
    n_ws = 0
    if split and q.dtype != torch.float32:
        n_ws = attn_fwd_workspace_floats(B, Hq, Hkv, N, D, causal)
    if n_ws > 0:
        if ws is None:
            ws = torch.empty((n_ws,), dtype=torch.float32, device=q.device)
        if ws.dtype != torch.float32 or not ws.is_contiguous() or not ws.is_cuda:
            raise ValueError("ws must be a contiguous float32 device tensor")
        st = attn_fwd_ws(qv.data_ptr(), qv.stride()[:3], kv.data_ptr(), kv.stride()[:3],
                         vv.data_ptr(), vv.stride()[:3], ov.data_ptr(), ov.stride()[:3], lse_ptr,
                         ws.data_ptr(), ws.numel(), B, Hq, Hkv, N, D, float(scale),
                         int(bool(causal)), vl_ptr, _dtype_code(q), stream.cuda_stream)
        where = "attn_fwd_ws"
    elif all(t.is_contiguous() for t in (qv, kv, vv, ov)):
        st = attn_fwd(qv.data_ptr(), kv.data_ptr(), vv.data_ptr(), ov.data_ptr(), lse_ptr, B, Hq,
                      Hkv, N, D, float(scale), int(bool(causal)), vl_ptr, _dtype_code(q),
                      stream.cuda_stream)
        where = "attn_fwd"
    else:
        st = attn_fwd_strided(qv.data_ptr(), qv.stride()[:3], kv.data_ptr(), kv.stride()[:3],
                              vv.data_ptr(), vv.stride()[:3], ov.data_ptr(), ov.stride()[:3],
                              lse_ptr, B, Hq, Hkv, N, D, float(scale), int(bool(causal)),
                              vl_ptr, _dtype_code(q), stream.cuda_stream)
        where = "attn_fwd_strided"
    if st != ATTN_OK:
        raise AttnError(st, where)
    return out, lse


def backward(q, k, v, out, dout, lse, causal: bool, valid_len=None,
             scale: Optional[float] = None, dq=None, dk=None, dv=None, ws=None, stream=None,
             layout: str = "bhnd", attn_mask=None):
    """Run the attention backward on torch device tensors; returns (dq, dk, dv).

    ``out`` and ``lse`` are the forward's outputs for the same inputs; ``dout`` is the gradient
    of the loss with respect to ``out``. ``layout`` names the dimension order of q, k, v, out,
    dout and the gradients ("bhnd" = [B, H, N, D], "bnhd" = [B, N, H, D]); any strides with a
    contiguous D dimension are accepted (contiguous [B, H, N, D] tensors take attn_bwd, others
    attn_bwd_strided, with no copies). ``attn_mask`` is the forward's explicit mask (as in
    forward(); the call then goes to attn_bwd_masked). Gradients (each in its input's layout)
    and the float32 workspace ``ws`` are allocated with torch when not given. A workspace of
    exactly 2 * B * Hq * N values (Delta, then the LSE in base 2) takes attn_bwd /
    attn_bwd_strided / attn_bwd_masked; an allocated or larger one (attn_bwd_workspace_floats
    values) takes attn_bwd_ws, which may split the dK/dV work over more workgroups.
    """
    import torch
    if layout not in ("bhnd", "bnhd"):
        raise ValueError("layout must be 'bhnd' or 'bnhd'")
    tr = (lambda t: t.transpose(1, 2)) if layout == "bnhd" else (lambda t: t)
    qv, kv, vv, ov, gv = tr(q), tr(k), tr(v), tr(out), tr(dout)
    B, Hq, N, D = qv.shape
    Hkv = kv.shape[1]
    for name, t, shape in (("q", qv, (B, Hq, N, D)), ("k", kv, (B, Hkv, N, D)),
                           ("v", vv, (B, Hkv, N, D)), ("out", ov, (B, Hq, N, D)),
                           ("dout", gv, (B, Hq, N, D))):
        if tuple(t.shape) != shape or t.dtype != q.dtype or not t.is_cuda:
            raise ValueError("%s must be a device tensor of shape %s and q's dtype" % (name, shape))
        if t.stride(3) != 1:
            raise ValueError("%s: the D dimension must be contiguous" % name)
    if lse is None or lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, N):
        raise ValueError("lse must be the forward's float32 [B, Hq, N] tensor")
    if not lse.is_contiguous():
        raise ValueError("lse must be contiguous")
    if scale is None:
        scale = 1.0 / float(D) ** 0.5
    dq = torch.empty_like(q, memory_format=torch.contiguous_format) if dq is None else dq
    dk = torch.empty_like(k, memory_format=torch.contiguous_format) if dk is None else dk
    dv = torch.empty_like(v, memory_format=torch.contiguous_format) if dv is None else dv
    dqv, dkv, dvv = tr(dq), tr(dk), tr(dv)
    for name, t, shape in (("dq", dqv, (B, Hq, N, D)), ("dk", dkv, (B, Hkv, N, D)),
                           ("dv", dvv, (B, Hkv, N, D))):
        if tuple(t.shape) != shape or t.dtype != q.dtype or not t.is_cuda or t.stride(3) != 1:
            raise ValueError("%s must be a device tensor of shape %s, q's dtype, D contiguous"
                             % (name, shape))
    if ws is None:
        ws = torch.empty((attn_bwd_workspace_floats(B, Hq, Hkv, N, D),), dtype=torch.float32,
                         device=q.device)
    elif ws.dtype != torch.float32 or ws.numel() < 2 * B * Hq * N or not ws.is_contiguous():
        raise ValueError("ws must be a contiguous float32 tensor of 2 * B * Hq * N values")
    vl_ptr = None
    if valid_len is not None:
        if valid_len.dtype != torch.int32 or tuple(valid_len.shape) != (B,) or not valid_len.is_cuda:
            raise ValueError("valid_len must be an int32 device tensor of shape [B]")
        vl_ptr = valid_len.data_ptr()
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    views = (qv, kv, vv, ov, gv, dqv, dkv, dvv)
    if ws.numel() > 2 * B * Hq * N:
        m, mtype = None, ATTN_MASK_NONE
        if attn_mask is not None:
            m, mtype = _mask_view(attn_mask, q.dtype, B, Hq, N)
        st = attn_bwd_ws(
            qv.data_ptr(), qv.stride()[:3], kv.data_ptr(), kv.stride()[:3], vv.data_ptr(),
            vv.stride()[:3], ov.data_ptr(), ov.stride()[:3], gv.data_ptr(), gv.stride()[:3],
            lse.data_ptr(), dqv.data_ptr(), dqv.stride()[:3], dkv.data_ptr(), dkv.stride()[:3],
            dvv.data_ptr(), dvv.stride()[:3], ws.data_ptr(), ws.numel(), B, Hq, Hkv, N, D,
            float(scale), int(bool(causal)), vl_ptr, None if m is None else m.data_ptr(), mtype,
            None if m is None else m.stride()[:3], _dtype_code(q), stream.cuda_stream)
        name = "attn_bwd_ws"
    elif attn_mask is not None:
        m, mtype = _mask_view(attn_mask, q.dtype, B, Hq, N)
        st = attn_bwd_masked(
            qv.data_ptr(), qv.stride()[:3], kv.data_ptr(), kv.stride()[:3], vv.data_ptr(),
            vv.stride()[:3], ov.data_ptr(), ov.stride()[:3], gv.data_ptr(), gv.stride()[:3],
            lse.data_ptr(), dqv.data_ptr(), dqv.stride()[:3], dkv.data_ptr(), dkv.stride()[:3],
            dvv.data_ptr(), dvv.stride()[:3], ws.data_ptr(), B, Hq, Hkv, N, D, float(scale),
            int(bool(causal)), vl_ptr, m.data_ptr(), mtype, m.stride()[:3], _dtype_code(q),
            stream.cuda_stream)
        name = "attn_bwd_masked"
    elif all(t.is_contiguous() for t in views):
        st = attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dout.data_ptr(),
                      lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws.data_ptr(),
                      B, Hq, Hkv, N, D, float(scale), int(bool(causal)), vl_ptr,
                      _dtype_code(q), stream.cuda_stream)
        name = "attn_bwd"
    else:
        st = attn_bwd_strided(
            qv.data_ptr(), qv.stride()[:3], kv.data_ptr(), kv.stride()[:3], vv.data_ptr(),
            vv.stride()[:3], ov.data_ptr(), ov.stride()[:3], gv.data_ptr(), gv.stride()[:3],
            lse.data_ptr(), dqv.data_ptr(), dqv.stride()[:3], dkv.data_ptr(), dkv.stride()[:3],
            dvv.data_ptr(), dvv.stride()[:3], ws.data_ptr(), B, Hq, Hkv, N, D, float(scale),
            int(bool(causal)), vl_ptr, _dtype_code(q), stream.cuda_stream)
        name = "attn_bwd_strided"
    if st != ATTN_OK:
        raise AttnError(st, name)
    return dq, dk, dv


def _autograd_function():
    import torch

    class _Attention(torch.autograd.Function):
        @staticmethod
        def forward(ctx, q, k, v, causal, valid_len, scale, layout, attn_mask):
            out, lse = forward(q, k, v, causal=causal, valid_len=valid_len, scale=scale,
                               layout=layout, attn_mask=attn_mask)
            ctx.save_for_backward(q, k, v, out, lse, valid_len, attn_mask)
            ctx.causal, ctx.scale, ctx.layout = causal, scale, layout
            return out

        @staticmethod
        def backward(ctx, dout):
            q, k, v, out, lse, valid_len, attn_mask = ctx.saved_tensors
            if dout.stride(-1) != 1 or 0 in dout.stride():
                dout = dout.contiguous()   # e.g. a broadcast gradient
            dq, dk, dv = backward(q, k, v, out, dout, lse, causal=ctx.causal,
                                  valid_len=valid_len, scale=ctx.scale, layout=ctx.layout,
                                  attn_mask=attn_mask)
            return dq, dk, dv, None, None, None, None, None

    return _Attention


_ATTENTION = None


def attention(q, k, v, causal: bool, valid_len=None, scale: Optional[float] = None,
              layout: str = "bhnd", attn_mask=None):
    """Differentiable attention on [B, H, N, D] (or, with layout="bnhd", [B, N, H, D]) tensors:
    forward through attn_fwd, gradients through attn_bwd (torch.autograd glue only; strided
    inputs are used in place)."""
    global _ATTENTION
    if _ATTENTION is None:
        _ATTENTION = _autograd_function()
    return _ATTENTION.apply(q, k, v, causal, valid_len, scale, layout, attn_mask)
