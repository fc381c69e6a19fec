"""Fused masked multi-head attention forward for AMD Instinct MI355X (gfx950).

A thin ctypes binding over ``libattn.so`` (C ABI declared in ``include/attn.h``). Every step of
the computation runs in the library's HIP kernels; this module only marshals arguments. There is
no fallback: if the library is missing, calls raise ``ImportError``.

Raw entry points (same names and argument order as the C ABI; pointers are integers):
    attn_fwd, attn_fwd_validate, attn_status_string, attn_version
Convenience for torch tensors (device memory and streams only):
    forward(q, k, v, causal=..., valid_len=None, scale=None, out=None, lse=None)
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

__all__ = ["ATTN_F16", "ATTN_BF16", "AttnError", "attn_fwd", "attn_fwd_validate",
           "attn_status_string", "attn_version", "forward", "library_path", "load_library"]

ATTN_F16 = 0
ATTN_BF16 = 1

ATTN_OK = 0
ATTN_ERR_NULL = -1
ATTN_ERR_SHAPE = -2
ATTN_ERR_HEAD_DIM = -3
ATTN_ERR_DTYPE = -4
ATTN_ERR_SCALE = -5
ATTN_ERR_LAUNCH = -6
ATTN_ERR_ALIAS = -7

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libattn.so")
_lib: Optional[ctypes.CDLL] = None

_c_int, _c_float, _vp = ctypes.c_int, ctypes.c_float, ctypes.c_void_p


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
    raise TypeError("q/k/v must be float16 or bfloat16, got %s" % t.dtype)


def forward(q, k, v, causal: bool, valid_len=None, scale: Optional[float] = None, out=None,
            lse=None, want_lse: bool = True, stream=None) -> Tuple[object, Optional[object]]:
    """Run attn_fwd on contiguous [B,H,N,D] torch tensors on the current (or given) stream.

    Allocates ``out`` ([B,Hq,N,D], q's dtype) and ``lse`` ([B,Hq,N] float32) with torch when
    they are not given. Returns (out, lse); lse is None when want_lse is False and none given.
    """
    import torch
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D [B, H, N, D]")
    B, Hq, N, D = q.shape
    Hkv = k.shape[1]
    if tuple(k.shape) != (B, Hkv, N, D) or tuple(v.shape) != tuple(k.shape):
        raise ValueError("shape mismatch: q %s k %s v %s" % (tuple(q.shape), tuple(k.shape),
                                                              tuple(v.shape)))
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share a dtype")
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k, v must be device tensors")
    if scale is None:
        scale = 1.0 / float(D) ** 0.5
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    if lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, N)
                            or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 [B, Hq, N] tensor")
    if tuple(out.shape) != (B, Hq, N, D) or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous [B, Hq, N, D] tensor of q's dtype")
    vl_ptr = None
    if valid_len is not None:
        if valid_len.dtype != torch.int32 or tuple(valid_len.shape) != (B,) or not valid_len.is_cuda:
            raise ValueError("valid_len must be an int32 device tensor of shape [B]")
        vl_ptr = valid_len.data_ptr()
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    st = attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                  lse.data_ptr() if lse is not None else None, B, Hq, Hkv, N, D, float(scale),
                  int(bool(causal)), vl_ptr, _dtype_code(q), stream.cuda_stream)
    if st != ATTN_OK:
        raise AttnError(st)
    return out, lse
