"""fp64 CPU oracle for masked multi-head attention forward -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import this package. The product path (``scaled_dot_product_fwd_amd``) never imports it and
shares no code with it.

The arithmetic lives in ``attn_oracle.c`` (plain C, IEEE double, OpenMP over independent query
rows); this module only builds that file with gcc and marshals numpy arrays into it. The C file's
header states the definition it follows and the page passages it cites.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile the oracle with gcc (no fast-math: IEEE double semantics are the point)."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def load(path: str = _LIB_PATH) -> ctypes.CDLL:
    lib = ctypes.CDLL(path)
    f = lib.oracle_attn_fwd
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int64] * 5 + [
        ctypes.c_double, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
        ctypes.c_int]
    g = lib.oracle_attn_fwd_masked
    g.restype = ctypes.c_int
    g.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int64] * 5 + [
        ctypes.c_double, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int]
    h = lib.oracle_attn_bwd
    h.restype = ctypes.c_int
    h.argtypes = [ctypes.c_void_p] * 7 + [ctypes.c_int64] * 5 + [
        ctypes.c_double, ctypes.c_int, ctypes.c_void_p, ctypes.c_int]
    hm = lib.oracle_attn_bwd_masked
    hm.restype = ctypes.c_int
    hm.argtypes = [ctypes.c_void_p] * 7 + [ctypes.c_int64] * 5 + [
        ctypes.c_double, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
        ctypes.c_void_p, ctypes.c_int]
    lib.oracle_max_threads.restype = ctypes.c_int
    return lib


def _get_lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or (
                os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
            build()
        _lib = load()
    return _lib


def max_threads() -> int:
    return int(_get_lib().oracle_max_threads())


def _mask_arg(keep_mask, add_mask, B, Hq, N):
    """(kind, array, element strides) of an explicit mask broadcast to [B, Hq, N, N]."""
    if keep_mask is not None and add_mask is not None:
        raise ValueError("give at most one of keep_mask and add_mask")
    if keep_mask is None and add_mask is None:
        return 0, None, None
    kind = 1 if keep_mask is not None else 2
    m = keep_mask if kind == 1 else add_mask
    m = np.asarray(m, dtype=np.uint8 if kind == 1 else np.float64)
    m = np.broadcast_to(m, (B, Hq, N, N))
    if m.strides[3] != m.itemsize:
        m = np.ascontiguousarray(m)
    return kind, m, (ctypes.c_int64 * 3)(*[st // m.itemsize for st in m.strides[:3]])


def attn_fwd(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, causal: bool,
             valid_len: Optional[np.ndarray] = None, rows: Optional[np.ndarray] = None,
             threads: int = 0, lib: Optional[ctypes.CDLL] = None, keep_mask=None,
             add_mask=None) -> Tuple[np.ndarray, np.ndarray]:
    """Attention forward in fp64.

    q: [B,Hq,N,D] float64, k/v: [B,Hkv,N,D] float64, valid_len: int32[B] or None.
    keep_mask (uint8/bool) or add_mask (float64): an explicit mask broadcastable to
    [B,Hq,N,N] (at most one of them).
    rows: optional int64 flat row indices (b*Hq + hq)*N + i; when given the outputs are
    [len(rows), D] and [len(rows)], else [B,Hq,N,D] and [B,Hq,N].
    Returns (O, LSE) as float64; LSE is the natural-log log-sum-exp (-inf for an empty row).
    """
    lib = lib or _get_lib()
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    B, Hq, N, D = q.shape
    Bk, Hkv, Nk, Dk = k.shape
    if (Bk, Nk, Dk) != (B, N, D) or v.shape != k.shape:
        raise ValueError("shape mismatch: q %s k %s v %s" % (q.shape, k.shape, v.shape))
    vl_ptr = None
    if valid_len is not None:
        valid_len = np.ascontiguousarray(valid_len, dtype=np.int32)
        if valid_len.shape != (B,):
            raise ValueError("valid_len must have shape [B]")
        vl_ptr = valid_len.ctypes.data
    if rows is None:
        out = np.empty((B, Hq, N, D), np.float64)
        lse = np.empty((B, Hq, N), np.float64)
        rows_ptr, nrows = None, B * Hq * N
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        nrows = rows.shape[0]
        out = np.empty((nrows, D), np.float64)
        lse = np.empty((nrows,), np.float64)
        rows_ptr = rows.ctypes.data
    kind, mask_arr, mst = _mask_arg(keep_mask, add_mask, B, Hq, N)
    mptr = mask_arr.ctypes.data if mask_arr is not None else None
    rc = lib.oracle_attn_fwd_masked(q.ctypes.data, k.ctypes.data, v.ctypes.data, out.ctypes.data,
                                    lse.ctypes.data, B, Hq, Hkv, N, D, float(scale),
                                    int(bool(causal)), vl_ptr, mptr, kind, mst, rows_ptr, nrows,
                                    int(threads))
    if rc != 0:
        raise ValueError("oracle_attn_fwd rejected its arguments (rc=%d)" % rc)
    return out, lse


def attn_bwd(q: np.ndarray, k: np.ndarray, v: np.ndarray, dout: np.ndarray, scale: float,
             causal: bool, valid_len: Optional[np.ndarray] = None, threads: int = 0,
             lib: Optional[ctypes.CDLL] = None, keep_mask=None,
             add_mask=None) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Gradients (dQ, dK, dV) in fp64 of sum(O * dout) for the forward above (causal /
    valid_len and an optional explicit mask as in attn_fwd). q, dout: [B,Hq,N,D];
    k, v: [B,Hkv,N,D]."""
    lib = lib or _get_lib()
    q, k, v, dout = (np.ascontiguousarray(x, dtype=np.float64) for x in (q, k, v, dout))
    B, Hq, N, D = q.shape
    Bk, Hkv, Nk, Dk = k.shape
    if (Bk, Nk, Dk) != (B, N, D) or v.shape != k.shape or dout.shape != q.shape:
        raise ValueError("shape mismatch")
    vl_ptr = None
    if valid_len is not None:
        valid_len = np.ascontiguousarray(valid_len, dtype=np.int32)
        if valid_len.shape != (B,):
            raise ValueError("valid_len must have shape [B]")
        vl_ptr = valid_len.ctypes.data
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    kind, mask_arr, mst = _mask_arg(keep_mask, add_mask, B, Hq, N)
    mptr = mask_arr.ctypes.data if mask_arr is not None else None
    rc = lib.oracle_attn_bwd_masked(q.ctypes.data, k.ctypes.data, v.ctypes.data,
                                    dout.ctypes.data, dq.ctypes.data, dk.ctypes.data,
                                    dv.ctypes.data, B, Hq, Hkv, N, D, float(scale),
                                    int(bool(causal)), vl_ptr, mptr, kind, mst, int(threads))
    if rc != 0:
        raise ValueError("oracle_attn_bwd rejected its arguments (rc=%d)" % rc)
    return dq, dk, dv
