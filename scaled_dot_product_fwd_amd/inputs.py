"""Seeded synthetic inputs for attention forward, shared by the device path's tests and bench
and by the oracle's checks.

This module draws random numbers and rounds them to 16 bits; it holds none of the attention
arithmetic. Every array it returns is plain numpy on the host.

Recipe (one rule for every workload):
  * generator ``numpy.random.default_rng([20, c])``; 20 is the seed the Triton file
    tiny_flash_attn_triton.py uses in its test (``causal_test``), c is the workload number;
  * draw Q, K, V in that order with ``standard_normal(dtype=float32)`` (iid N(0, 1)), times an
    optional standard deviation;
  * for padded workloads, then draw ``valid_len`` as ``integers(1, N + 1, size=B)`` (uniform in
    [1, N]) and set ``valid_len[0] = 0`` so that batch 0 has fully masked rows;
  * round each float32 value to the nearest 16-bit value (ties to even) of the workload's type
    (fp32 cases keep the float32 draws as they are);
  * for the backward pass, the upstream gradient dO comes from its own generator
    ``default_rng([21, *seed])`` (``make_grad``), also iid N(0, 1) rounded to the same type.
The device receives the 16-bit bit patterns; the oracle receives the same values widened
exactly to float64.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np

DTYPES = ("f16", "bf16", "f32")


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest, ties to even (NaN -> quiet NaN)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    if nan.any():
        rounded[nan] = 0x7FC0
    return rounded


def round_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> IEEE binary16 bit patterns; numpy's conversion rounds to nearest even."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def round_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 values -> bit patterns of `dtype` (uint16, or uint32 for f32, which is exact)."""
    if dtype == "bf16":
        return round_to_bf16_bits(x)
    if dtype == "f16":
        return round_to_f16_bits(x)
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    raise ValueError("dtype must be one of %s" % (DTYPES,))


def widen(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Bit patterns of `dtype` -> exact float64 values."""
    if dtype == "f32":
        return np.ascontiguousarray(bits, dtype=np.uint32).view(np.float32).astype(np.float64)
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float64)
    raise ValueError("dtype must be one of %s" % (DTYPES,))


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    c: int            # workload number; the generator is default_rng([20, c])
    B: int
    Hq: int
    Hkv: int
    N: int
    D: int
    dtype: str
    causal: bool
    padded: bool
    note: str = ""

    @property
    def scale(self) -> float:
        """1/sqrt(D) rounded to float32, as a Python float."""
        return float(np.float32(1.0 / np.sqrt(self.D)))


WORKLOADS: Dict[str, Workload] = {w.name: w for w in [
    Workload("tiny", 1, 1, 2, 2, 128, 64, "f16", False, False,
             "tiny non-causal MHA"),
    Workload("causal_mha", 2, 2, 8, 8, 1024, 64, "f16", True, False,
             "causal MHA"),
    Workload("causal_gqa", 3, 4, 32, 8, 2048, 128, "bf16", True, False,
             "causal GQA, group 4"),
    Workload("causal_padded", 4, 8, 16, 16, 2048, 64, "f16", True, True,
             "causal + valid_len padding, valid_len[0] = 0"),
    Workload("long_gqa", 5, 8, 32, 8, 4096, 128, "bf16", True, False,
             "long-context causal GQA (the headline shape)"),
    Workload("long_mqa", 6, 1, 32, 1, 16384, 128, "bf16", True, False,
             "long-context causal MQA"),
]}

HEADLINE = "long_gqa"


@dataclasses.dataclass
class Case:
    B: int
    Hq: int
    Hkv: int
    N: int
    D: int
    dtype: str
    causal: bool
    scale: float
    q_bits: np.ndarray            # uint16 [B,Hq,N,D] (uint32 for f32)
    k_bits: np.ndarray            # uint16 [B,Hkv,N,D] (uint32 for f32)
    v_bits: np.ndarray            # uint16 [B,Hkv,N,D] (uint32 for f32)
    valid_len: Optional[np.ndarray]  # int32 [B] or None

    def widened(self):
        return (widen(self.q_bits, self.dtype), widen(self.k_bits, self.dtype),
                widen(self.v_bits, self.dtype))


def make_case(B: int, Hq: int, Hkv: int, N: int, D: int, dtype: str, causal: bool,
              padded: bool, seed, scale: Optional[float] = None, std: float = 1.0,
              valid_len: Optional[np.ndarray] = None, zero_first: bool = True) -> Case:
    """Draw one case by the module recipe. ``seed`` is passed to default_rng as is.

    ``valid_len`` overrides the drawn lengths; ``zero_first`` sets valid_len[0] = 0 for drawn
    lengths.
    """
    rng = np.random.default_rng(seed)
    arrays = []
    for shape in ((B, Hq, N, D), (B, Hkv, N, D), (B, Hkv, N, D)):
        x = rng.standard_normal(shape, dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        arrays.append(round_bits(x, dtype))
    vl = None
    if padded:
        if valid_len is not None:
            vl = np.ascontiguousarray(valid_len, dtype=np.int32)
        else:
            vl = rng.integers(1, N + 1, size=B).astype(np.int32)
            if zero_first:
                vl[0] = 0
    if scale is None:
        scale = float(np.float32(1.0 / np.sqrt(D)))
    return Case(B, Hq, Hkv, N, D, dtype, causal, float(scale), arrays[0], arrays[1],
                arrays[2], vl)


def make_workload(w: Workload) -> Case:
    return make_case(w.B, w.Hq, w.Hkv, w.N, w.D, w.dtype, w.causal, w.padded, [20, w.c],
                     scale=w.scale)


def make_grad(case: Case, seed) -> np.ndarray:
    """The upstream gradient dO for a case: bits of the case's type [B, Hq, N, D] (uint16, or
    uint32 for f32), iid N(0, 1) rounded to that type, drawn from ``default_rng([21, *seed])``
    (``seed`` an int or a list)."""
    seed = list(seed) if isinstance(seed, (list, tuple)) else [seed]
    rng = np.random.default_rng([21] + seed)
    x = rng.standard_normal((case.B, case.Hq, case.N, case.D), dtype=np.float32)
    return round_bits(x, case.dtype)
