"""Helpers for GPU parity tests: move seeded cases to the device, run the HIP path through the
C ABI, run the oracle on all rows or on a sample of rows, and compare."""
from __future__ import annotations

import sys

import numpy as np

import oracle
import scaled_dot_product_fwd_amd as sdp
from scaled_dot_product_fwd_amd import inputs

# Tolerances (max abs error against the fp64 oracle): O within 2e-2 for bf16 inputs and 5e-3 for
# fp16 inputs, LSE within 1e-3 on rows with a visible key; rows with none are exactly 0 / -inf.
# fp32 inputs (fp32 products throughout): 1e-4 for O and LSE. A score of D fp32 products carries
# an error of at most about D * 2^-24 of sum |scale q_d k_d| (7.6e-6 of it at D = 128), i.e.
# ~1e-4 for the largest scores of these cases (|s| up to ~100 with the keys grown 13x); O and
# LSE inherit that absolute error. Measured: <= 2.5e-5.
O_TOL = {"bf16": 2e-2, "f16": 5e-3, "f32": 1e-4}
LSE_TOL = {"bf16": 1e-3, "f16": 1e-3, "f32": 1e-4}


def log(msg):
    sys.stdout.write(msg + "\n")
    sys.stdout.flush()


def to_device(bits: np.ndarray, dtype: str):
    import torch
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.float32)).cuda()
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    t = t.view(torch.bfloat16 if dtype == "bf16" else torch.float16)
    return t.cuda()


def from_device(t, dtype: str) -> np.ndarray:
    import torch
    if dtype == "f32":
        return t.contiguous().cpu().numpy().astype(np.float64)
    bits = t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return inputs.widen(bits, dtype)


def run_device(case: inputs.Case, want_lse=True, stream=None, split=True):
    """Returns (O float64 [B,Hq,N,D], LSE float64 [B,Hq,N] or None, device tensors)."""
    import torch
    q = to_device(case.q_bits, case.dtype)
    k = to_device(case.k_bits, case.dtype)
    v = to_device(case.v_bits, case.dtype)
    vl = None
    if case.valid_len is not None:
        vl = torch.from_numpy(case.valid_len.astype(np.int32)).cuda()
    out, lse = sdp.forward(q, k, v, causal=case.causal, valid_len=vl, scale=case.scale,
                           want_lse=want_lse, stream=stream, split=split)
    torch.cuda.synchronize()
    O = from_device(out, case.dtype)
    L = lse.cpu().numpy().astype(np.float64) if lse is not None else None
    return O, L


def run_oracle(case: inputs.Case, rows=None, threads=0):
    q, k, v = case.widened()
    return oracle.attn_fwd(q, k, v, case.scale, case.causal, case.valid_len, rows=rows,
                           threads=threads)


def run_oracle_masked(case: inputs.Case, keep_mask=None, add_mask=None, threads=0):
    q, k, v = case.widened()
    return oracle.attn_fwd(q, k, v, case.scale, case.causal, case.valid_len, threads=threads,
                           keep_mask=keep_mask, add_mask=add_mask)


def sample_rows(case: inputs.Case, per_head: int, seed=0) -> np.ndarray:
    """Flat row indices covering every (b, hq): the first and last rows, tile edges, the rows
    around valid_len[b], and random rows."""
    rng = np.random.default_rng(seed)
    N = case.N
    special = {0, 1, N - 1, N - 2, 63, 64, 127, 128, 129, 255, 256, N // 2}
    rows = []
    for b in range(case.B):
        sp = set(special)
        if case.valid_len is not None:
            vl = int(case.valid_len[b])
            sp |= {vl - 1, vl, vl + 1}
        sp = sorted(i for i in sp if 0 <= i < N)
        for hq in range(case.Hq):
            picks = set(sp[: max(2, per_head // 2)])
            picks |= set(rng.integers(0, N, size=per_head).tolist())
            base = (b * case.Hq + hq) * N
            rows.extend(base + i for i in sorted(picks))
    return np.array(rows, dtype=np.int64)


def compare(case: inputs.Case, O, L, O_ref, L_ref, rows=None, tag=""):
    """Assert O/LSE match the oracle (O, L possibly full tensors; O_ref/L_ref per rows)."""
    D = case.D
    if rows is not None:
        O = O.reshape(-1, D)[rows]
        L = L.reshape(-1)[rows] if L is not None else None
    else:
        O = O.reshape(-1, D)
        L = L.reshape(-1) if L is not None else None
        O_ref = O_ref.reshape(-1, D)
        L_ref = L_ref.reshape(-1)
    assert not np.isnan(O).any(), "%s: NaN in O" % tag
    empty = np.isneginf(L_ref)
    err = np.abs(O - O_ref).max() if O.size else 0.0
    assert np.all(O[empty] == 0.0), "%s: rows with no visible key are not exactly 0" % tag
    assert err <= O_TOL[case.dtype], "%s: max |O - oracle| = %.3g > %.3g" % (
        tag, err, O_TOL[case.dtype])
    lerr = 0.0
    if L is not None:
        assert not np.isnan(L).any(), "%s: NaN in LSE" % tag
        assert np.all(np.isneginf(L[empty])), "%s: empty rows must have LSE = -inf" % tag
        if (~empty).any():
            lerr = np.abs(L[~empty] - L_ref[~empty]).max()
        assert lerr <= LSE_TOL[case.dtype], "%s: max |LSE - oracle| = %.3g" % (tag, lerr)
    log("%s: max|dO| %.3g  max|dLSE| %.3g  rows %d (empty %d)" % (
        tag, err, lerr, O.shape[0], int(empty.sum())))
    return err, lerr


def mask_values(kind, pattern, dtype, B, Hq, N, rng):
    """Mask values as [B or 1, Hq or 1, N, N] (uint8 keep, or 16-bit bits for additive)."""
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    if kind == "keep":
        if pattern == "random_bh":
            return (rng.random((B, Hq, N, N)) < 0.7).astype(np.uint8)
        if pattern == "random_b":
            return (rng.random((B, 1, N, N)) < 0.6).astype(np.uint8)
        if pattern == "window":
            return (np.abs(i - j) < 40).astype(np.uint8)[None, None]
        if pattern == "empty_rows":
            m = (rng.random((B, Hq, N, N)) < 0.5).astype(np.uint8)
            m[:, :, ::7] = 0          # every 7th query sees nothing
            return m
    x = None
    if pattern == "random_bh":
        x = rng.normal(0.0, 2.0, (B, Hq, N, N)).astype(np.float32)
        x[rng.random(x.shape) < 0.25] = -np.inf
    elif pattern == "random_b":
        x = rng.normal(0.0, 1.0, (B, 1, N, N)).astype(np.float32)
        x[rng.random(x.shape) < 0.3] = -np.inf
    elif pattern == "alibi":
        slopes = 2.0 ** (-8.0 * (np.arange(Hq) + 1) / Hq)
        x = (-slopes[:, None, None] * np.abs(i - j)[None]).astype(np.float32)[None]
    elif pattern == "window_neginf":
        x = np.where(np.abs(i - j) < 50, 0.0, -np.inf).astype(np.float32)[None, None]
    elif pattern == "large_negative":
        x = np.where(rng.random((1, Hq, N, N)) < 0.5, -1.0e4, 0.0).astype(np.float32)
    return inputs.round_bits(x, dtype)


def device_mask(kind, pattern, dtype, mv, N):
    """The device view of mask values from mask_values: rows padded to 16 bytes (a
    [.., N, Npad] view, as the layout rules require); [B, N, N] when shared by the heads and
    [N, N] (bool) for the shared window. Additive masks have the inputs' type (fp32 for f32)."""
    import torch
    es = 1 if kind == "keep" else (4 if dtype == "f32" else 2)
    npad = -(-N * es // 16) * 16 // es
    host = np.zeros(mv.shape[:3] + (npad,), mv.dtype)
    host[..., :N] = mv
    if kind == "add":
        host = host.view(np.int32 if dtype == "f32" else np.int16)
    t = torch.from_numpy(host).cuda()
    if kind == "add":
        t = t.view({"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[dtype])
    else:
        t = t.view(torch.bool) if pattern == "window" else t
    dmask = t[..., :N]
    if dmask.shape[1] == 1 and pattern != "window":
        dmask = dmask[:, 0]                       # [B, N, N]: shared by the heads
    elif pattern == "window":
        dmask = dmask[0, 0]                       # [N, N]: shared by everything
    return dmask
