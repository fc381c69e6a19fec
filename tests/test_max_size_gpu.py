"""The forward at the longest sequence the library accepts (N = 2^22 rows per head), through the
C ABI, against the fp64 oracle on sampled rows.

Inputs repeat one seeded block of P = 4093 rows (a prime, so a row read at any power-of-two
offset from the right one holds other values) along the sequence, with a different block for
every (batch, head); this keeps host generation cheap at 2^22 rows.
"""
import numpy as np
import pytest

from gpu_util import compare, from_device, log, run_oracle, sample_rows, to_device
import scaled_dot_product_fwd_amd as sdp
from scaled_dot_product_fwd_amd import inputs

pytestmark = pytest.mark.gpu

NMAX = 1 << 22
P = 4093


def tiled(block: np.ndarray, N: int) -> np.ndarray:
    """[.., P, D] -> [.., N, D], the block repeated along the rows."""
    out = np.empty(block.shape[:-2] + (N, block.shape[-1]), block.dtype)
    for s in range(0, N, P):
        n = min(P, N - s)
        out[..., s:s + n, :] = block[..., :n, :]
    return out


def device_rows(out, lse, rows, dtype, D):
    """The sampled flat rows of the device outputs, as float64."""
    import torch
    idx = torch.from_numpy(rows).cuda()
    O = from_device(out.reshape(-1, D).index_select(0, idx), dtype)
    L = lse.reshape(-1).index_select(0, idx).cpu().numpy().astype(np.float64)
    return O, L


def test_max_length_causal_needles():
    """One head of 2^22 rows, D = 128, causal: the last rows see every key. A few keys are
    'needles' aligned with one query row (score about 34 against about N(0, 1) elsewhere), so
    that row's output is close to the needle's value row: a key tile read from the wrong place,
    or skipped, anywhere in the 2^22 keys moves that output by far more than the tolerance."""
    import torch
    N, D, dtype = NMAX, 128, "bf16"
    block = inputs.make_case(1, 1, 1, P, D, dtype, True, False, seed=[140, 1])
    q = tiled(block.q_bits, N)
    k = tiled(block.k_bits, N)
    v = tiled(block.v_bits, N)
    # (query row, needle key): the farthest key, both sides of the middle, the diagonal, the
    # tile just before it, and a mid-sequence row reaching back to the start.
    needles = [(N - 1, 0), (N - 2, (1 << 21) - 1), (N - 3, 1 << 21), (N - 4, N - 4),
               (N - 5, N - 70), (3 * (N // 4) + 9, 5), (12345, 100)]
    assert len({r % P for r, _ in needles}) == len(needles)
    for i, (r, j) in enumerate(needles):
        qr = inputs.widen(q[0, 0, r], dtype).astype(np.float32)
        k[0, 0, j] = inputs.round_bits(3.0 * qr, dtype)
        sign = np.where((np.arange(D) + i) % 2 == 0, 1.0, -1.0).astype(np.float32)
        v[0, 0, j] = inputs.round_bits(4.0 * sign, dtype)
    case = inputs.Case(1, 1, 1, N, D, dtype, True, block.scale, q, k, v, None)
    # The oracle streams every visible key per row, so the sample stays small: the needle
    # rows, tile edges near the start, the middle, the tile edge before the end, random rows.
    rng = np.random.default_rng(7)
    rows = np.union1d(np.array([0, 1, 63, 64, 127, 128, 129, N // 2, N - 65, N - 64], np.int64),
                      np.array([r for r, _ in needles], np.int64))
    rows = np.union1d(rows, rng.integers(0, N, size=4))
    log("max-length causal: N=%d D=%d rows=%d" % (N, D, rows.size))

    out, lse = sdp.forward(to_device(q, dtype), to_device(k, dtype), to_device(v, dtype),
                           causal=True, scale=case.scale)
    torch.cuda.synchronize()
    O, L = device_rows(out, lse, rows, dtype, D)
    del out, lse
    torch.cuda.empty_cache()
    O_ref, L_ref = run_oracle(case, rows=rows)
    compare(case, O, L, O_ref, L_ref, tag="max-length causal")   # all [rows, ..] already
    for i, (r, j) in enumerate(needles):
        at = int(np.searchsorted(rows, r))
        vj = inputs.widen(v[0, 0, j], dtype)
        assert np.abs(O_ref[at] - vj).max() < 0.05, "needle %d does not dominate its row" % i
        assert np.abs(O[at] - vj).max() < 0.05 + 2e-2, "row %d misses its needle at key %d" % (
            r, j)



# (dtype, valid_len): 2^22 rows for each of 3 batches x 2 query heads sharing 1 KV head, D = 64,
# without the causal mask. The query and output tensors pass 2^31 bytes, so the last heads sit
# beyond 32-bit byte offsets; batch 0 has no visible key, batch 1 a ragged last key tile.
PADDED = [("bf16", (0, 257, 70001)), ("f32", (0, 257, 20001))]


@pytest.mark.parametrize("cfg", PADDED, ids=lambda c: c[0])
def test_max_length_padded_gqa(cfg):
    """Every row is computed over the keys below valid_len[b] only (no causal mask), so the
    oracle's value for a sampled row equals its value on a shorter case that holds that row's
    query and the first max(valid_len) keys. That shorter case is what the oracle runs."""
    import torch
    dtype, vls = cfg
    B, Hq, Hkv, N, D = 3, 2, 1, NMAX, 64
    block = inputs.make_case(B, Hq, Hkv, P, D, dtype, False, False, seed=[141, len(dtype)])
    q = tiled(block.q_bits, N)
    k = tiled(block.k_bits, N)
    v = tiled(block.v_bits, N)
    valid_len = np.array(vls, np.int32)
    case = inputs.Case(B, Hq, Hkv, N, D, dtype, False, block.scale, q, k, v, valid_len)
    rows = sample_rows(case, per_head=16, seed=8)
    log("max-length padded %s: B=%d Hq=%d N=%d D=%d valid_len=%s rows=%d" % (
        dtype, B, Hq, N, D, list(vls), rows.size))

    vl_dev = torch.from_numpy(valid_len).cuda()
    out, lse = sdp.forward(to_device(q, dtype), to_device(k, dtype), to_device(v, dtype),
                           causal=False, valid_len=vl_dev, scale=case.scale)
    torch.cuda.synchronize()
    O, L = device_rows(out, lse, rows, dtype, D)
    del out, lse
    torch.cuda.empty_cache()

    # The shorter case: each (b, hq)'s sampled queries first, then the keys below max(valid_len).
    bh, i = rows // N, rows % N
    counts = np.bincount(bh, minlength=B * Hq)
    N2 = int(max(max(vls), counts.max()))
    q2 = np.zeros((B, Hq, N2, D), q.dtype)
    rows2 = np.empty_like(rows)
    for g in range(B * Hq):
        sel = np.nonzero(bh == g)[0]
        q2[g // Hq, g % Hq, :sel.size] = q[g // Hq, g % Hq, i[sel]]
        rows2[sel] = g * N2 + np.arange(sel.size)
    short = inputs.Case(B, Hq, Hkv, N2, D, dtype, False, case.scale, q2,
                        np.ascontiguousarray(k[:, :, :N2]), np.ascontiguousarray(v[:, :, :N2]),
                        valid_len)
    O_ref, L_ref = run_oracle(short, rows=rows2)
    compare(case, O, L, O_ref, L_ref, tag="max-length padded %s" % dtype)
    assert np.all(np.isneginf(L[bh < Hq]))          # batch 0: no visible key


def test_max_length_backward_padded():
    """The backward at N = 1024 x 4093 = 4,191,232 rows (just under 2^22; a whole number of
    blocks), 2 query heads over 1 KV head, D = 64, without the causal mask, valid_len 1000.
    Every row sees the same 1000 keys, so a row repeats the gradient terms of the block row it
    copies: dQ of row i is the block's dQ of row i mod 4093, dK and dV of a key below
    valid_len are 1024 times the block's, and keys past valid_len get exactly 0. The block
    itself (N = 4093) is what the oracle runs."""
    import torch
    import oracle
    from test_bwd_gpu import check_grad
    M, D, dtype, VL = 1024, 64, "bf16", 1000
    N = M * P
    vl = np.array([VL], np.int32)
    block = inputs.make_case(1, 2, 1, P, D, dtype, False, True, seed=[142, 1], valid_len=vl)
    dout_block = inputs.make_grad(block, [142, 1])
    rep = lambda x: np.tile(x, (1, 1, M, 1))   # noqa: E731
    log("max-length backward: N=%d D=%d valid_len=%d" % (N, D, VL))
    q, k, v, do = (to_device(rep(x), dtype) for x in (block.q_bits, block.k_bits, block.v_bits,
                                                      dout_block))
    vl_dev = torch.from_numpy(vl).cuda()
    out, lse = sdp.forward(q, k, v, causal=False, valid_len=vl_dev, scale=block.scale)
    dq, dk, dv = sdp.backward(q, k, v, out, do, lse, causal=False, valid_len=vl_dev,
                              scale=block.scale)
    torch.cuda.synchronize()
    assert dk[:, :, VL:].abs().max().item() == 0.0 and dv[:, :, VL:].abs().max().item() == 0.0
    rng = np.random.default_rng(9)
    rows = np.union1d(np.array([0, 1, 127, 128, P - 1, P, N // 2, N - 2, N - 1]),
                      rng.integers(0, N, size=24))
    idx = torch.from_numpy(rows).cuda()
    got_q = from_device(dq.index_select(2, idx), dtype)
    got_k = from_device(dk[:, :, :VL], dtype)
    got_v = from_device(dv[:, :, :VL], dtype)
    del q, k, v, do, out, lse, dq, dk, dv
    torch.cuda.empty_cache()

    qw, kw, vw = block.widened()
    rq, rk, rv = oracle.attn_bwd(qw, kw, vw, inputs.widen(dout_block, dtype), block.scale,
                                 False, vl)
    e = [check_grad("dQ", got_q, rq[:, :, rows % P], dtype, "max-length backward"),
         check_grad("dK", got_k, M * rk[:, :, :VL], dtype, "max-length backward"),
         check_grad("dV", got_v, M * rv[:, :, :VL], dtype, "max-length backward")]
    log("max-length backward: rel err dQ %.2e dK %.2e dV %.2e" % tuple(e))
