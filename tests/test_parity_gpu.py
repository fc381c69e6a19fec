"""Parity of the HIP path (through the C ABI) with the fp64 oracle, element by element.

Small cases compare every output; the full-size workloads compare a sample of rows (every
(batch, head), first/last rows, tile edges, rows around valid_len, random rows) that the oracle
computes one by one, with the HIP path run in the same launch configuration the benchmark
times.
"""
import numpy as np
import pytest

from gpu_util import (compare, device_mask, from_device, log, mask_values, run_device,
                      run_oracle, run_oracle_masked, sample_rows, to_device)
import scaled_dot_product_fwd_amd as sdp
from scaled_dot_product_fwd_amd import inputs

pytestmark = pytest.mark.gpu

# (dtype, D, causal, padded, B, Hq, Hkv, N): ragged N, N below one tile, exact tiles, GQA, MQA.
SMALL = [
    ("f16", 64, False, False, 1, 2, 2, 128),
    ("f16", 64, True, False, 2, 4, 4, 200),
    ("bf16", 64, True, True, 3, 4, 2, 257),
    ("bf16", 64, False, True, 2, 2, 1, 77),
    ("f16", 64, True, True, 2, 6, 3, 1),
    ("f16", 64, False, False, 1, 1, 1, 2),
    ("bf16", 128, False, False, 1, 4, 4, 384),
    ("bf16", 128, True, False, 2, 8, 2, 333),
    ("f16", 128, True, True, 3, 4, 1, 300),
    ("bf16", 128, False, True, 2, 4, 2, 129),
    ("f16", 128, True, False, 1, 2, 2, 63),
    ("bf16", 128, True, True, 4, 2, 2, 640),
    ("f16", 64, True, False, 1, 8, 8, 1000),
    ("bf16", 128, False, False, 1, 2, 1, 1),
]


# Each small case runs twice: split=True lets forward() take attn_fwd_ws (key ranges split over
# several workgroups, then merged) where the grid is small, split=False keeps one workgroup per
# query tile (attn_fwd).
@pytest.mark.parametrize("split", [False, True], ids=["one-pass", "split"])
@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: "%s-D%d-c%d-p%d-B%d-H%d-%d-N%d" % c)
def test_small_full(cfg, split):
    dtype, D, causal, padded, B, Hq, Hkv, N = cfg
    case = inputs.make_case(B, Hq, Hkv, N, D, dtype, causal, padded, seed=[101, D, N, B])
    log("case %s split %s valid_len %s" % (cfg, split, case.valid_len))
    O, L = run_device(case, split=split)
    O_ref, L_ref = run_oracle(case)
    compare(case, O, L, O_ref, L_ref, tag=str(cfg))


# Head dimensions 16 and 32 (zero-padded to the D = 64 geometry inside the kernel) and 256 (one
# workgroup per CU, unpipelined loop): ragged N, GQA / MQA, causal and padded, both types, every
# row compared.
SMALL_D = [
    ("f16", 16, False, False, 1, 2, 2, 128),
    ("bf16", 16, True, True, 3, 4, 2, 257),
    ("f16", 16, True, False, 2, 8, 1, 1000),
    ("bf16", 16, False, True, 2, 2, 1, 1),
    ("f16", 32, True, True, 2, 6, 3, 300),
    ("bf16", 32, False, False, 1, 4, 4, 65),
    ("bf16", 32, True, False, 2, 8, 2, 1100),
    ("f16", 32, False, True, 4, 2, 2, 513),
    ("bf16", 256, True, True, 3, 4, 2, 257),
    ("f16", 256, False, False, 1, 4, 4, 200),
    ("bf16", 256, True, False, 2, 8, 1, 1000),
    ("f16", 256, True, True, 2, 6, 3, 65),
    ("bf16", 256, False, True, 2, 2, 2, 1),
]


@pytest.mark.parametrize("split", [False, True], ids=["one-pass", "split"])
@pytest.mark.parametrize("cfg", SMALL_D, ids=lambda c: "%s-D%d-c%d-p%d-B%d-H%d-%d-N%d" % c)
def test_small_head_dims(cfg, split):
    dtype, D, causal, padded, B, Hq, Hkv, N = cfg
    case = inputs.make_case(B, Hq, Hkv, N, D, dtype, causal, padded, seed=[115, D, N, B])
    log("case %s split %s valid_len %s" % (cfg, split, case.valid_len))
    O, L = run_device(case, split=split)
    O_ref, L_ref = run_oracle(case)
    compare(case, O, L, O_ref, L_ref, tag=str(cfg))


# fp32 inputs (fp32 products on the fp32 matrix cores): head dims 16 ... 256, ragged N,
# GQA / MQA, causal and padded, a grid larger than the resident workgroups, every row compared.
SMALL_F32 = [
    (32, False, False, 1, 2, 2, 128),
    (64, True, True, 3, 4, 2, 257),
    (128, True, False, 2, 8, 2, 333),
    (128, False, True, 2, 4, 1, 1000),
    (64, False, False, 1, 1, 1, 1),
    (32, True, True, 2, 6, 3, 300),
    (128, True, True, 4, 16, 4, 1100),
    (16, True, True, 3, 4, 2, 257),
    (16, False, False, 2, 8, 1, 1000),
    (256, True, False, 2, 4, 2, 333),
    (256, False, True, 2, 6, 3, 200),
    (256, True, True, 1, 2, 1, 1),
]


@pytest.mark.parametrize("cfg", SMALL_F32, ids=lambda c: "f32-D%d-c%d-p%d-B%d-H%d-%d-N%d" % c)
def test_f32_inputs(cfg):
    D, causal, padded, B, Hq, Hkv, N = cfg
    case = inputs.make_case(B, Hq, Hkv, N, D, "f32", causal, padded, seed=[117, D, N, B])
    log("f32 case %s valid_len %s" % (cfg, case.valid_len))
    O, L = run_device(case)
    O_ref, L_ref = run_oracle(case)
    compare(case, O, L, O_ref, L_ref, tag="f32 " + str(cfg))


@pytest.mark.parametrize("scale", [-0.125, 0.0, 2.0])
def test_f32_scale_values(scale):
    case = inputs.make_case(1, 4, 2, 257, 64, "f32", True, True, seed=[119, 1], scale=scale,
                            valid_len=np.array([250], np.int32))
    O, L = run_device(case)
    O_ref, L_ref = run_oracle(case)
    compare(case, O, L, O_ref, L_ref, tag="f32 scale=%g" % scale)


def test_f32_rising_row_maximum():
    case = inputs.make_case(1, 2, 2, 1024, 128, "f32", False, False, seed=121)
    k = inputs.widen(case.k_bits, "f32")
    k *= (1.0 + 12.0 * np.arange(case.N) / case.N)[None, None, :, None]
    case.k_bits = inputs.round_bits(k.astype(np.float32), "f32")
    for causal in (False, True):
        case.causal = causal
        O, L = run_device(case)
        O_ref, L_ref = run_oracle(case)
        compare(case, O, L, O_ref, L_ref, tag="f32 rising causal=%d" % causal)


def test_f32_headline_shape_sampled():
    """The headline shape (B=8, Hq=32, Hkv=8, N=4096, D=128, causal) in fp32, sampled rows."""
    w = inputs.WORKLOADS["long_gqa"]
    case = inputs.make_case(w.B, w.Hq, w.Hkv, w.N, w.D, "f32", w.causal, w.padded,
                            seed=[20, w.c], scale=w.scale)
    rows = sample_rows(case, per_head=12, seed=w.c)
    log("f32 long_gqa (%d sampled rows)" % len(rows))
    O, L = run_device(case)
    O_ref, L_ref = run_oracle(case, rows=rows)
    compare(case, O, L, O_ref, L_ref, rows=rows, tag="f32 long_gqa")


# More 128-query tiles (B * Hq * ceil(N / 128)) than the 512 workgroups the device holds at
# once, every row compared: the XCD-grouped workgroup order (B * Hkv % 8 == 0) and the plain
# one, padding with an empty batch (a tile with no visible key), odd and even tile counts.
MANY = [
    ("bf16", 128, True, True, 4, 16, 4, 1100),
    ("f16", 64, False, True, 3, 24, 3, 1050),
    ("bf16", 64, True, False, 2, 40, 8, 1000),
    ("f16", 128, False, False, 9, 8, 1, 1000),
]


@pytest.mark.parametrize("cfg", MANY, ids=lambda c: "%s-D%d-c%d-p%d-B%d-H%d-%d-N%d" % c)
def test_more_tiles_than_resident_workgroups(cfg):
    dtype, D, causal, padded, B, Hq, Hkv, N = cfg
    assert B * Hq * -(-N // 128) > 512
    case = inputs.make_case(B, Hq, Hkv, N, D, dtype, causal, padded, seed=[103, D, N, B])
    log("case %s valid_len %s" % (cfg, case.valid_len))
    O, L = run_device(case)
    O_ref, L_ref = run_oracle(case)
    compare(case, O, L, O_ref, L_ref, tag=str(cfg))


@pytest.mark.parametrize("name", ["tiny", "causal_mha", "causal_padded"])
def test_workload_full(name):
    w = inputs.WORKLOADS[name]
    case = inputs.make_workload(w)
    log("workload %s (all rows)" % name)
    O, L = run_device(case)
    O_ref, L_ref = run_oracle(case)
    compare(case, O, L, O_ref, L_ref, tag=name)


def test_long_gqa_every_row():
    """The headline workload (B=8, Hq=32, Hkv=8, N=4096, D=128, bf16, causal), in the launch
    configuration the benchmark times, against the oracle on every one of its 1,048,576 rows
    (about 10 s of the oracle on 16 host threads)."""
    case = inputs.make_workload(inputs.WORKLOADS["long_gqa"])
    O, L = run_device(case)
    O_ref, L_ref = run_oracle(case)
    compare(case, O, L, O_ref, L_ref, tag="long_gqa every row")


@pytest.mark.parametrize("name", ["causal_gqa", "long_mqa"])
def test_workload_sampled(name):
    w = inputs.WORKLOADS[name]
    case = inputs.make_workload(w)
    per_head = 12 if w.B * w.Hq >= 64 else 48
    rows = sample_rows(case, per_head=per_head, seed=w.c)
    log("workload %s (%d sampled rows)" % (name, len(rows)))
    O, L = run_device(case)
    O_ref, L_ref = run_oracle(case, rows=rows)
    compare(case, O, L, O_ref, L_ref, rows=rows, tag=name)
    # properties that hold on every row: finite, bounded by max |V| of the head
    assert np.isfinite(O).all() and not np.isnan(L).any()


def test_padding_edge_values():
    """valid_len 0, negative, 1, exactly N and beyond N; causal and not."""
    for causal in (False, True):
        case = inputs.make_case(5, 4, 2, 200, 64, "f16", causal, True, seed=[5, causal],
                                valid_len=np.array([0, -7, 1, 200, 4000], np.int32))
        O, L = run_device(case)
        O_ref, L_ref = run_oracle(case)
        compare(case, O, L, O_ref, L_ref, tag="padding-edges causal=%d" % causal)
        assert np.all(O[0:2] == 0) and np.all(np.isneginf(L[0:2]))


def test_all_rows_masked():
    case = inputs.make_case(2, 4, 4, 300, 128, "bf16", True, True, seed=6,
                            valid_len=np.zeros(2, np.int32))
    O, L = run_device(case)
    assert np.all(O == 0) and np.all(np.isneginf(L))


@pytest.mark.parametrize("scale", [-0.125, 0.0, 0.5, 2.0])
def test_scale_values(scale):
    case = inputs.make_case(1, 4, 2, 257, 64, "bf16", True, True, seed=[8, 1],
                            scale=scale, valid_len=np.array([250], np.int32))
    O, L = run_device(case)
    O_ref, L_ref = run_oracle(case)
    compare(case, O, L, O_ref, L_ref, tag="scale=%g" % scale)


def test_peaked_scores():
    """Q multiplied by 8 (exact in 16 bits), K and V unchanged: very peaked softmax rows."""
    case = inputs.make_case(2, 4, 4, 512, 128, "bf16", True, False, seed=9)
    case.q_bits = inputs.round_bits((inputs.widen(case.q_bits, "bf16") * 8).astype(np.float32),
                                    "bf16")
    O, L = run_device(case)
    O_ref, L_ref = run_oracle(case)
    compare(case, O, L, O_ref, L_ref, tag="peaked")


def test_rising_row_maximum():
    """Keys scaled up along the sequence so each row's maximum keeps rising by more than the
    rescale threshold from tile to tile."""
    case = inputs.make_case(1, 2, 2, 1024, 128, "f16", False, False, seed=10)
    k = inputs.widen(case.k_bits, "f16")
    k *= (1.0 + 12.0 * np.arange(case.N) / case.N)[None, None, :, None]
    case.k_bits = inputs.round_bits(k.astype(np.float32), "f16")
    for causal in (False, True):
        case.causal = causal
        O, L = run_device(case)
        O_ref, L_ref = run_oracle(case)
        compare(case, O, L, O_ref, L_ref, tag="rising causal=%d" % causal)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("where", ["first", "last"])
def test_weights_below_the_fp16_normal_range(dtype, where):
    """One key scores 10.4 above the 4095 others, whose weights e^-10.4 ~ 3.0e-5 lie below the
    smallest normal fp16 value (6.1e-5) once rounded for P V (and, with fp16 inputs, for the row
    sum): together they hold 11 % of each row's mass, so flushing them to zero would move O by
    0.11 and LSE by 0.12. V is 0 on the large key and 1 elsewhere. With the large key last, the
    reference maximum jumps by 15 (log2 units) at the last tile and the accumulated state is
    rescaled."""
    import torch
    N, D = 4096, 64
    j = 0 if where == "first" else N - 1
    q = np.zeros((1, 2, N, D), np.float32)
    q[..., 0] = 1.0
    k = np.zeros((1, 1, N, D), np.float32)
    k[0, 0, j, 0] = 10.4
    v = np.ones((1, 1, N, D), np.float32)
    v[0, 0, j, :] = 0.0
    case = inputs.make_case(1, 2, 1, N, D, dtype, False, False, seed=12, scale=1.0)
    case.q_bits, case.k_bits, case.v_bits = (inputs.round_bits(x, dtype) for x in (q, k, v))
    O, L = run_device(case)
    O_ref, L_ref = run_oracle(case)
    assert O_ref[0, 0, 0, 0] > 0.1
    compare(case, O, L, O_ref, L_ref, tag="small weights %s %s" % (dtype, where))


@pytest.mark.parametrize("causal", [False, True])
def test_tiny_flash_attn_triton_workload(causal):
    """The workload of the Triton file's own test: B=1, H=2, N=1024, D=64, fp16 values drawn
    from N(0, 0.5), scale 0.5, seed 20."""
    case = inputs.make_case(1, 2, 2, 1024, 64, "f16", causal, False, seed=20, std=0.5,
                            scale=0.5)
    O, L = run_device(case)
    O_ref, L_ref = run_oracle(case)
    compare(case, O, L, O_ref, L_ref, tag="triton-file workload causal=%d" % causal)


def test_deterministic():
    case = inputs.make_case(2, 8, 2, 700, 128, "bf16", True, True, seed=11)
    O1, L1 = run_device(case)
    O2, L2 = run_device(case)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2, equal_nan=False)


def test_guard_regions_untouched():
    """out and lse are views into larger buffers filled with a sentinel: nothing outside the
    views may change."""
    import torch
    import scaled_dot_product_fwd_amd as sdp
    from gpu_util import to_device
    case = inputs.make_case(2, 4, 2, 333, 64, "f16", True, True, seed=12)
    q, k, v = (to_device(b, "f16") for b in (case.q_bits, case.k_bits, case.v_bits))
    vl = torch.from_numpy(case.valid_len).cuda()
    n_o, n_l, pad = q.numel(), 2 * 4 * 333, 4096
    obuf = torch.full((n_o + 2 * pad,), 1234.0, dtype=torch.float16, device="cuda")
    lbuf = torch.full((n_l + 2 * pad,), 777.0, dtype=torch.float32, device="cuda")
    out = obuf[pad:pad + n_o].view(q.shape)
    lse = lbuf[pad:pad + n_l].view(2, 4, 333)
    sdp.forward(q, k, v, causal=True, valid_len=vl, scale=case.scale, out=out, lse=lse)
    torch.cuda.synchronize()
    assert torch.all(obuf[:pad] == 1234.0) and torch.all(obuf[pad + n_o:] == 1234.0)
    assert torch.all(lbuf[:pad] == 777.0) and torch.all(lbuf[pad + n_l:] == 777.0)
    O_ref, L_ref = run_oracle(case)
    from gpu_util import from_device
    compare(case, from_device(out, "f16"), lse.cpu().numpy().astype(np.float64), O_ref, L_ref,
            tag="guarded")


def test_without_lse_and_on_side_stream():
    import torch
    case = inputs.make_case(1, 4, 4, 300, 128, "f16", True, False, seed=13)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        O, L = run_device(case, want_lse=False, stream=s)
    assert L is None
    O_ref, L_ref = run_oracle(case)
    compare(case, O, None, O_ref, L_ref, tag="no-lse side-stream")


# ---- strided inputs and outputs (attn_fwd_strided): the same logical [B, H, N, D] values as
# the oracle sees, stored in other layouts.
def _dev(bits, dtype):
    return to_device(bits, dtype)


STRIDED = [
    ("bnhd", "bf16", 128, True, True, 2, 8, 2, 333),
    ("bnhd", "f16", 64, False, False, 3, 4, 4, 200),
    ("padded_rows", "bf16", 64, True, True, 2, 6, 3, 257),
    ("padded_rows", "f16", 128, False, True, 2, 2, 1, 130),
    ("shared_kv", "bf16", 128, True, False, 3, 4, 2, 300),
    ("packed_qkv", "f16", 128, True, True, 2, 4, 4, 190),
    ("packed_qkv", "bf16", 64, False, False, 1, 8, 8, 64),
    ("strided_out", "bf16", 128, True, False, 2, 4, 1, 270),
    ("bnhd", "bf16", 32, True, True, 2, 4, 2, 200),
    ("padded_rows", "f16", 16, False, False, 2, 4, 1, 150),
    ("packed_qkv", "bf16", 16, True, False, 1, 4, 4, 100),
    ("bnhd", "f16", 256, True, False, 2, 4, 2, 300),
    ("padded_rows", "bf16", 256, False, True, 2, 2, 1, 130),
    ("bnhd", "f32", 128, True, True, 2, 4, 2, 200),
    ("padded_rows", "f32", 64, False, False, 2, 4, 1, 150),
    ("packed_qkv", "f32", 32, True, False, 1, 4, 4, 100),
    ("bnhd", "f32", 256, False, True, 2, 2, 1, 130),
    ("padded_rows", "f32", 16, True, False, 2, 4, 2, 90),
]


@pytest.mark.parametrize("cfg", STRIDED, ids=lambda c: "%s-%s-D%d-c%d-p%d-B%d-H%d-%d-N%d" % c)
def test_strided_layouts(cfg):
    import torch
    mode, dtype, D, causal, padded, B, Hq, Hkv, N = cfg
    case = inputs.make_case(B, Hq, Hkv, N, D, dtype, causal, padded, seed=[107, D, N, B])
    if mode == "shared_kv":   # one K/V for every batch: the oracle sees it repeated
        k1 = case.k_bits[:1].copy()
        v1 = case.v_bits[:1].copy()
        case.k_bits[:] = k1
        case.v_bits[:] = v1
    log("strided case %s valid_len %s" % (cfg, case.valid_len))
    vl = None
    if case.valid_len is not None:
        vl = torch.from_numpy(case.valid_len.astype(np.int32)).cuda()
    q = _dev(case.q_bits, dtype)
    k = _dev(case.k_bits, dtype)
    v = _dev(case.v_bits, dtype)
    out = None
    layout = "bhnd"
    if mode == "bnhd":
        q, k, v = (t.transpose(1, 2).contiguous() for t in (q, k, v))
        layout = "bnhd"
    elif mode == "padded_rows":
        def pad(t, extra):
            big = torch.full(t.shape[:3] + (t.shape[3] + extra,), float("nan"), dtype=t.dtype,
                             device=t.device)
            big[..., :t.shape[3]] = t
            return big[..., :t.shape[3]]
        q, k, v = pad(q, 8), pad(k, 24), pad(v, 16)
        out = pad(torch.empty_like(q), 8)
    elif mode == "shared_kv":
        k = k[:1].expand(B, -1, -1, -1)
        v = v[:1].expand(B, -1, -1, -1)
    elif mode == "packed_qkv":
        packed = torch.stack([t.transpose(1, 2) for t in (q, k, v)], dim=2).contiguous()
        q, k, v = (packed[:, :, i].transpose(1, 2) for i in range(3))
    elif mode == "strided_out":
        big = torch.full((B, N, Hq, D + 8), float("nan"), dtype=q.dtype, device=q.device)
        out = big[..., :D].transpose(1, 2)
    o, lse = sdp.forward(q, k, v, causal=causal, valid_len=vl, scale=case.scale, out=out,
                         layout=layout)
    torch.cuda.synchronize()
    if layout == "bnhd":
        o = o.transpose(1, 2)
    O = from_device(o, dtype)
    L = lse.cpu().numpy().astype(np.float64)
    O_ref, L_ref = run_oracle(case)
    compare(case, O, L, O_ref, L_ref, tag=str(cfg))
    if mode in ("padded_rows", "strided_out"):   # the padding around the output is untouched
        base = out._base if out._base is not None else out
        pad_cols = base[..., D:]
        assert torch.isnan(pad_cols.float()).all()


# ---- explicit masks (attn_fwd_masked): keep masks and additive masks, compared with the
# oracle given the exact mask values the device reads.
MASKED = [
    # (kind, pattern, dtype, D, causal, padded, B, Hq, Hkv, N)
    ("keep", "random_bh", "bf16", 128, True, True, 2, 4, 2, 300),
    ("keep", "window", "f16", 64, False, False, 2, 4, 4, 256),
    ("keep", "random_b", "f16", 128, False, True, 3, 2, 1, 1000),
    ("keep", "empty_rows", "bf16", 64, True, False, 1, 4, 2, 130),
    ("add", "random_bh", "bf16", 128, True, False, 2, 4, 2, 257),
    ("add", "alibi", "bf16", 64, True, True, 2, 8, 2, 512),
    ("add", "random_b", "f16", 64, False, True, 2, 4, 1, 200),
    ("add", "large_negative", "f16", 128, False, False, 1, 2, 2, 64),
    # rows whose first tiles are wholly hidden while other rows of the wave rescale
    ("add", "window_neginf", "bf16", 128, False, False, 2, 4, 4, 300),
    ("keep", "random_bh", "f16", 16, True, True, 2, 4, 2, 200),
    ("add", "alibi", "bf16", 32, False, False, 2, 4, 1, 300),
    ("keep", "window", "bf16", 256, True, False, 2, 4, 2, 300),
    ("add", "random_bh", "f16", 256, False, True, 2, 2, 1, 200),
    # fp32 inputs: uint8 keep masks and fp32 additive masks
    ("keep", "random_bh", "f32", 128, True, True, 2, 4, 2, 300),
    ("keep", "window", "f32", 64, False, False, 2, 4, 4, 256),
    ("keep", "empty_rows", "f32", 32, True, False, 1, 4, 2, 130),
    ("keep", "random_b", "f32", 16, False, True, 3, 2, 1, 200),
    ("add", "random_bh", "f32", 128, True, False, 2, 4, 2, 257),
    ("add", "alibi", "f32", 64, True, True, 2, 8, 2, 512),
    ("add", "window_neginf", "f32", 128, False, False, 2, 4, 4, 300),
    ("add", "large_negative", "f32", 32, False, False, 1, 2, 2, 64),
    ("add", "random_b", "f32", 16, True, True, 2, 4, 1, 100),
    ("keep", "random_bh", "f32", 256, True, True, 2, 2, 1, 200),
    ("add", "alibi", "f32", 256, False, False, 1, 4, 2, 300),
]


@pytest.mark.parametrize("cfg", MASKED, ids=lambda c: "%s-%s-%s-D%d-c%d-p%d-B%d-H%d-%d-N%d" % c)
def test_explicit_masks(cfg):
    import torch
    kind, pattern, dtype, D, causal, padded, B, Hq, Hkv, N = cfg
    case = inputs.make_case(B, Hq, Hkv, N, D, dtype, causal, padded, seed=[109, D, N, B])
    rng = np.random.default_rng([113, D, N, B])
    mv = mask_values(kind, pattern, dtype, B, Hq, N, rng)
    log("masked case %s valid_len %s mask %s" % (cfg, case.valid_len, mv.shape))
    dmask = device_mask(kind, pattern, dtype, mv, N)
    vl = None
    if case.valid_len is not None:
        vl = torch.from_numpy(case.valid_len.astype(np.int32)).cuda()
    q, k, v = (_dev(b, dtype) for b in (case.q_bits, case.k_bits, case.v_bits))
    o, lse = sdp.forward(q, k, v, causal=causal, valid_len=vl, scale=case.scale,
                         attn_mask=dmask)
    torch.cuda.synchronize()
    O = from_device(o, dtype)
    L = lse.cpu().numpy().astype(np.float64)
    if kind == "keep":
        O_ref, L_ref = run_oracle_masked(case, keep_mask=mv)
    else:
        O_ref, L_ref = run_oracle_masked(case, add_mask=inputs.widen(mv, dtype))
    compare(case, O, L, O_ref, L_ref, tag=str(cfg))
