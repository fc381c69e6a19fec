"""Parity of the HIP path (through the C ABI) with the fp64 oracle, element by element.

Small cases compare every output; the full-size workloads compare a sample of rows (every
(batch, head), first/last rows, tile edges, rows around valid_len, random rows) that the oracle
computes one by one, with the HIP path run in the same launch configuration the benchmark
times.
"""
import numpy as np
import pytest

from gpu_util import compare, log, run_device, run_oracle, sample_rows
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


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: "%s-D%d-c%d-p%d-B%d-H%d-%d-N%d" % c)
def test_small_full(cfg):
    dtype, D, causal, padded, B, Hq, Hkv, N = cfg
    case = inputs.make_case(B, Hq, Hkv, N, D, dtype, causal, padded, seed=[101, D, N, B])
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


@pytest.mark.parametrize("name", ["causal_gqa", "long_gqa", "long_mqa"])
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
