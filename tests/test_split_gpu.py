"""Parity of the split forward (attn_fwd_ws: each query tile's key range cut into chunks that
run as separate workgroups, then merged by their log-sum-exp) with the fp64 oracle, on grids
small enough that the split applies: every row compared, at the tolerances of the one-pass
kernel. Covers rows with no visible key, valid_len at and around tile edges, ragged N, chunks of
two and three key tiles (chunk boundaries at and inside the causal diagonal), GQA / MQA, every
head dimension, strided [B, N, H, D] tensors and workspaces too small for the full split."""
import numpy as np
import pytest

from gpu_util import compare, from_device, log, run_device, run_oracle, to_device
import scaled_dot_product_fwd_amd as sdp
from scaled_dot_product_fwd_amd import inputs

pytestmark = pytest.mark.gpu


def split_size(case):
    return sdp.attn_fwd_workspace_floats(case.B, case.Hq, case.Hkv, case.N, case.D, case.causal)


# (dtype, D, causal, B, Hq, Hkv, N, valid_len or None): few query tiles over long key ranges
# (the split applies: at most 128 query tiles, 64 at D = 256, and at least 48 key tiles)
CASES = [
    # 64 query tiles over up to 64 key tiles
    ("f16", 64, True, 1, 2, 2, 4096, None),
    # chunks of 2 key tiles: a chunk boundary at the start of every diagonal pair of tiles
    ("bf16", 128, True, 1, 1, 1, 3072, None),
    # chunks of 3 key tiles: the two diagonal tiles of some query tiles fall into different
    # chunks (causal), and a non-causal case
    ("bf16", 64, True, 1, 1, 1, 4200, None),
    ("f16", 64, False, 1, 1, 1, 3200, None),
    # valid_len: an empty batch, one key, a tile edge, ragged
    ("f16", 64, True, 4, 1, 1, 3200, [0, 1, 64, 3199]),
    ("bf16", 128, True, 2, 2, 1, 3500, [0, 3000]),
    ("bf16", 64, True, 1, 2, 2, 8192, [4097]),
    # MQA, non-causal, ragged
    ("f16", 128, False, 1, 4, 1, 3100, None),
    # head dims 16, 32 (the D = 64 geometry) and 256 (one workgroup per CU)
    ("bf16", 16, True, 1, 4, 2, 4000, None),
    ("f16", 32, False, 2, 1, 1, 3300, [3300, 1]),
    ("bf16", 256, True, 1, 1, 1, 6000, None),
    ("f16", 256, False, 1, 2, 1, 3200, None),
]


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: "%s-D%d-c%d-B%d-H%d-%d-N%d" % c[:7])
def test_split_matches_oracle(cfg):
    dtype, D, causal, B, Hq, Hkv, N, vl = cfg
    case = inputs.make_case(B, Hq, Hkv, N, D, dtype, causal, vl is not None,
                            seed=[401, D, N, B],
                            valid_len=np.array(vl, np.int32) if vl is not None else None)
    assert split_size(case) > 0, "no split for %s" % (cfg,)
    log("split case %s: workspace %d floats" % (cfg, split_size(case)))
    O, L = run_device(case, split=True)
    O_ref, L_ref = run_oracle(case)
    compare(case, O, L, O_ref, L_ref, tag="split %s" % (cfg,))
    if vl is not None:
        for b, n in enumerate(vl):
            if n <= 0:
                assert np.all(O[b] == 0) and np.all(np.isneginf(L[b]))


def test_split_deterministic_and_close_to_one_pass():
    case = inputs.make_case(1, 2, 2, 8192, 64, "f16", True, False, seed=403)
    a = run_device(case, split=True)
    b = run_device(case, split=True)
    c = run_device(case, split=False)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    d_o = np.abs(a[0] - c[0]).max()
    d_l = np.abs(a[1] - c[1]).max()
    log("split vs one-pass: max|dO| %.3g max|dLSE| %.3g" % (d_o, d_l))
    assert d_o <= 5e-3 and d_l <= 1e-3


@pytest.mark.parametrize("frac", [0.5, 0.2, 0.0])
def test_split_with_smaller_workspaces(frac):
    """A workspace below attn_fwd_workspace_floats gets a coarser split (or none); the result
    still matches the oracle."""
    import torch
    case = inputs.make_case(1, 2, 2, 4096, 128, "bf16", True, False, seed=405)
    q, k, v = (to_device(x, "bf16") for x in (case.q_bits, case.k_bits, case.v_bits))
    full = split_size(case)
    assert full > 0
    n = int(full * frac)
    ws = torch.empty((max(n, 1),), dtype=torch.float32, device="cuda")
    out, lse = torch.empty_like(q), torch.empty((1, 2, 4096), dtype=torch.float32, device="cuda")
    st = sdp.attn_fwd_ws(q.data_ptr(), None, k.data_ptr(), None, v.data_ptr(), None,
                         out.data_ptr(), None, lse.data_ptr(), ws.data_ptr(), n, 1, 2, 2, 4096,
                         128, case.scale, True, None, sdp.ATTN_BF16,
                         torch.cuda.current_stream().cuda_stream)
    assert st == sdp.ATTN_OK
    torch.cuda.synchronize()
    O, L = from_device(out, "bf16"), lse.cpu().numpy().astype(np.float64)
    O_ref, L_ref = run_oracle(case)
    compare(case, O, L, O_ref, L_ref, tag="split ws %d of %d floats" % (n, full))


def test_split_strided_bnhd():
    """[B, N, H, D] tensors (strided rows) through the split."""
    import torch
    case = inputs.make_case(2, 2, 1, 3500, 64, "bf16", True, True, seed=407,
                            valid_len=np.array([3500, 1750], np.int32))
    assert split_size(case) > 0
    q, k, v = (to_device(x, "bf16").transpose(1, 2).contiguous()
               for x in (case.q_bits, case.k_bits, case.v_bits))
    vl = torch.from_numpy(case.valid_len).cuda()
    out, lse = sdp.forward(q, k, v, causal=True, valid_len=vl, scale=case.scale, layout="bnhd")
    torch.cuda.synchronize()
    O = from_device(out.transpose(1, 2), "bf16")
    L = lse.cpu().numpy().astype(np.float64)
    O_ref, L_ref = run_oracle(case)
    compare(case, O, L, O_ref, L_ref, tag="split bnhd")


def test_split_without_lse():
    """forward(want_lse=False): the split writes O only (the merge kernel skips the LSE)."""
    import torch
    case = inputs.make_case(1, 2, 2, 4096, 64, "f16", True, True, seed=409,
                            valid_len=np.array([3000], np.int32))
    assert split_size(case) > 0
    O, L = run_device(case, want_lse=False, split=True)
    assert L is None
    O_ref, _ = run_oracle(case)
    err = np.abs(O - O_ref).max()
    log("split without LSE: max|dO| %.3g" % err)
    assert err <= 5e-3


def test_f32_ignores_the_workspace():
    """fp32 inputs never split: attn_fwd_ws runs the one-pass fp32 kernel and leaves the
    workspace untouched."""
    import torch
    case = inputs.make_case(1, 2, 2, 3200, 64, "f32", True, False, seed=411)
    q, k, v = (to_device(x, "f32") for x in (case.q_bits, case.k_bits, case.v_bits))
    out = torch.empty_like(q)
    lse = torch.empty((1, 2, 3200), dtype=torch.float32, device="cuda")
    n = sdp.attn_fwd_workspace_floats(1, 2, 2, 3200, 64, True)
    assert n > 0   # these sizes would split with 16-bit inputs
    ws = torch.full((n,), 7.0, dtype=torch.float32, device="cuda")
    st = sdp.attn_fwd_ws(q.data_ptr(), None, k.data_ptr(), None, v.data_ptr(), None,
                         out.data_ptr(), None, lse.data_ptr(), ws.data_ptr(), n, 1, 2, 2, 3200,
                         64, case.scale, True, None, sdp.ATTN_F32,
                         torch.cuda.current_stream().cuda_stream)
    assert st == sdp.ATTN_OK
    torch.cuda.synchronize()
    assert torch.all(ws == 7.0)
    O, L = from_device(out, "f32"), lse.cpu().numpy().astype(np.float64)
    O_ref, L_ref = run_oracle(case)
    compare(case, O, L, O_ref, L_ref, tag="f32 through attn_fwd_ws")
