"""attn_bwd_scratch, the backward on the library's static device workspace (for callers that
cannot allocate), against attn_bwd_ws given a caller-owned workspace of the same size
(ATTN_SCRATCH_FLOATS floats, hence the same dK/dV split): the gradients must be bitwise equal.
Two calls go out back to back on one stream, the second with a smaller input over whatever the
first left in the shared array; a third mixes in an explicit mask and fp32 tensors."""
import numpy as np
import pytest

from gpu_util import from_device, log, to_device
import scaled_dot_product_fwd_amd as sdp
from scaled_dot_product_fwd_amd import inputs

GB = 1 << 30


def test_scratch_rejects_sizes_beyond_its_array():
    # host-side check, before any HIP call: 2 * B * Hq * N = 8388864 > ATTN_SCRATCH_FLOATS
    B, Hq, Hkv, N, D = 1, 128, 8, 32769, 128
    assert 2 * B * Hq * N > sdp.ATTN_SCRATCH_FLOATS
    st = sdp.attn_bwd_scratch(1 * GB, None, 3 * GB, None, 5 * GB, None, 7 * GB, None, 9 * GB,
                              None, 11 * GB, 13 * GB, None, 15 * GB, None, 17 * GB, None, B, Hq,
                              Hkv, N, D, 0.088, 1, None, None, sdp.ATTN_MASK_NONE, None,
                              sdp.ATTN_BF16, None)
    assert st == sdp.ATTN_ERR_SCRATCH
    assert "ATTN_SCRATCH_FLOATS" in sdp.attn_status_string(st)


def _prepare(dtype, D, causal, padded, B, Hq, Hkv, N, seed, keep_mask=False):
    import torch
    case = inputs.make_case(B, Hq, Hkv, N, D, dtype, causal, padded, seed=seed)
    dout = inputs.make_grad(case, seed)
    t = {name: to_device(bits, dtype) for name, bits in
         (("q", case.q_bits), ("k", case.k_bits), ("v", case.v_bits), ("do", dout))}
    t["vl"] = (torch.from_numpy(case.valid_len.astype(np.int32)).cuda()
               if case.valid_len is not None else None)
    t["mask"] = None
    if keep_mask:
        rng = np.random.default_rng(seed)
        m = (rng.random((B, Hq, N, N)) < 0.7).astype(np.uint8)
        m[..., 0] = 1
        t["mask"] = torch.from_numpy(m).cuda()
    out, lse = sdp.forward(t["q"], t["k"], t["v"], causal=causal, valid_len=t["vl"],
                           scale=case.scale, attn_mask=t["mask"])
    t["out"], t["lse"] = out, lse
    return case, t


def _call(case, t, grads, ws=None):
    import torch
    mask = t["mask"]
    args_in = (t["q"].data_ptr(), None, t["k"].data_ptr(), None, t["v"].data_ptr(), None,
               t["out"].data_ptr(), None, t["do"].data_ptr(), None, t["lse"].data_ptr(),
               grads[0].data_ptr(), None, grads[1].data_ptr(), None, grads[2].data_ptr(), None)
    code = {"bf16": sdp.ATTN_BF16, "f16": sdp.ATTN_F16, "f32": sdp.ATTN_F32}[case.dtype]
    tail = (case.B, case.Hq, case.Hkv, case.N, case.D, case.scale, case.causal,
            t["vl"].data_ptr() if t["vl"] is not None else None,
            mask.data_ptr() if mask is not None else None,
            sdp.ATTN_MASK_KEEP_U8 if mask is not None else sdp.ATTN_MASK_NONE,
            [case.Hq * case.N * case.N, case.N * case.N, case.N] if mask is not None else None,
            code, torch.cuda.current_stream().cuda_stream)
    if ws is None:
        return sdp.attn_bwd_scratch(*args_in, *tail)
    return sdp.attn_bwd_ws(*args_in, ws.data_ptr(), ws.numel(), *tail)


def _grads(t):
    import torch
    return [torch.full_like(t["q"], float("nan")), torch.full_like(t["k"], float("nan")),
            torch.full_like(t["v"], float("nan"))]


CASES = [
    # (dtype, D, causal, padded, B, Hq, Hkv, N, seed, keep_mask): MQA with a dK/dV split of 8
    # in the static array, then a smaller padded GQA case, then fp32 with a keep mask
    ("bf16", 128, True, False, 1, 32, 1, 2048, 311, False),
    ("f16", 64, True, True, 2, 4, 2, 200, 313, False),
    ("f32", 64, False, True, 2, 4, 2, 144, 317, True),
]


@pytest.mark.gpu
def test_scratch_matches_workspace_entry_point():
    import torch
    prepared = [_prepare(*c) for c in CASES]
    torch.cuda.synchronize()
    # the allocation-free calls, back to back on one stream
    got = []
    for cfg, (case, t) in zip(CASES, prepared):
        log("attn_bwd_scratch case %s" % (cfg,))
        g = _grads(t)
        assert _call(case, t, g) == sdp.ATTN_OK
        got.append(g)
    torch.cuda.synchronize()
    for cfg, (case, t), g in zip(CASES, prepared, got):
        ws = torch.full((sdp.ATTN_SCRATCH_FLOATS,), float("nan"), dtype=torch.float32,
                        device=t["q"].device)
        ref = _grads(t)
        assert _call(case, t, ref, ws) == sdp.ATTN_OK
        torch.cuda.synchronize()
        for name, a, b in zip(("dQ", "dK", "dV"), g, ref):
            x, y = from_device(a, case.dtype), from_device(b, case.dtype)
            assert np.isfinite(x).all(), (cfg, name)
            assert np.array_equal(x, y), (cfg, name, np.abs(x - y).max())
        log("  bitwise equal to attn_bwd_ws: %s" % (cfg,))
    # the first case again, after the smaller ones: still the same gradients
    case, t = prepared[0]
    g = _grads(t)
    assert _call(case, t, g) == sdp.ATTN_OK
    torch.cuda.synchronize()
    for a, b in zip(g, got[0]):
        assert torch.equal(a, b)
