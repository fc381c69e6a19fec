"""The forward and the allocation-free backward captured in a HIP graph (torch.cuda.CUDAGraph):
every replay must reproduce the eager results bit for bit (the kernels are deterministic), with
eager work and synchronisations between the replays, and a replay after the captured input
tensors were overwritten in place must match an eager call on the new values.

The captured calls allocate nothing: forward() gets its O and LSE tensors, attn_bwd_scratch
runs on the library's static device array; the library records no memset."""
import numpy as np
import pytest

from gpu_util import log, to_device
import scaled_dot_product_fwd_amd as sdp
from scaled_dot_product_fwd_amd import inputs

pytestmark = pytest.mark.gpu

# B, Hq, Hkv, N, D: one-pass forward (16 key tiles per row block), dK/dV split in two parts
SHAPE = (2, 8, 2, 1000, 128)


def _tensors(seed):
    B, Hq, Hkv, N, D = SHAPE
    case = inputs.make_case(B, Hq, Hkv, N, D, "bf16", True, False, seed=seed)
    dout = inputs.make_grad(case, seed)
    return case, [to_device(b, "bf16") for b in (case.q_bits, case.k_bits, case.v_bits, dout)]


def _step(case, q, k, v, do, out, lse, dq, dk, dv):
    """forward, then attn_bwd_scratch, on the current stream, into the given tensors"""
    import torch
    B, Hq, Hkv, N, D = SHAPE
    sdp.forward(q, k, v, causal=True, scale=case.scale, out=out, lse=lse, split=False)
    st = sdp.attn_bwd_scratch(
        q.data_ptr(), None, k.data_ptr(), None, v.data_ptr(), None, out.data_ptr(), None,
        do.data_ptr(), None, lse.data_ptr(), dq.data_ptr(), None, dk.data_ptr(), None,
        dv.data_ptr(), None, B, Hq, Hkv, N, D, case.scale, True, None, None, sdp.ATTN_MASK_NONE,
        None, sdp.ATTN_BF16, torch.cuda.current_stream().cuda_stream)
    assert st == sdp.ATTN_OK, sdp.attn_status_string(st)


def test_forward_backward_graph_replays():
    import torch
    case, (q, k, v, do) = _tensors(401)
    outs = [torch.empty_like(q), torch.empty(q.shape[:3], dtype=torch.float32, device=q.device),
            torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)]
    ref = [torch.empty_like(t) for t in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _step(case, q, k, v, do, *ref)          # eager, also the static array's first use
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _step(case, q, k, v, do, *outs)
    names = ("O", "LSE", "dQ", "dK", "dV")
    for rep in range(3):
        for t in outs:
            t.fill_(float("nan"))
        # unrelated eager work on the device between replays
        x = torch.randn(1 << 20, device=q.device)
        float((x * x).sum())
        graph.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(names, outs, ref):
            assert torch.equal(a, b), "replay %d: %s differs from the eager call" % (rep, name)
        log("graph replay %d matches the eager call" % rep)
    # new values in the captured input tensors: the replay reads them
    case2, (q2, k2, v2, do2) = _tensors(403)
    for dst, src in zip((q, k, v, do), (q2, k2, v2, do2)):
        dst.copy_(src)
    _step(case, q, k, v, do, *ref)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    for name, a, b in zip(names, outs, ref):
        assert torch.equal(a, b), "replay on new inputs: %s differs" % name
    assert not np.isnan(outs[2].float().cpu().numpy()).any()
    log("graph replay on new inputs matches the eager call")
