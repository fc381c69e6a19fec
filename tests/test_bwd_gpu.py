"""Parity of the backward pass (attn_bwd through the C ABI) with the fp64 oracle's gradients.

The device forward produces O and LSE; attn_bwd consumes them with the upstream gradient dO.
The oracle recomputes everything from Q, K, V, dO in fp64. Each gradient tensor G is compared
as max |G - G_ref| / max(max |G_ref|, GRAD_FLOOR) (relative to the tensor's largest gradient),
within BWD_TOL;
gradients that must vanish (rows with no visible key in dQ, keys no query sees in dK and dV)
must be exactly 0, and Delta (the row sums of dO * O) within DELTA_TOL of the oracle's.
"""
import numpy as np
import pytest

from gpu_util import from_device, log, to_device
import oracle
import scaled_dot_product_fwd_amd as sdp
from scaled_dot_product_fwd_amd import inputs

pytestmark = pytest.mark.gpu

# fp32: every product and sum in fp32 (no 16-bit rounding of P or dS); 1e-4 of the largest
# gradient leaves room for fp32 accumulation over a few thousand keys (~1e-6 relative each).
BWD_TOL = {"bf16": 2e-2, "f16": 5e-3, "f32": 1e-4}
# Normaliser floor: where every gradient of a tensor cancels to ~0 in exact arithmetic (one key
# per row, so dS = P (dP - D) = 0), the device's rounding leaves values near 1e-7 that are
# compared against this floor instead of against 0. In fp32 the residue of that cancellation is
# the rounding of dP and D themselves (|dO| |v| ~ sqrt(D) times ~1e-7: ~2e-6 in dQ, and dK, dV
# sum it over every query row of the group, ~5e-6 at 200 rows), so a fully cancelling fp32
# tensor is held to 1e-5 absolute: a floor of 1e-5 / 1e-4.
GRAD_FLOOR = {"bf16": 1e-3, "f16": 1e-3, "f32": 1e-1}
DELTA_TOL = {"bf16": 2e-2, "f16": 5e-3, "f32": 1e-4}


def run_bwd(case, dout_bits, dout_scale=1.0, split_ws=False):
    """Forward, then backward through backward(); split_ws passes the workspace size of
    attn_bwd_workspace_floats (attn_bwd_ws, the dK/dV split where the shape wants one) instead
    of the minimal 2 * B * Hq * N values (attn_bwd)."""
    import torch
    q = to_device(case.q_bits, case.dtype)
    k = to_device(case.k_bits, case.dtype)
    v = to_device(case.v_bits, case.dtype)
    do = to_device(dout_bits, case.dtype)
    vl = None
    if case.valid_len is not None:
        vl = torch.from_numpy(case.valid_len.astype(np.int32)).cuda()
    out, lse = sdp.forward(q, k, v, causal=case.causal, valid_len=vl, scale=case.scale)
    base = 2 * lse.numel()
    n_ws = sdp.attn_bwd_workspace_floats(case.B, case.Hq, case.Hkv, case.N, case.D) \
        if split_ws else base
    ws = torch.empty((n_ws,), dtype=torch.float32, device=q.device)
    dq, dk, dv = sdp.backward(q, k, v, out, do, lse, causal=case.causal, valid_len=vl,
                              scale=case.scale, ws=ws)
    torch.cuda.synchronize()
    L = lse.cpu().numpy()
    # the workspace's second row is the device's LSE in base 2 (0 on empty rows)
    ws = ws[:base].view((2,) + tuple(lse.shape))
    l2 = ws[1].cpu().numpy()
    want = np.where(np.isneginf(L), np.float32(0), L * np.float32(1.4426950408889634))
    assert np.allclose(l2, want, rtol=1e-6, atol=0), "workspace LSE row"
    return (from_device(dq, case.dtype), from_device(dk, case.dtype),
            from_device(dv, case.dtype), ws[0].cpu().numpy().astype(np.float64),
            from_device(out, case.dtype), L.astype(np.float64))


def visibility(case):
    """(rows with a visible key [B,N], keys some query sees [B,N]) from causal / valid_len."""
    N = case.N
    valid = np.full(case.B, N, np.int64)
    if case.valid_len is not None:
        valid = np.clip(case.valid_len.astype(np.int64), 0, N)
    idx = np.arange(N)
    # padding hides keys j >= valid only; key 0 is visible to every row (also under the causal
    # mask) once valid >= 1, and key j < valid is seen at least by query j
    row_has = np.broadcast_to((valid >= 1)[:, None], (case.B, N))
    key_seen = idx[None, :] < valid[:, None]
    return row_has, key_seen


def check_grad(name, got, ref, dtype, tag, zero=None):
    assert np.isfinite(got).all(), "%s %s: non-finite values" % (tag, name)
    if zero is not None and zero.any():
        assert np.all(got[zero] == 0.0), "%s %s: gradients that must vanish are not 0" % (
            tag, name)
    scale = max(np.abs(ref).max(), GRAD_FLOOR[dtype])
    err = np.abs(got - ref).max() if got.size else 0.0
    rel = err / scale
    assert rel <= BWD_TOL[dtype], "%s %s: max err %.3g = %.3g of max |ref| %.3g" % (
        tag, name, err, rel, scale)
    return rel


def compare_case(case, dout_bits, tag, split_ws=False):
    dq, dk, dv, delta, O, L = run_bwd(case, dout_bits, split_ws=split_ws)
    q, k, v = case.widened()
    do = inputs.widen(dout_bits, case.dtype)
    rq, rk, rv = oracle.attn_bwd(q, k, v, do, case.scale, case.causal, case.valid_len)
    O_ref, _ = oracle.attn_fwd(q, k, v, case.scale, case.causal, case.valid_len)
    row_has, key_seen = visibility(case)
    zq = np.broadcast_to(~row_has[:, None, :, None], dq.shape)
    zk = np.broadcast_to(~key_seen[:, None, :, None], dk.shape)
    e = [check_grad("dQ", dq, rq, case.dtype, tag, zq),
         check_grad("dK", dk, rk, case.dtype, tag, zk),
         check_grad("dV", dv, rv, case.dtype, tag, zk)]
    d_ref = (do * O_ref).sum(-1)
    derr = np.abs(delta - d_ref).max()
    dscale = max(np.abs(d_ref).max(), 1.0)
    assert derr / dscale <= DELTA_TOL[case.dtype], "%s Delta err %.3g" % (tag, derr)
    log("%s: rel err dQ %.2e dK %.2e dV %.2e Delta %.2e" % (tag, e[0], e[1], e[2],
                                                             derr / dscale))
    return e


# (dtype, D, causal, padded, B, Hq, Hkv, N): ragged N, N below one tile, exact tiles, GQA, MQA,
# head dims 16 / 32 (the D = 64 geometry with zero-filled chunks) and 64 / 128.
BWD_SMALL = [
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
    ("bf16", 128, True, True, 2, 2, 2, 640),
    ("bf16", 64, True, False, 1, 8, 1, 520),
    ("bf16", 128, False, False, 1, 2, 1, 1),
    ("f16", 16, True, True, 3, 4, 2, 257),
    ("bf16", 16, False, False, 1, 4, 4, 300),
    ("bf16", 32, True, False, 2, 8, 2, 333),
    ("f16", 32, False, True, 2, 6, 3, 1000),
    ("bf16", 16, True, False, 2, 2, 1, 1),
    # fp32 (attn_bwd_f32.hip): head dims 16 (the D = 32 geometry, half zeros), 32, 64, 128
    ("f32", 128, True, False, 2, 8, 2, 333),
    ("f32", 128, False, True, 2, 4, 2, 129),
    ("f32", 64, True, True, 3, 4, 2, 257),
    ("f32", 64, False, False, 1, 2, 2, 128),
    ("f32", 32, True, False, 2, 8, 2, 333),
    ("f32", 32, False, True, 2, 6, 3, 100),
    ("f32", 16, True, True, 3, 4, 2, 257),
    ("f32", 16, False, False, 1, 4, 4, 300),
    ("f32", 128, True, True, 2, 6, 3, 1),
    # D = 256 (16-bit): two head-dimension parts per kernel
    ("bf16", 256, True, False, 2, 8, 2, 333),
    ("f16", 256, False, True, 2, 4, 2, 257),
    ("bf16", 256, True, True, 3, 4, 1, 130),
    ("f16", 256, True, False, 1, 2, 2, 1),
    # D = 256 (fp32): two (dQ) and four (dK/dV) head-dimension parts
    ("f32", 256, True, False, 2, 8, 2, 333),
    ("f32", 256, False, True, 2, 4, 2, 257),
    ("f32", 256, True, True, 3, 4, 1, 130),
    ("f32", 256, True, False, 1, 2, 2, 1),
]


@pytest.mark.parametrize("cfg", BWD_SMALL, ids=lambda c: "%s-D%d-c%d-p%d-B%d-H%d-%d-N%d" % c)
def test_bwd_small_full(cfg):
    dtype, D, causal, padded, B, Hq, Hkv, N = cfg
    case = inputs.make_case(B, Hq, Hkv, N, D, dtype, causal, padded, seed=[201, D, N, B])
    dout = inputs.make_grad(case, [201, D, N, B])
    log("bwd case %s valid_len %s" % (cfg, case.valid_len))
    compare_case(case, dout, str(cfg))


# More query tiles and key tiles than the device holds workgroups at once, every element
# compared: the XCD-grouped order (B * Hkv % 8 == 0) and the plain one, an empty batch.
BWD_MANY = [
    ("bf16", 128, True, True, 4, 16, 4, 1100),
    ("f16", 64, False, True, 3, 24, 3, 1050),
    ("bf16", 64, True, False, 2, 40, 8, 1000),
    ("f32", 128, True, True, 4, 16, 4, 1100),
    ("f32", 64, False, False, 3, 24, 3, 700),
    ("bf16", 256, True, True, 4, 16, 4, 600),
    ("f32", 256, True, True, 4, 16, 4, 600),
]


@pytest.mark.parametrize("cfg", BWD_MANY, ids=lambda c: "%s-D%d-c%d-p%d-B%d-H%d-%d-N%d" % c)
def test_bwd_many_tiles(cfg):
    dtype, D, causal, padded, B, Hq, Hkv, N = cfg
    case = inputs.make_case(B, Hq, Hkv, N, D, dtype, causal, padded, seed=[203, D, N, B])
    dout = inputs.make_grad(case, [203, D, N, B])
    log("bwd case %s valid_len %s" % (cfg, case.valid_len))
    compare_case(case, dout, str(cfg))


def test_bwd_padding_edge_values():
    """valid_len 0, negative, 1, exactly N and beyond N; causal and not."""
    for causal in (False, True):
        case = inputs.make_case(5, 4, 2, 200, 64, "f16", causal, True, seed=[205, causal],
                                valid_len=np.array([0, -7, 1, 200, 4000], np.int32))
        dout = inputs.make_grad(case, [205, causal])
        log("bwd padding edges causal=%d" % causal)
        compare_case(case, dout, "bwd padding-edges causal=%d" % causal)


@pytest.mark.parametrize("scale", [-0.125, 0.0, 0.5, 2.0])
def test_bwd_scale_values(scale):
    case = inputs.make_case(1, 4, 2, 257, 64, "bf16", True, True, seed=[207, 1],
                            scale=scale, valid_len=np.array([250], np.int32))
    dout = inputs.make_grad(case, [207, 1])
    log("bwd scale %g" % scale)
    compare_case(case, dout, "bwd scale=%g" % scale)


@pytest.mark.parametrize("scale", [-0.125, 0.0, 2.0])
def test_bwd_f32_scale_values(scale):
    case = inputs.make_case(1, 4, 2, 200, 128, "f32", True, True, seed=[225, 1],
                            scale=scale, valid_len=np.array([190], np.int32))
    dout = inputs.make_grad(case, [225, 1])
    log("bwd f32 scale %g" % scale)
    compare_case(case, dout, "bwd f32 scale=%g" % scale)


def test_bwd_f32_padding_edge_values():
    """fp32: valid_len 0, negative, 1, exactly N and beyond N; causal and not."""
    for causal in (False, True):
        case = inputs.make_case(5, 4, 2, 150, 64, "f32", causal, True, seed=[227, causal],
                                valid_len=np.array([0, -7, 1, 150, 4000], np.int32))
        dout = inputs.make_grad(case, [227, causal])
        log("bwd f32 padding edges causal=%d" % causal)
        compare_case(case, dout, "bwd f32 padding-edges causal=%d" % causal)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_bwd_deterministic(dtype):
    """No atomics: two calls give bitwise equal gradients and workspace."""
    case = inputs.make_case(2, 8, 2, 700, 128, dtype, True, True, seed=[231, len(dtype)])
    dout = inputs.make_grad(case, [231, len(dtype)])
    a = run_bwd(case, dout)
    b = run_bwd(case, dout)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_bwd_guard_regions_untouched():
    """dq, dk, dv and ws are views into larger buffers filled with a sentinel: nothing outside
    the views may change, and the gradients inside still match the oracle."""
    import torch
    case = inputs.make_case(2, 4, 2, 333, 64, "f16", True, True, seed=233)
    dout_bits = inputs.make_grad(case, 233)
    q, k, v = (to_device(x, "f16") for x in (case.q_bits, case.k_bits, case.v_bits))
    do = to_device(dout_bits, "f16")
    vl = torch.from_numpy(case.valid_len).cuda()
    out, lse = sdp.forward(q, k, v, causal=True, valid_len=vl, scale=case.scale)
    pad = 4096

    def guarded(shape, dtype, value):
        n = int(np.prod(shape))
        buf = torch.full((n + 2 * pad,), value, dtype=dtype, device="cuda")
        return buf, buf[pad:pad + n].view(shape), n, value

    g = [guarded(tuple(q.shape), torch.float16, 1234.0),
         guarded(tuple(k.shape), torch.float16, -55.0),
         guarded(tuple(v.shape), torch.float16, 99.0),
         guarded((2,) + tuple(lse.shape), torch.float32, 777.0)]
    sdp.backward(q, k, v, out, do, lse, causal=True, valid_len=vl, scale=case.scale,
                 dq=g[0][1], dk=g[1][1], dv=g[2][1], ws=g[3][1])
    torch.cuda.synchronize()
    for buf, _, n, value in g:
        assert torch.all(buf[:pad] == value) and torch.all(buf[pad + n:] == value)
    qw, kw, vw = case.widened()
    ref = oracle.attn_bwd(qw, kw, vw, inputs.widen(dout_bits, "f16"), case.scale, True,
                          case.valid_len)
    for name, (_, view, _, _), r in zip(("dQ", "dK", "dV"), g[:3], ref):
        check_grad(name, from_device(view, "f16"), r, "f16", "guarded")


@pytest.mark.parametrize("dtype", ["f16", "f32"])
def test_bwd_on_side_stream(dtype):
    """forward and backward queued on a non-default stream (torch's current stream)."""
    import torch
    case = inputs.make_case(1, 4, 4, 300, 128, dtype, True, False, seed=[235, len(dtype)])
    dout = inputs.make_grad(case, [235, len(dtype)])
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        compare_case(case, dout, "side stream %s" % dtype)


# ---- the dK/dV split of attn_bwd_ws: key tiles whose (query head, query tile) iterations are
# shared by several workgroups, partial sums added in a fixed order. Shapes with few key tiles
# and long groups (MQA), where attn_bwd_workspace_floats asks for a split of 2 to 16.
BWD_SPLIT = [
    # (dtype, D, causal, padded, B, Hq, Hkv, N)
    ("bf16", 64, True, False, 1, 8, 1, 1024),
    ("f16", 128, False, True, 2, 16, 2, 700),
    ("bf16", 128, True, False, 1, 32, 1, 2048),
    ("f16", 32, True, False, 1, 16, 1, 1500),
    ("f32", 64, True, False, 1, 8, 1, 1024),
    ("f32", 128, False, True, 2, 16, 2, 700),
    ("bf16", 256, True, False, 1, 16, 1, 1024),
    ("f32", 256, True, False, 1, 16, 1, 1024),
]


def split_of(case):
    f = sdp.attn_bwd_workspace_floats(case.B, case.Hq, case.Hkv, case.N, case.D)
    base = 2 * case.B * case.Hq * case.N
    return 1 if f == base else (f - base - 4) // (2 * case.B * case.Hkv * case.N * case.D)


@pytest.mark.parametrize("cfg", BWD_SPLIT, ids=lambda c: "%s-D%d-c%d-p%d-B%d-H%d-%d-N%d" % c)
def test_bwd_split_parts(cfg):
    dtype, D, causal, padded, B, Hq, Hkv, N = cfg
    case = inputs.make_case(B, Hq, Hkv, N, D, dtype, causal, padded, seed=[237, D, N, B])
    dout = inputs.make_grad(case, [237, D, N, B])
    S = split_of(case)
    assert S > 1, "shape %s does not split" % (cfg,)
    log("bwd split case %s (%d parts) valid_len %s" % (cfg, S, case.valid_len))
    compare_case(case, dout, "%s split %d" % (cfg, S), split_ws=True)


def test_bwd_split_deterministic_and_close_to_unsplit():
    """The split path is deterministic too, and agrees with the unsplit kernels to rounding."""
    case = inputs.make_case(1, 16, 1, 1500, 128, "bf16", True, False, seed=239)
    dout = inputs.make_grad(case, 239)
    assert split_of(case) > 1
    a = run_bwd(case, dout, split_ws=True)
    b = run_bwd(case, dout, split_ws=True)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    c = run_bwd(case, dout)
    for name, x, y in zip(("dQ", "dK", "dV"), a[:3], c[:3]):
        rel = np.abs(x - y).max() / max(np.abs(y).max(), GRAD_FLOOR["bf16"])
        log("split vs unsplit %s: %.2e" % (name, rel))
        assert rel <= BWD_TOL["bf16"]
    assert np.array_equal(a[0], c[0])   # dQ does not depend on the split


def test_bwd_split_masked_and_strided():
    """attn_bwd_ws with an explicit mask and [B, N, H, D] tensors, split 4."""
    import torch
    from gpu_util import device_mask, mask_values
    case = inputs.make_case(1, 8, 1, 1024, 64, "bf16", True, False, seed=241)
    assert split_of(case) > 1
    dout_bits = inputs.make_grad(case, 241)
    rng = np.random.default_rng(243)
    mv = mask_values("add", "alibi", "bf16", 1, 8, 1024, rng)
    dmask = device_mask("add", "alibi", "bf16", mv, 1024)
    q, k, v, do = (to_device(x, "bf16").transpose(1, 2).contiguous()
                   for x in (case.q_bits, case.k_bits, case.v_bits, dout_bits))
    out, lse = sdp.forward(q, k, v, causal=True, scale=case.scale, layout="bnhd",
                           attn_mask=dmask)
    dq, dk, dv = sdp.backward(q, k, v, out, do, lse, causal=True, scale=case.scale,
                              layout="bnhd", attn_mask=dmask)
    torch.cuda.synchronize()
    got = [from_device(t.transpose(1, 2), "bf16") for t in (dq, dk, dv)]
    qw, kw, vw = case.widened()
    ref = oracle.attn_bwd(qw, kw, vw, inputs.widen(dout_bits, "bf16"), case.scale, True, None,
                          add_mask=inputs.widen(mv, "bf16"))
    e = [check_grad(n, g, r, "bf16", "split masked bnhd") for n, g, r in
         zip(("dQ", "dK", "dV"), got, ref)]
    log("split masked bnhd: rel err dQ %.2e dK %.2e dV %.2e" % tuple(e))


@pytest.mark.parametrize("kind", ["keep", "add"])
def test_bwd_f32_split_masked(kind):
    """fp32 tensors, an explicit mask and the split dK/dV work (attn_bwd_ws, MQA)."""
    import torch
    from gpu_util import device_mask, mask_values
    case = inputs.make_case(1, 8, 1, 1024, 64, "f32", True, False, seed=245)
    assert split_of(case) > 1
    dout_bits = inputs.make_grad(case, 245)
    rng = np.random.default_rng(247)
    pattern = "random_bh" if kind == "keep" else "alibi"
    mv = mask_values(kind, pattern, "f32", 1, 8, 1024, rng)
    dmask = device_mask(kind, pattern, "f32", mv, 1024)
    q, k, v, do = (to_device(x, "f32") for x in (case.q_bits, case.k_bits, case.v_bits,
                                                  dout_bits))
    out, lse = sdp.forward(q, k, v, causal=True, scale=case.scale, attn_mask=dmask)
    dq, dk, dv = sdp.backward(q, k, v, out, do, lse, causal=True, scale=case.scale,
                              attn_mask=dmask)
    torch.cuda.synchronize()
    got = [from_device(t, "f32") for t in (dq, dk, dv)]
    qw, kw, vw = case.widened()
    mk = {"keep_mask": mv} if kind == "keep" else {"add_mask": inputs.widen(mv, "f32")}
    ref = oracle.attn_bwd(qw, kw, vw, inputs.widen(dout_bits, "f32"), case.scale, True, None,
                          **mk)
    e = [check_grad(n, g, r, "f32", "f32 split masked " + kind) for n, g, r in
         zip(("dQ", "dK", "dV"), got, ref)]
    log("f32 split masked %s: rel err dQ %.2e dK %.2e dV %.2e" % (kind, *e))


def pairs_key_tiles(case, split, mask="none"):
    """Whether the dK/dV kernel pairs key tiles i and nkt - 1 - i for this call: under causal
    masking, up to D = 128, when the pairs fill at least 15/16 of their last round of resident
    workgroups (256 CUs of a whole MI355X x 2 or 3 per CU by head dim and mask)."""
    nkt = -(-case.N // 128)
    items = case.B * case.Hkv * ((nkt + 1) // 2) * split
    per_cu = 3 if case.D <= 64 and mask == "none" else 2
    slots = 256 * per_cu
    rounds = -(-items // slots)
    return bool(case.causal) and case.D <= 128 and items * 16 >= rounds * slots * 15


# (dtype, D, padded, B, Hq, Hkv, N, split workspace): paired dK/dV items at small N: an even
# key-tile count (tiles 0 and 1), an odd one (0 with 2, 1 alone) with padding and a ragged last
# tile, pairs whose work is also split over two workgroups each, and the D = 64 kernel.
BWD_PAIRED = [
    ("bf16", 128, False, 8, 64, 64, 256, False),
    ("f16", 128, True, 4, 64, 64, 380, False),
    ("bf16", 128, False, 2, 128, 32, 1024, True),
    ("f16", 64, True, 8, 96, 96, 200, False),      # three workgroups per CU
]


@pytest.mark.parametrize("cfg", BWD_PAIRED, ids=lambda c: "%s-D%d-p%d-B%d-H%d-%d-N%d-ws%d" % c)
def test_bwd_paired_key_tiles(cfg):
    dtype, D, padded, B, Hq, Hkv, N, split_ws = cfg
    case = inputs.make_case(B, Hq, Hkv, N, D, dtype, True, padded, seed=[251, N, B])
    split = split_of(case) if split_ws else 1
    assert pairs_key_tiles(case, split), "shape %s does not pair its key tiles" % (cfg,)
    if split_ws:
        assert split > 1
    dout = inputs.make_grad(case, [251, N, B])
    log("bwd paired case %s (split %d) valid_len %s" % (cfg, split, case.valid_len))
    compare_case(case, dout, "%s paired" % (cfg,), split_ws=split_ws)


@pytest.mark.parametrize("kind", ["keep", "add"])
def test_bwd_paired_key_tiles_masked(kind):
    """Paired dK/dV items with an explicit mask (random per head: a keep mask, or additive values
    with -inf entries) on top of the causal mask."""
    import torch
    from gpu_util import device_mask, mask_values
    case = inputs.make_case(8, 64, 64, 256, 128, "bf16", True, False, seed=253)
    assert pairs_key_tiles(case, 1, kind)
    dout_bits = inputs.make_grad(case, 253)
    rng = np.random.default_rng(255)
    mv = mask_values(kind, "random_bh", "bf16", 8, 64, 256, rng)
    dmask = device_mask(kind, "random_bh", "bf16", mv, 256)
    q, k, v, do = (to_device(x, "bf16") for x in (case.q_bits, case.k_bits, case.v_bits,
                                                   dout_bits))
    out, lse = sdp.forward(q, k, v, causal=True, scale=case.scale, attn_mask=dmask)
    dq, dk, dv = sdp.backward(q, k, v, out, do, lse, causal=True, scale=case.scale,
                              attn_mask=dmask)
    torch.cuda.synchronize()
    got = [from_device(t, "bf16") for t in (dq, dk, dv)]
    qw, kw, vw = case.widened()
    mk = {"keep_mask": mv} if kind == "keep" else {"add_mask": inputs.widen(mv, "bf16")}
    ref = oracle.attn_bwd(qw, kw, vw, inputs.widen(dout_bits, "bf16"), case.scale, True, None,
                          **mk)
    e = [check_grad(n, g, r, "bf16", "paired %s mask" % kind) for n, g, r in
         zip(("dQ", "dK", "dV"), got, ref)]
    log("paired %s mask: rel err dQ %.2e dK %.2e dV %.2e" % (kind, *e))


def test_bwd_rising_row_maximum():
    """Keys scaled up along the sequence: rows whose maximum moves from tile to tile, so P
    rebuilt from the forward's LSE must still match."""
    case = inputs.make_case(1, 2, 2, 1024, 128, "f16", False, False, seed=209)
    k = inputs.widen(case.k_bits, "f16")
    k *= (1.0 + 12.0 * np.arange(case.N) / case.N)[None, None, :, None]
    case.k_bits = inputs.round_bits(k.astype(np.float32), "f16")
    dout = inputs.make_grad(case, 209)
    for causal in (False, True):
        case.causal = causal
        log("bwd rising maximum causal=%d" % causal)
        compare_case(case, dout, "bwd rising causal=%d" % causal)


@pytest.mark.parametrize("name", ["long_gqa", "causal_padded", "long_gqa_f32"])
def test_bwd_workload_slices(name):
    """Full-size workload in the benchmark's launch configuration; the oracle recomputes the
    gradients of eight (batch, KV head) groups, each with all its query heads."""
    w = inputs.WORKLOADS[name.replace("_f32", "")]
    if name.endswith("_f32"):
        case = inputs.make_case(w.B, w.Hq, w.Hkv, w.N, w.D, "f32", w.causal, w.padded,
                                seed=[20, w.c], scale=w.scale)
    else:
        case = inputs.make_workload(w)
    dout = inputs.make_grad(case, [w.c])
    log("bwd workload %s" % name)
    dq, dk, dv, delta, O, L = run_bwd(case, dout)
    for t in (dq, dk, dv, delta):
        assert np.isfinite(t).all()
    g = case.Hq // case.Hkv
    picks = sorted({(0, 0), (case.B - 1, case.Hkv - 1)} |
                   {(b % case.B, (3 * b + 1) % case.Hkv) for b in range(6)})[:8]
    qs = np.stack([case.q_bits[b, h * g:(h + 1) * g] for b, h in picks])
    ks = np.stack([case.k_bits[b, h:h + 1] for b, h in picks])
    vs = np.stack([case.v_bits[b, h:h + 1] for b, h in picks])
    ds = np.stack([dout[b, h * g:(h + 1) * g] for b, h in picks])
    vl = None if case.valid_len is None else np.array([case.valid_len[b] for b, _ in picks],
                                                      np.int32)
    wd = lambda x: inputs.widen(x, case.dtype)
    rq, rk, rv = oracle.attn_bwd(wd(qs), wd(ks), wd(vs), wd(ds), case.scale, case.causal, vl)
    for s, (b, h) in enumerate(picks):
        tag = "%s slice b=%d kv=%d" % (name, b, h)
        e = [check_grad("dQ", dq[b, h * g:(h + 1) * g], rq[s], case.dtype, tag),
             check_grad("dK", dk[b, h], rk[s, 0], case.dtype, tag),
             check_grad("dV", dv[b, h], rv[s, 0], case.dtype, tag)]
        log("%s: rel err dQ %.2e dK %.2e dV %.2e" % (tag, *e))


def test_autograd_function_matches_entry_point():
    """attention() (torch.autograd glue) returns exactly attn_bwd's gradients."""
    import torch
    case = inputs.make_case(2, 4, 2, 300, 128, "bf16", True, True, seed=211)
    dout = to_device(inputs.make_grad(case, 211), "bf16")
    q = to_device(case.q_bits, "bf16").requires_grad_()
    k = to_device(case.k_bits, "bf16").requires_grad_()
    v = to_device(case.v_bits, "bf16").requires_grad_()
    vl = torch.from_numpy(case.valid_len).cuda()
    out = sdp.attention(q, k, v, causal=True, valid_len=vl, scale=case.scale)
    out.backward(dout)
    o2, lse = sdp.forward(q.detach(), k.detach(), v.detach(), causal=True, valid_len=vl,
                          scale=case.scale)
    g = sdp.backward(q.detach(), k.detach(), v.detach(), o2, dout, lse, causal=True,
                     valid_len=vl, scale=case.scale)
    torch.cuda.synchronize()
    assert torch.equal(out, o2)
    for a, b in zip((q.grad, k.grad, v.grad), g):
        assert torch.equal(a, b)


def test_autograd_f32_matches_entry_point():
    """attention() on fp32 tensors returns exactly attn_bwd's fp32 gradients."""
    import torch
    case = inputs.make_case(2, 4, 2, 300, 64, "f32", True, True, seed=229)
    dout = to_device(inputs.make_grad(case, 229), "f32")
    base = [to_device(x, "f32") for x in (case.q_bits, case.k_bits, case.v_bits)]
    a = [t.clone().requires_grad_() for t in base]
    vl = torch.from_numpy(case.valid_len).cuda()
    out = sdp.attention(*a, causal=True, valid_len=vl, scale=case.scale)
    out.backward(dout)
    o2, lse = sdp.forward(*base, causal=True, valid_len=vl, scale=case.scale)
    g = sdp.backward(*base, o2, dout, lse, causal=True, valid_len=vl, scale=case.scale)
    torch.cuda.synchronize()
    assert out.dtype == torch.float32 and torch.equal(out, o2)
    for x, y in zip(a, g):
        assert y.dtype == torch.float32 and torch.equal(x.grad, y)


# ---- strided tensors (attn_bwd_strided): the same logical values in other layouts
BWD_STRIDED = [
    ("bnhd", "bf16", 128, True, True, 2, 8, 2, 300),
    ("bnhd", "f32", 128, True, False, 2, 4, 2, 200),
    ("bnhd", "bf16", 256, True, True, 2, 4, 2, 200),
    ("bnhd", "f32", 256, False, True, 2, 4, 2, 200),
    ("padded_rows", "f32", 64, False, True, 2, 4, 4, 130),
    ("bnhd", "f16", 64, False, False, 2, 4, 4, 200),
    ("padded_rows", "bf16", 64, True, False, 2, 6, 3, 257),
    ("packed_qkv", "f16", 128, True, True, 2, 4, 4, 190),
    ("transposed_dout", "bf16", 32, True, True, 3, 4, 2, 150),
]


@pytest.mark.parametrize("cfg", BWD_STRIDED, ids=lambda c: "%s-%s-D%d-c%d-p%d-B%d-H%d-%d-N%d" % c)
def test_bwd_strided_layouts(cfg):
    import torch
    mode, dtype, D, causal, padded, B, Hq, Hkv, N = cfg
    case = inputs.make_case(B, Hq, Hkv, N, D, dtype, causal, padded, seed=[213, D, N, B])
    dout_bits = inputs.make_grad(case, [213, D, N, B])
    log("bwd strided case %s valid_len %s" % (cfg, case.valid_len))
    q, k, v = (to_device(x, dtype) for x in (case.q_bits, case.k_bits, case.v_bits))
    do = to_device(dout_bits, dtype)
    vl = None
    if case.valid_len is not None:
        vl = torch.from_numpy(case.valid_len.astype(np.int32)).cuda()
    layout = "bhnd"
    if mode == "bnhd":
        q, k, v, do = (t.transpose(1, 2).contiguous() for t in (q, k, v, do))
        layout = "bnhd"
    elif mode == "padded_rows":
        def pad(t, extra):
            big = torch.full(t.shape[:3] + (t.shape[3] + extra,), float("nan"), dtype=t.dtype,
                             device=t.device)
            big[..., :t.shape[3]] = t
            return big[..., :t.shape[3]]
        q, k, v, do = pad(q, 8), pad(k, 24), pad(v, 16), pad(do, 8)
    elif mode == "packed_qkv":
        packed = torch.stack([t.transpose(1, 2) for t in (q, k, v)], dim=2).contiguous()
        q, k, v = (packed[:, :, i].transpose(1, 2) for i in range(3))
    elif mode == "transposed_dout":
        do = do.transpose(1, 2).contiguous().transpose(1, 2)   # [B, H, N, D] view of [B, N, H, D]
    out, lse = sdp.forward(q, k, v, causal=causal, valid_len=vl, scale=case.scale, layout=layout)
    dq, dk, dv = sdp.backward(q, k, v, out, do, lse, causal=causal, valid_len=vl,
                              scale=case.scale, layout=layout)
    torch.cuda.synchronize()
    if layout == "bnhd":
        dq, dk, dv = (t.transpose(1, 2) for t in (dq, dk, dv))
    got = [from_device(t, dtype) for t in (dq, dk, dv)]
    qw, kw, vw = case.widened()
    rq, rk, rv = oracle.attn_bwd(qw, kw, vw, inputs.widen(dout_bits, dtype), case.scale, causal,
                                 case.valid_len)
    e = [check_grad(n, g, r, dtype, str(cfg)) for n, g, r in zip(("dQ", "dK", "dV"), got,
                                                                   (rq, rk, rv))]
    log("%s: rel err dQ %.2e dK %.2e dV %.2e" % (cfg, *e))


def test_autograd_bnhd_matches_contiguous():
    """attention(layout="bnhd") on [B, N, H, D] tensors gives the gradients of the contiguous
    [B, H, N, D] call, transposed (same kernels, other strides: bitwise equal)."""
    import torch
    case = inputs.make_case(2, 4, 2, 300, 64, "f16", True, False, seed=215)
    dout = to_device(inputs.make_grad(case, 215), "f16")
    base = [to_device(x, "f16") for x in (case.q_bits, case.k_bits, case.v_bits)]
    a = [t.clone().requires_grad_() for t in base]
    b = [t.transpose(1, 2).contiguous().requires_grad_() for t in base]
    oa = sdp.attention(*a, causal=True, scale=case.scale)
    oa.backward(dout)
    ob = sdp.attention(*b, causal=True, scale=case.scale, layout="bnhd")
    ob.backward(dout.transpose(1, 2))
    torch.cuda.synchronize()
    assert torch.equal(oa, ob.transpose(1, 2))
    for x, y in zip(a, b):
        assert torch.equal(x.grad, y.grad.transpose(1, 2))


# ---- explicit masks (attn_bwd_masked): the forward's masks, the oracle's masked gradients
BWD_MASKED = [
    # (kind, pattern, dtype, D, causal, padded, B, Hq, Hkv, N)
    ("keep", "random_bh", "bf16", 128, True, True, 2, 4, 2, 300),
    ("keep", "window", "f16", 64, False, False, 2, 4, 4, 256),
    ("keep", "random_b", "f16", 128, False, True, 3, 2, 1, 333),
    ("keep", "empty_rows", "bf16", 64, True, False, 1, 4, 2, 130),
    ("add", "random_bh", "bf16", 128, True, False, 2, 4, 2, 257),
    ("add", "alibi", "bf16", 64, True, True, 2, 8, 2, 512),
    ("add", "random_b", "f16", 64, False, True, 2, 4, 1, 200),
    ("add", "window_neginf", "bf16", 128, False, False, 2, 4, 4, 300),
    ("keep", "random_bh", "f16", 32, True, False, 2, 4, 2, 200),
    ("add", "alibi", "bf16", 16, False, True, 2, 4, 1, 150),
    ("keep", "random_bh", "bf16", 256, True, True, 2, 4, 2, 200),
    ("add", "window_neginf", "f16", 256, False, False, 2, 2, 1, 150),
    # fp32 tensors: uint8 keep masks and fp32 additive masks
    ("keep", "random_bh", "f32", 128, True, True, 2, 4, 2, 300),
    ("keep", "empty_rows", "f32", 64, True, False, 1, 4, 2, 130),
    ("keep", "window", "f32", 32, False, False, 2, 4, 4, 256),
    ("add", "random_bh", "f32", 128, True, False, 2, 4, 2, 257),
    ("add", "alibi", "f32", 64, True, True, 2, 8, 2, 200),
    ("add", "window_neginf", "f32", 16, False, False, 2, 2, 1, 150),
    ("add", "large_negative", "f32", 128, False, True, 1, 2, 2, 100),
    ("keep", "random_bh", "f32", 256, True, True, 2, 4, 2, 200),
    ("add", "alibi", "f32", 256, False, False, 2, 4, 1, 150),
]


@pytest.mark.parametrize("cfg", BWD_MASKED,
                         ids=lambda c: "%s-%s-%s-D%d-c%d-p%d-B%d-H%d-%d-N%d" % c)
def test_bwd_explicit_masks(cfg):
    import torch
    from gpu_util import device_mask, mask_values
    kind, pattern, dtype, D, causal, padded, B, Hq, Hkv, N = cfg
    case = inputs.make_case(B, Hq, Hkv, N, D, dtype, causal, padded, seed=[217, D, N, B])
    dout_bits = inputs.make_grad(case, [217, D, N, B])
    rng = np.random.default_rng([219, D, N, B])
    mv = mask_values(kind, pattern, dtype, B, Hq, N, rng)
    log("bwd masked case %s valid_len %s mask %s" % (cfg, case.valid_len, mv.shape))
    dmask = device_mask(kind, pattern, dtype, mv, N)
    vl = None
    if case.valid_len is not None:
        vl = torch.from_numpy(case.valid_len.astype(np.int32)).cuda()
    q, k, v = (to_device(x, dtype) for x in (case.q_bits, case.k_bits, case.v_bits))
    do = to_device(dout_bits, dtype)
    out, lse = sdp.forward(q, k, v, causal=causal, valid_len=vl, scale=case.scale,
                           attn_mask=dmask)
    dq, dk, dv = sdp.backward(q, k, v, out, do, lse, causal=causal, valid_len=vl,
                              scale=case.scale, attn_mask=dmask)
    torch.cuda.synchronize()
    got = [from_device(t, dtype) for t in (dq, dk, dv)]
    qw, kw, vw = case.widened()
    mk = {"keep_mask": mv} if kind == "keep" else {"add_mask": inputs.widen(mv, dtype)}
    rq, rk, rv = oracle.attn_bwd(qw, kw, vw, inputs.widen(dout_bits, dtype), case.scale, causal,
                                 case.valid_len, **mk)
    e = [check_grad(n, g, r, dtype, str(cfg)) for n, g, r in zip(("dQ", "dK", "dV"), got,
                                                                   (rq, rk, rv))]
    log("%s: rel err dQ %.2e dK %.2e dV %.2e" % (cfg, *e))


def test_autograd_with_mask_matches_entry_point():
    """attention(attn_mask=...) returns exactly the masked entry points' output and gradients."""
    import torch
    from gpu_util import device_mask, mask_values
    case = inputs.make_case(2, 4, 2, 200, 64, "bf16", True, False, seed=221)
    rng = np.random.default_rng(223)
    mv = mask_values("add", "alibi", "bf16", 2, 4, 200, rng)
    dmask = device_mask("add", "alibi", "bf16", mv, 200)
    dout = to_device(inputs.make_grad(case, 221), "bf16")
    base = [to_device(x, "bf16") for x in (case.q_bits, case.k_bits, case.v_bits)]
    a = [t.clone().requires_grad_() for t in base]
    o = sdp.attention(*a, causal=True, scale=case.scale, attn_mask=dmask)
    o.backward(dout)
    o2, lse = sdp.forward(*base, causal=True, scale=case.scale, attn_mask=dmask)
    g = sdp.backward(*base, o2, dout, lse, causal=True, scale=case.scale, attn_mask=dmask)
    torch.cuda.synchronize()
    assert torch.equal(o, o2)
    for x, y in zip(a, g):
        assert torch.equal(x.grad, y)
