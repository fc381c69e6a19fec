"""The C-ABI library on the host: it loads, exports every function include/attn.h declares,
and its host-side argument check returns the documented codes. No compute call is made."""
import os
import re
import subprocess

import pytest

import scaled_dot_product_fwd_amd as sdp
from scaled_dot_product_fwd_amd import build as sdp_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(sdp.library_path()):
        sdp_build.build()
    return sdp.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(attn_\w+)\s*\(", text,
                                 flags=re.M)))


def test_header_declares_the_entry_points():
    assert declared_functions() == ["attn_bwd", "attn_bwd_masked", "attn_bwd_masked_validate",
                                    "attn_bwd_scratch", "attn_bwd_strided",
                                    "attn_bwd_strided_validate",
                                    "attn_bwd_validate", "attn_bwd_workspace_floats",
                                    "attn_bwd_ws", "attn_bwd_ws_validate", "attn_fwd",
                                    "attn_fwd_masked", "attn_fwd_masked_validate",
                                    "attn_fwd_strided", "attn_fwd_strided_validate",
                                    "attn_fwd_validate", "attn_fwd_workspace_floats",
                                    "attn_fwd_ws", "attn_fwd_ws_validate", "attn_status_string",
                                    "attn_version"]


def test_library_exports_every_declared_function(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", sdp.library_path()],
                         stdout=subprocess.PIPE, text=True, check=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name), name


def test_version(lib):
    assert sdp.attn_version() == 14


def test_status_strings(lib):
    codes = [sdp.ATTN_OK, sdp.ATTN_ERR_NULL, sdp.ATTN_ERR_SHAPE, sdp.ATTN_ERR_HEAD_DIM,
             sdp.ATTN_ERR_DTYPE, sdp.ATTN_ERR_SCALE, sdp.ATTN_ERR_LAUNCH, sdp.ATTN_ERR_ALIAS,
             sdp.ATTN_ERR_LAYOUT, sdp.ATTN_ERR_MASK, sdp.ATTN_ERR_WORKSPACE,
             sdp.ATTN_ERR_SCRATCH]
    texts = [sdp.attn_status_string(c) for c in codes]
    assert len(set(texts)) == len(texts)
    assert sdp.attn_status_string(12345) == "unknown status"


# Fake, well-separated device addresses: attn_fwd_validate compares pointers, never reads them.
GB = 1 << 30
Q, K, V, O, L, VL = 1 * GB, 3 * GB, 5 * GB, 7 * GB, 9 * GB, 11 * GB


def call(**kw):
    a = dict(q=Q, k=K, v=V, out=O, lse=L, B=2, Hq=8, Hkv=2, N=1000, D=128, scale=0.088,
             causal=1, valid_len=VL, dtype=sdp.ATTN_BF16)
    a.update(kw)
    return sdp.attn_fwd_validate(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["Hq"],
                                 a["Hkv"], a["N"], a["D"], a["scale"], a["causal"],
                                 a["valid_len"], a["dtype"])


def test_validate_accepts_good_arguments(lib):
    assert call() == sdp.ATTN_OK
    assert call(lse=None, valid_len=None) == sdp.ATTN_OK
    assert call(D=64, dtype=sdp.ATTN_F16, causal=0) == sdp.ATTN_OK
    assert call(Hkv=1) == sdp.ATTN_OK
    assert call(N=1) == sdp.ATTN_OK
    assert call(scale=0.0) == sdp.ATTN_OK
    assert call(scale=-0.5) == sdp.ATTN_OK
    assert call(D=16) == sdp.ATTN_OK
    assert call(D=32, dtype=sdp.ATTN_F16) == sdp.ATTN_OK
    assert call(D=256) == sdp.ATTN_OK
    for d in (16, 32, 64, 128, 256):
        assert call(D=d, dtype=sdp.ATTN_F32) == sdp.ATTN_OK


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), sdp.ATTN_ERR_NULL),
    (dict(k=None), sdp.ATTN_ERR_NULL),
    (dict(v=None), sdp.ATTN_ERR_NULL),
    (dict(out=None), sdp.ATTN_ERR_NULL),
    (dict(B=0), sdp.ATTN_ERR_SHAPE),
    (dict(Hq=0), sdp.ATTN_ERR_SHAPE),
    (dict(Hkv=0), sdp.ATTN_ERR_SHAPE),
    (dict(N=0), sdp.ATTN_ERR_SHAPE),
    (dict(N=-3), sdp.ATTN_ERR_SHAPE),
    (dict(Hq=8, Hkv=3), sdp.ATTN_ERR_SHAPE),
    (dict(N=(1 << 22) + 1), sdp.ATTN_ERR_SHAPE),
    (dict(D=96), sdp.ATTN_ERR_HEAD_DIM),
    (dict(D=512), sdp.ATTN_ERR_HEAD_DIM),
    (dict(D=48), sdp.ATTN_ERR_HEAD_DIM),
    (dict(D=8), sdp.ATTN_ERR_HEAD_DIM),
    (dict(dtype=3), sdp.ATTN_ERR_DTYPE),
    (dict(dtype=sdp.ATTN_F32, D=48), sdp.ATTN_ERR_HEAD_DIM),
    (dict(dtype=-1), sdp.ATTN_ERR_DTYPE),
    (dict(scale=float("nan")), sdp.ATTN_ERR_SCALE),
    (dict(scale=float("inf")), sdp.ATTN_ERR_SCALE),
    (dict(out=Q), sdp.ATTN_ERR_ALIAS),
    (dict(out=K + 1024), sdp.ATTN_ERR_ALIAS),
    (dict(out=K + 1000), sdp.ATTN_ERR_LAYOUT),   # misaligned before overlapping
    (dict(q=Q + 8), sdp.ATTN_ERR_LAYOUT),
    (dict(v=V + 2), sdp.ATTN_ERR_LAYOUT),
    (dict(lse=O + 64), sdp.ATTN_ERR_ALIAS),
    (dict(lse=V), sdp.ATTN_ERR_ALIAS),
    (dict(valid_len=O + 8), sdp.ATTN_ERR_ALIAS),
])
def test_validate_rejects(lib, kw, code):
    assert call(**kw) == code


def test_validate_size_limits(lib):
    """The largest shapes: N = 2^22 fits while K/V heads stay within 2^31 bytes, and a launch
    holds at most 2^24 - 1 workgroups of 128 query rows."""
    one = dict(B=1, Hq=1, Hkv=1, N=1 << 22, valid_len=None)
    assert call(D=128, **one) == sdp.ATTN_OK
    assert call(D=64, dtype=sdp.ATTN_F32, **one) == sdp.ATTN_OK
    assert call(D=256, **one) == sdp.ATTN_ERR_SHAPE          # a K head of 2 GiB
    assert call(D=128, dtype=sdp.ATTN_F32, **one) == sdp.ATTN_ERR_SHAPE
    # Pointers 1 TiB apart so that no span overlaps: 2^24 - 1 tiles pass, 2^24 do not.
    T = 1 << 40
    far = dict(q=T, k=2 * T, v=3 * T, out=4 * T, lse=5 * T, valid_len=6 * T, Hq=1, Hkv=1,
               N=128, D=16)
    assert call(B=(1 << 24) - 1, **far) == sdp.ATTN_OK
    assert call(B=1 << 24, **far) == sdp.ATTN_ERR_SHAPE
    assert call(B=1 << 16, **dict(far, Hq=256, Hkv=256)) == sdp.ATTN_ERR_SHAPE
    assert call(B=1 << 10, **dict(far, Hq=128, Hkv=1, N=1 << 14)) == sdp.ATTN_ERR_SHAPE
    assert call(B=1 << 10, **dict(far, Hq=128, Hkv=1, N=(1 << 14) - 128)) == sdp.ATTN_OK


def test_validate_order_null_before_shape(lib):
    assert call(q=None, B=0) == sdp.ATTN_ERR_NULL


def test_forward_rejects_bad_tensors_before_any_call():
    torch = pytest.importorskip("torch")
    q = torch.zeros(1, 2, 8, 64, dtype=torch.float16)
    with pytest.raises(ValueError):
        sdp.forward(q, q, q, causal=True)            # host tensors
    with pytest.raises(ValueError):
        sdp.forward(q, q[:, :, :4], q, causal=True)  # shape mismatch
    with pytest.raises(ValueError):
        sdp.forward(q[0], q, q, causal=True)         # not 4-D


# ---- attn_fwd_strided_validate: layouts given by (batch, head, row) element strides
SB, SH, SN = 2, 8, 1000   # shapes of the strided checks (B, Hq, N); Hkv = 2, D = 128


def bhnd(H, N=SN, D=128):
    return (H * N * D, N * D, D)


def bnhd(H, N=SN, D=128):
    return (N * H * D, D, H * D)


def scall(**kw):
    a = dict(q=Q, qs=bhnd(8), k=K, ks=bhnd(2), v=V, vs=bhnd(2), out=O, os=bhnd(8), lse=L, B=SB,
             Hq=SH, Hkv=2, N=SN, D=128, scale=0.088, causal=1, valid_len=VL,
             dtype=sdp.ATTN_BF16)
    a.update(kw)
    return sdp.attn_fwd_strided_validate(a["q"], a["qs"], a["k"], a["ks"], a["v"], a["vs"],
                                         a["out"], a["os"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                                         a["N"], a["D"], a["scale"], a["causal"],
                                         a["valid_len"], a["dtype"])


def test_strided_validate_accepts(lib):
    assert scall() == sdp.ATTN_OK
    assert scall(qs=None, ks=None, vs=None, os=None) == sdp.ATTN_OK
    assert scall(qs=bnhd(8), ks=bnhd(2), vs=bnhd(2), os=bnhd(8)) == sdp.ATTN_OK
    # padded rows, K/V shared by every batch, Q/K/V as views of one packed [B, N, 3, H, D]
    assert scall(qs=(8 * SN * 136, SN * 136, 136)) == sdp.ATTN_OK
    assert scall(ks=(0, SN * 128, 128), vs=(0, SN * 128, 128)) == sdp.ATTN_OK
    packed = (SN * 3 * 8 * 128, 128, 3 * 8 * 128)
    assert scall(q=Q, k=Q + 8 * 256, v=Q + 16 * 256, qs=packed, ks=packed, vs=packed,
                 Hkv=8) == sdp.ATTN_OK
    # an output whose heads are outermost
    assert scall(os=(SN * 128, SB * SN * 128, 128)) == sdp.ATTN_OK


@pytest.mark.parametrize("kw,code", [
    (dict(qs=(-8, SN * 128, 128)), sdp.ATTN_ERR_LAYOUT),
    (dict(ks=(2 * SN * 128, SN * 128, 132)), sdp.ATTN_ERR_LAYOUT),   # row stride not 8k
    (dict(vs=(2 * SN * 128, 4, 128)), sdp.ATTN_ERR_LAYOUT),          # head stride not 8k
    (dict(qs=(8 * SN * 128, SN * 128, 120)), sdp.ATTN_ERR_LAYOUT),   # rows overlap
    (dict(os=(8 * SN * 128, SN * 128, 0)), sdp.ATTN_ERR_LAYOUT),     # output rows collide
    (dict(os=(8 * SN * 128, 128, 128)), sdp.ATTN_ERR_LAYOUT),        # output heads collide
    (dict(os=(0, SN * 128, 128)), sdp.ATTN_ERR_LAYOUT),              # output batches collide
    (dict(out=O + 4), sdp.ATTN_ERR_LAYOUT),
    (dict(ks=(0, 0, 1 << 20)), sdp.ATTN_ERR_SHAPE),                  # K head beyond 2^31 bytes
    (dict(out=Q + 64 * 1024), sdp.ATTN_ERR_ALIAS),
    (dict(out=K - 1024 * 1024), sdp.ATTN_ERR_ALIAS),                 # span reaches into K
    (dict(lse=V + 4096), sdp.ATTN_ERR_ALIAS),
    (dict(q=None), sdp.ATTN_ERR_NULL),
    (dict(D=96), sdp.ATTN_ERR_HEAD_DIM),
])
def test_strided_validate_rejects(lib, kw, code):
    assert scall(**kw) == code


def test_strided_validate_needs_three_strides(lib):
    with pytest.raises(ValueError):
        scall(qs=(1, 2))


# ---- attn_fwd_masked_validate: explicit [B, H, N, N] masks
MK = 13 * GB
MN = 1024   # N of the mask checks (a multiple of 16, so contiguous rows are aligned)


def mcall(**kw):
    a = dict(mask=MK, mtype=sdp.ATTN_MASK_KEEP_U8, ms=None, N=MN, B=SB, Hq=SH, Hkv=2)
    a.update(kw)
    N, B, Hq, Hkv = a["N"], a["B"], a["Hq"], a["Hkv"]
    return sdp.attn_fwd_masked_validate(Q, None, K, None, V, None, a.get("out", O), None,
                                        a.get("lse", L), B, Hq, Hkv, N, 128, 0.088, 1, VL,
                                        a["mask"], a["mtype"], a["ms"],
                                        a.get("dtype", sdp.ATTN_BF16))


def test_masked_validate_f32(lib):
    """fp32 inputs take uint8 keep masks and fp32 additive masks (4-byte elements: rows 16-byte
    aligned at 4 elements, twice the bytes of a 16-bit mask)."""
    f32, add = sdp.ATTN_F32, sdp.ATTN_MASK_ADD
    assert mcall(dtype=f32) == sdp.ATTN_OK
    assert mcall(dtype=f32, mtype=add) == sdp.ATTN_OK
    assert mcall(dtype=f32, mtype=add, ms=(SH * MN * MN, MN * MN, MN)) == sdp.ATTN_OK
    padded = dict(mtype=add, ms=(MN * (MN + 4), 0, MN + 4))
    assert mcall(**padded) == sdp.ATTN_ERR_LAYOUT                   # 2056-byte rows
    assert mcall(dtype=f32, **padded) == sdp.ATTN_OK                # 4112-byte rows
    far_rows = dict(mtype=add, ms=(0, 0, 1 << 19))
    assert mcall(**far_rows) == sdp.ATTN_OK
    assert mcall(dtype=f32, **far_rows) == sdp.ATTN_ERR_SHAPE      # rows past 2^31 bytes
    after16 = dict(mtype=add, out=MK + SB * MN * MN * 2)            # just past a 16-bit mask
    assert mcall(**after16) == sdp.ATTN_OK
    assert mcall(dtype=f32, **after16) == sdp.ATTN_ERR_ALIAS


def test_masked_validate_accepts(lib):
    assert mcall() == sdp.ATTN_OK                                   # [B, N, N] bytes
    assert mcall(mtype=sdp.ATTN_MASK_ADD) == sdp.ATTN_OK            # [B, N, N] 16-bit
    assert mcall(mtype=sdp.ATTN_MASK_NONE, mask=None) == sdp.ATTN_OK
    assert mcall(ms=(0, 0, MN)) == sdp.ATTN_OK                      # one [N, N] for all
    assert mcall(ms=(SH * MN * MN, MN * MN, MN)) == sdp.ATTN_OK     # per head
    assert mcall(N=1000, ms=(1000 * 1008, 0, 1008)) == sdp.ATTN_OK  # ragged N, padded rows
    assert mcall(N=1000, mtype=sdp.ATTN_MASK_ADD) == sdp.ATTN_OK    # 2000-byte rows


@pytest.mark.parametrize("kw,code", [
    (dict(mtype=3), sdp.ATTN_ERR_MASK),
    (dict(mtype=-1), sdp.ATTN_ERR_MASK),
    (dict(mask=None), sdp.ATTN_ERR_NULL),
    (dict(mask=MK + 8), sdp.ATTN_ERR_LAYOUT),
    (dict(N=1000), sdp.ATTN_ERR_LAYOUT),                        # 1000-byte rows unaligned
    (dict(N=1004, mtype=sdp.ATTN_MASK_ADD), sdp.ATTN_ERR_LAYOUT),
    (dict(ms=(MN * MN, 0, MN - 16)), sdp.ATTN_ERR_LAYOUT),      # row stride < N
    (dict(ms=(-MN * MN, 0, MN)), sdp.ATTN_ERR_LAYOUT),
    (dict(ms=(MN * MN, 8, MN)), sdp.ATTN_ERR_LAYOUT),           # head stride not 16 bytes
    (dict(ms=(0, 0, 1 << 22)), sdp.ATTN_ERR_SHAPE),             # rows beyond 2^31 bytes
    (dict(out=MK + 4096), sdp.ATTN_ERR_ALIAS),
    (dict(lse=MK + 65536), sdp.ATTN_ERR_ALIAS),
])
def test_masked_validate_rejects(lib, kw, code):
    assert mcall(**kw) == code


# ---- attn_bwd_validate
DO, DQ, DK, DV, DL = 15 * GB, 17 * GB, 19 * GB, 21 * GB, 23 * GB


def bcall(**kw):
    a = dict(q=Q, k=K, v=V, out=O, dout=DO, lse=L, dq=DQ, dk=DK, dv=DV, ws=DL, B=2, Hq=8,
             Hkv=2, N=1000, D=128, scale=0.088, causal=1, valid_len=VL, dtype=sdp.ATTN_BF16)
    a.update(kw)
    return sdp.attn_bwd_validate(a["q"], a["k"], a["v"], a["out"], a["dout"], a["lse"], a["dq"],
                                 a["dk"], a["dv"], a["ws"], a["B"], a["Hq"], a["Hkv"],
                                 a["N"], a["D"], a["scale"], a["causal"], a["valid_len"],
                                 a["dtype"])


def test_bwd_validate_accepts(lib):
    assert bcall() == sdp.ATTN_OK
    assert bcall(valid_len=None, D=64, dtype=sdp.ATTN_F16, causal=0, Hkv=8) == sdp.ATTN_OK
    assert bcall(D=16) == sdp.ATTN_OK
    assert bcall(D=32) == sdp.ATTN_OK
    assert bcall(D=256) == sdp.ATTN_OK
    assert bcall(D=256, dtype=sdp.ATTN_F16) == sdp.ATTN_OK
    assert bcall(D=256, dtype=sdp.ATTN_F32) == sdp.ATTN_OK
    for d in (16, 32, 64, 128):
        assert bcall(D=d, dtype=sdp.ATTN_F32) == sdp.ATTN_OK


def test_bwd_validate_size_limits(lib):
    """As in the forward: at most 2^24 - 1 tiles of 128 rows per launch (pointers 1 TiB apart,
    so that no span overlaps)."""
    T = 1 << 40
    far = dict(q=T, k=2 * T, v=3 * T, out=4 * T, dout=5 * T, lse=6 * T, dq=7 * T, dk=8 * T,
               dv=9 * T, ws=10 * T, valid_len=11 * T, Hq=1, Hkv=1, N=128, D=16)
    assert bcall(B=(1 << 24) - 1, **far) == sdp.ATTN_OK
    assert bcall(B=1 << 24, **far) == sdp.ATTN_ERR_SHAPE
    one = dict(B=1, Hq=1, Hkv=1, N=1 << 22, valid_len=None)
    assert bcall(D=128, **one) == sdp.ATTN_OK
    assert bcall(D=128, **dict(one, N=(1 << 22) + 1)) == sdp.ATTN_ERR_SHAPE


@pytest.mark.parametrize("kw,code", [
    (dict(lse=None), sdp.ATTN_ERR_NULL),
    (dict(ws=None), sdp.ATTN_ERR_NULL),
    (dict(dout=None), sdp.ATTN_ERR_NULL),
    (dict(Hq=8, Hkv=3), sdp.ATTN_ERR_SHAPE),
    (dict(D=512), sdp.ATTN_ERR_HEAD_DIM),
    (dict(D=48), sdp.ATTN_ERR_HEAD_DIM),
    (dict(dtype=7), sdp.ATTN_ERR_DTYPE),
    (dict(scale=float("nan")), sdp.ATTN_ERR_SCALE),
    # dq right after a 16-bit-sized q overlaps q once elements are 4 bytes
    (dict(dq=Q + 2 * 8 * 1000 * 128 * 2, dtype=sdp.ATTN_F32), sdp.ATTN_ERR_ALIAS),
    (dict(dq=DQ + 8), sdp.ATTN_ERR_LAYOUT),
    (dict(ws=DL + 2), sdp.ATTN_ERR_LAYOUT),
    (dict(dq=Q + 1024), sdp.ATTN_ERR_ALIAS),            # dq overlaps q
    (dict(dk=DQ + 4096), sdp.ATTN_ERR_ALIAS),           # dk overlaps dq
    (dict(dv=DO), sdp.ATTN_ERR_ALIAS),                  # dv overlaps dout
    (dict(ws=L + 64), sdp.ATTN_ERR_ALIAS),              # workspace overlaps lse
    (dict(ws=VL - 64), sdp.ATTN_ERR_ALIAS),             # workspace overlaps valid_len
    (dict(ws=L - 2 * 2 * 8 * 1000 * 4 + 4), sdp.ATTN_ERR_ALIAS),   # its second row overlaps lse
])
def test_bwd_validate_rejects(lib, kw, code):
    assert bcall(**kw) == code


def test_f32_layouts(lib):
    """fp32 rows: strides in multiples of 4 elements (16 bytes), spans of 4-byte elements."""
    f32 = sdp.ATTN_F32
    assert scall(dtype=f32, qs=(8 * SN * 132, SN * 132, 132)) == sdp.ATTN_OK
    assert scall(dtype=f32, qs=(8 * SN * 130, SN * 130, 130)) == sdp.ATTN_ERR_LAYOUT
    # a 16-bit stride of 136 elements is fine, 132 is not a multiple of 8
    assert scall(qs=(8 * SN * 132, SN * 132, 132)) == sdp.ATTN_ERR_LAYOUT
    # out placed right after a 16-bit-sized q overlaps q once elements are 4 bytes
    qbytes16 = 2 * 8 * 1000 * 128 * 2
    assert call(out=Q + qbytes16) == sdp.ATTN_OK
    assert call(out=Q + qbytes16, dtype=f32) == sdp.ATTN_ERR_ALIAS
    # the forward takes explicit masks with fp32 inputs too
    assert sdp.attn_fwd_masked_validate(Q, None, K, None, V, None, O, None, L, SB, SH, 2, MN, 128,
                                        0.088, 1, VL, MK, sdp.ATTN_MASK_KEEP_U8, None,
                                        f32) == sdp.ATTN_OK


# ---- attn_bwd_strided_validate
def bscall(**kw):
    a = dict(q=Q, qs=None, k=K, ks=None, v=V, vs=None, out=O, os=None, dout=DO, gs=None, lse=L,
             dq=DQ, dqs=None, dk=DK, dks=None, dv=DV, dvs=None, ws=DL, B=2, Hq=8, Hkv=2, N=1000,
             D=128, scale=0.088, causal=1, valid_len=VL, dtype=sdp.ATTN_BF16)
    a.update(kw)
    return sdp.attn_bwd_strided_validate(
        a["q"], a["qs"], a["k"], a["ks"], a["v"], a["vs"], a["out"], a["os"], a["dout"], a["gs"],
        a["lse"], a["dq"], a["dqs"], a["dk"], a["dks"], a["dv"], a["dvs"], a["ws"], a["B"],
        a["Hq"], a["Hkv"], a["N"], a["D"], a["scale"], a["causal"], a["valid_len"], a["dtype"])


def test_bwd_strided_validate(lib):
    def bnhd_(H, N=1000, D=128):
        return (N * H * D, D, H * D)
    assert bscall() == sdp.ATTN_OK
    # every tensor [B, N, H, D]
    assert bscall(qs=bnhd_(8), ks=bnhd_(2), vs=bnhd_(2), os=bnhd_(8), gs=bnhd_(8),
                  dqs=bnhd_(8), dks=bnhd_(2), dvs=bnhd_(2)) == sdp.ATTN_OK
    # padded input rows; a transposed dO
    assert bscall(qs=(8 * 1000 * 136, 1000 * 136, 136), gs=bnhd_(8)) == sdp.ATTN_OK
    # a row stride that is not a multiple of 8 elements, a negative stride
    assert bscall(ks=(2 * 1000 * 132, 1000 * 132, 132)) == sdp.ATTN_ERR_LAYOUT
    assert bscall(vs=(-1000 * 128 * 2, 1000 * 128, 128)) == sdp.ATTN_ERR_LAYOUT
    # gradient rows that collide (head stride 0), rows closer than D
    assert bscall(dqs=(1000 * 128, 0, 128)) == sdp.ATTN_ERR_LAYOUT
    assert bscall(dks=(2 * 1000 * 64, 1000 * 64, 64)) == sdp.ATTN_ERR_LAYOUT
    # a strided dk whose span reaches into v
    assert bscall(dk=V - 1024, dks=bnhd_(2)) == sdp.ATTN_ERR_ALIAS
    # K and V shared by the batches (zero batch stride) are fine as inputs
    assert bscall(ks=(0, 1000 * 128, 128), vs=(0, 1000 * 128, 128)) == sdp.ATTN_OK
    # a row stride so large that a head no longer fits 32-bit buffer offsets
    assert bscall(ks=(0, 0, 1 << 20)) == sdp.ATTN_ERR_SHAPE


def test_no_fallback_path():
    """The product path fails loudly: a missing library is an ImportError, CPU tensors are
    rejected, and no module of the package refers to the oracle."""
    with pytest.raises(ImportError):
        sdp.load_library(os.path.join(os.path.dirname(sdp.library_path()), "missing_libattn.so"))
    import torch
    x = torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        sdp.forward(x, x, x, causal=True)
    pkg = os.path.dirname(sdp.__file__)
    pattern = re.compile(r"^\s*(import\s+oracle|from\s+oracle\b)|liboracle|attn_oracle", re.M)
    for root, _, files in os.walk(pkg):
        for name in files:
            if name.endswith((".py", ".hip", ".h")):
                text = open(os.path.join(root, name)).read()
                assert not pattern.search(text), "%s uses the oracle" % name


# ---- attn_bwd_masked_validate
def bmcall(**kw):
    a = dict(mask=MK, mtype=sdp.ATTN_MASK_KEEP_U8, ms=None, N=MN, dq=DQ, ws=DL,
             dtype=sdp.ATTN_BF16)
    a.update(kw)
    N = a["N"]
    return sdp.attn_bwd_masked_validate(Q, None, K, None, V, None, O, None, DO, None, L, a["dq"],
                                        None, DK, None, DV, None, a["ws"], SB, SH, 2, N, 128,
                                        0.088, 1, VL, a["mask"], a["mtype"], a["ms"],
                                        a["dtype"])


def test_bwd_masked_validate(lib):
    assert bmcall() == sdp.ATTN_OK
    assert bmcall(mtype=sdp.ATTN_MASK_ADD) == sdp.ATTN_OK
    assert bmcall(mtype=sdp.ATTN_MASK_NONE, mask=None) == sdp.ATTN_OK
    assert bmcall(ms=(0, MN * MN, MN)) == sdp.ATTN_OK                 # [Hq, N, N] per head
    assert bmcall(mtype=5) == sdp.ATTN_ERR_MASK
    assert bmcall(dtype=sdp.ATTN_F32) == sdp.ATTN_OK                    # fp32 with a keep mask
    add = sdp.ATTN_MASK_ADD
    assert bmcall(dtype=sdp.ATTN_F32, mtype=add) == sdp.ATTN_OK         # and an fp32 additive one
    assert bmcall(mtype=add, ms=(0, 0, 1 << 19)) == sdp.ATTN_OK
    assert bmcall(dtype=sdp.ATTN_F32, mtype=add, ms=(0, 0, 1 << 19)) == sdp.ATTN_ERR_SHAPE
    assert bmcall(dtype=sdp.ATTN_F32, mtype=add, ms=(MN * (MN + 4), 0, MN + 4)) == sdp.ATTN_OK
    assert bmcall(mtype=add, ms=(MN * (MN + 4), 0, MN + 4)) == sdp.ATTN_ERR_LAYOUT
    assert bmcall(mtype=sdp.ATTN_MASK_NONE, mask=None, dtype=sdp.ATTN_F32) == sdp.ATTN_OK
    assert bmcall(mask=None) == sdp.ATTN_ERR_NULL
    assert bmcall(mask=MK + 8) == sdp.ATTN_ERR_LAYOUT                 # misaligned
    assert bmcall(ms=(MN * MN, 0, MN - 16)) == sdp.ATTN_ERR_LAYOUT      # rows closer than N
    assert bmcall(ms=(0, 0, 1 << 21)) == sdp.ATTN_ERR_SHAPE             # rows past 32-bit reach
    assert bmcall(dq=MK + 1024) == sdp.ATTN_ERR_ALIAS                   # dq overlaps the mask
    assert bmcall(ws=MK - 1024) == sdp.ATTN_ERR_ALIAS                   # workspace overlaps it


# ---- attn_bwd_ws_validate and attn_bwd_workspace_floats
def wcall(**kw):
    a = dict(ws=DL, n=None, B=2, Hq=8, Hkv=2, N=1000, D=128, dq=DQ, dtype=sdp.ATTN_BF16,
             mask=None, mtype=sdp.ATTN_MASK_NONE)
    a.update(kw)
    n = a["n"] if a["n"] is not None else 2 * a["B"] * a["Hq"] * a["N"]
    return sdp.attn_bwd_ws_validate(Q, None, K, None, V, None, O, None, DO, None, L, a["dq"], None,
                                    DK, None, DV, None, a["ws"], n, a["B"], a["Hq"], a["Hkv"],
                                    a["N"], a["D"], 0.088, 1, VL, a["mask"], a["mtype"], None,
                                    a["dtype"])


def test_bwd_workspace_floats(lib):
    # enough key tiles: no split, the minimal workspace
    assert sdp.attn_bwd_workspace_floats(8, 32, 8, 4096, 128) == 2 * 8 * 32 * 4096
    # MQA with a long group: 128 key tiles split 8 ways
    assert sdp.attn_bwd_workspace_floats(1, 32, 1, 16384, 128) == (
        2 * 32 * 16384 + 4 + 2 * 8 * 16384 * 128)
    # short groups do not pay for partial sums
    assert sdp.attn_bwd_workspace_floats(2, 8, 8, 1024, 64) == 2 * 2 * 8 * 1024
    assert sdp.attn_bwd_workspace_floats(0, 8, 8, 1024, 64) == -1


def test_bwd_ws_validate(lib):
    base = 2 * 2 * 8 * 1000
    big = sdp.attn_bwd_workspace_floats(2, 8, 2, 1000, 128)
    assert big > base
    assert wcall() == sdp.ATTN_OK
    assert wcall(n=big) == sdp.ATTN_OK
    assert wcall(n=base - 1) == sdp.ATTN_ERR_WORKSPACE
    assert wcall(n=0) == sdp.ATTN_ERR_WORKSPACE
    assert wcall(dtype=sdp.ATTN_F32, n=big) == sdp.ATTN_OK
    f32keep = dict(dtype=sdp.ATTN_F32, mask=MK, mtype=sdp.ATTN_MASK_KEEP_U8)
    assert wcall(N=1024, **f32keep) == sdp.ATTN_OK
    assert wcall(**f32keep) == sdp.ATTN_ERR_LAYOUT          # 1000-byte mask rows
    assert wcall(mask=MK, mtype=sdp.ATTN_MASK_KEEP_U8, N=MN) == sdp.ATTN_OK
    assert wcall(mtype=7, mask=MK) == sdp.ATTN_ERR_MASK
    # dq right after the minimal workspace: fine when only that is used, an overlap with the
    # partial sums once the workspace is large enough to split
    after = DL + 4 * base
    assert wcall(dq=after) == sdp.ATTN_OK
    assert wcall(dq=after, n=big) == sdp.ATTN_ERR_ALIAS
    # exactly the split's size uses the partial sums; one float less drops the split
    assert wcall(dq=after, n=base + 4 + 2 * 2 * 2 * 2 * 1000 * 128) == sdp.ATTN_ERR_ALIAS
    assert wcall(dq=after, n=base + 4 + 2 * 2 * 2 * 2 * 1000 * 128 - 1) == sdp.ATTN_OK


# ---- the status strings describe what the entry points accept

def test_status_strings_match_what_the_library_accepts(lib):
    # The head-dimension string lists exactly the D the forward and the backward accept.
    txt = sdp.attn_status_string(sdp.ATTN_ERR_HEAD_DIM)
    listed = sorted(int(x) for x in re.findall(r"\b\d+\b", txt))
    fwd_ok = [D for D in range(1, 513) if call(D=D) != sdp.ATTN_ERR_HEAD_DIM]
    bwd_ok = [D for D in range(1, 513) if bcall(D=D) != sdp.ATTN_ERR_HEAD_DIM]
    assert listed == fwd_ok == bwd_ok, (txt, fwd_ok, bwd_ok)
    assert "backward" not in txt
    # The dtype string names every dtype the entry points take, and no restriction remains:
    # each dtype is accepted with an explicit keep or additive mask, forward and backward.
    txt = sdp.attn_status_string(sdp.ATTN_ERR_DTYPE)
    for name in ("ATTN_F16", "ATTN_BF16", "ATTN_F32"):
        assert name in txt
    assert "only" not in txt
    M = 13 * GB
    for dt in (sdp.ATTN_F16, sdp.ATTN_BF16, sdp.ATTN_F32):
        for mt in (sdp.ATTN_MASK_KEEP_U8, sdp.ATTN_MASK_ADD):
            st = sdp.attn_fwd_masked_validate(Q, None, K, None, V, None, O, None, L, 2, 8, 2,
                                              1000, 128, 0.088, 1, VL, M, mt, [0, 0, 1008], dt)
            assert st == sdp.ATTN_OK, (dt, mt, st)
            st = sdp.attn_bwd_masked_validate(Q, None, K, None, V, None, O, None, 15 * GB, None,
                                              L, 17 * GB, None, 19 * GB, None, 21 * GB, None,
                                              23 * GB, 2, 8, 2, 1000, 128, 0.088, 1, VL, M, mt,
                                              [0, 0, 1008], dt)
            assert st == sdp.ATTN_OK, (dt, mt, st)
    assert call(dtype=3) == sdp.ATTN_ERR_DTYPE


# ---- attn_fwd_ws: the split of the key range for small grids (host-side choice and checks)
WS = 13 * GB


def split_rule(B, Hq, N, D, causal, ws_floats=None):
    """The chunking the header describes, restated: where the (batch, head, 128-row query tile)
    items fill at most a quarter of the device (128 workgroups up to D = 128, 64 at D = 256) and
    the longest key range has at least 48 tiles of 64 keys, the smallest number of key tiles per
    chunk for which every chunk runs at once (512 workgroups up to D = 128, 256 at D = 256)."""
    nqt, nkt = -(-N // 128), -(-N // 64)
    slots = 256 if D > 128 else 512
    if B * Hq * nqt > slots // 4:
        return 0
    tiles = [min(2 * (qt + 1), nkt) if causal else nkt for qt in range(nqt)]
    if max(tiles) < 48:
        return 0
    for ct in range(1, max(tiles)):
        if B * Hq * sum(-(-t // ct) for t in tiles) <= slots:
            size = B * Hq * nqt * -(-max(tiles) // ct) * 128 * (D + 1) + 4
            if ws_floats is None or size <= ws_floats:
                return size
    return 0


@pytest.mark.parametrize("shape", [
    (1, 2, 8192, 64, True),     # 128 query tiles over up to 128 key tiles: chunks of 19
    (1, 1, 3072, 128, True),    # chunks of 2 key tiles
    (1, 1, 3200, 64, False),    # chunks of 3
    (1, 1, 6000, 256, True),    # D = 256: at most 64 query tiles
    (1, 2, 6000, 256, True),    # ... 94 are too many
    (2, 8, 1024, 64, True),     # the causal_mha workload: too few key tiles per row
    (8, 32, 4096, 128, True),   # the long_gqa workload fills the device
    (4, 32, 2048, 128, True),   # causal_gqa too
    (1, 8, 4096, 128, False),   # 256 query tiles: more than a quarter of the device
])
def test_fwd_workspace_floats(lib, shape):
    B, Hq, N, D, causal = shape
    got = sdp.attn_fwd_workspace_floats(B, Hq, 1, N, D, causal)
    assert got == split_rule(B, Hq, N, D, causal)
    if shape == (1, 2, 8192, 64, True):
        assert got == 128 * 7 * 128 * 65 + 4
    if shape == (1, 1, 3072, 128, True):
        assert got == 24 * 24 * 128 * 129 + 4
    if shape in ((2, 8, 1024, 64, True), (8, 32, 4096, 128, True), (4, 32, 2048, 128, True),
                 (1, 8, 4096, 128, False), (1, 2, 6000, 256, True)):
        assert got == 0


def test_fwd_workspace_floats_rejects_bad_sizes(lib):
    assert sdp.attn_fwd_workspace_floats(0, 8, 8, 1024, 64, True) == -1
    assert sdp.attn_fwd_workspace_floats(2, 8, 8, 0, 64, True) == -1


def wcall_fwd(**kw):
    a = dict(q=Q, k=K, v=V, out=O, lse=L, ws=WS, n=10 ** 8, B=1, Hq=2, Hkv=2, N=8192, D=64,
             causal=1, valid_len=VL, dtype=sdp.ATTN_F16)
    a.update(kw)
    return sdp.attn_fwd_ws_validate(a["q"], None, a["k"], None, a["v"], None, a["out"], None,
                                    a["lse"], a["ws"], a["n"], a["B"], a["Hq"], a["Hkv"], a["N"],
                                    a["D"], 0.125, a["causal"], a["valid_len"], a["dtype"])


def test_fwd_ws_validate(lib):
    full = sdp.attn_fwd_workspace_floats(1, 2, 2, 8192, 64, True)
    assert wcall_fwd() == sdp.ATTN_OK
    assert wcall_fwd(ws=None) == sdp.ATTN_OK              # no workspace: no split
    assert wcall_fwd(n=0) == sdp.ATTN_OK                  # too small for any split
    assert wcall_fwd(n=-1) == sdp.ATTN_ERR_WORKSPACE
    assert wcall_fwd(ws=WS + 4) == sdp.ATTN_ERR_LAYOUT    # float4 partials: 16-byte alignment
    # the used part of the workspace overlaps an input or output
    assert wcall_fwd(ws=Q - 4 * full + 64) == sdp.ATTN_ERR_ALIAS
    assert wcall_fwd(ws=O + 1024) == sdp.ATTN_ERR_ALIAS
    assert wcall_fwd(ws=L - 16) == sdp.ATTN_ERR_ALIAS
    assert wcall_fwd(ws=Q - 4 * full) == sdp.ATTN_OK      # just below Q
    # a smaller workspace uses a coarser split, so only that part must be clear of Q
    half = split_rule(1, 2, 8192, 64, True, full // 2)
    assert 0 < half < full
    assert wcall_fwd(ws=Q - 4 * half, n=full // 2) == sdp.ATTN_OK
    assert wcall_fwd(ws=Q - 4 * half + 16, n=full // 2) == sdp.ATTN_ERR_ALIAS
    # fp32 never splits: the workspace is not checked
    assert wcall_fwd(dtype=sdp.ATTN_F32, ws=O + 1024) == sdp.ATTN_OK
    # the attn_fwd_strided checks come first
    assert wcall_fwd(D=96) == sdp.ATTN_ERR_HEAD_DIM
    assert wcall_fwd(q=None) == sdp.ATTN_ERR_NULL
