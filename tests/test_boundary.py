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
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(attn_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    assert declared_functions() == ["attn_fwd", "attn_fwd_validate", "attn_status_string",
                                    "attn_version"]


def test_library_exports_every_declared_function(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", sdp.library_path()],
                         stdout=subprocess.PIPE, text=True, check=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name), name


def test_version(lib):
    assert sdp.attn_version() == 1


def test_status_strings(lib):
    codes = [sdp.ATTN_OK, sdp.ATTN_ERR_NULL, sdp.ATTN_ERR_SHAPE, sdp.ATTN_ERR_HEAD_DIM,
             sdp.ATTN_ERR_DTYPE, sdp.ATTN_ERR_SCALE, sdp.ATTN_ERR_LAUNCH, sdp.ATTN_ERR_ALIAS]
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
    (dict(D=256), sdp.ATTN_ERR_HEAD_DIM),
    (dict(D=32), sdp.ATTN_ERR_HEAD_DIM),
    (dict(dtype=2), sdp.ATTN_ERR_DTYPE),
    (dict(dtype=-1), sdp.ATTN_ERR_DTYPE),
    (dict(scale=float("nan")), sdp.ATTN_ERR_SCALE),
    (dict(scale=float("inf")), sdp.ATTN_ERR_SCALE),
    (dict(out=Q), sdp.ATTN_ERR_ALIAS),
    (dict(out=K + 1000), sdp.ATTN_ERR_ALIAS),
    (dict(lse=O + 64), sdp.ATTN_ERR_ALIAS),
    (dict(lse=V), sdp.ATTN_ERR_ALIAS),
    (dict(valid_len=O + 8), sdp.ATTN_ERR_ALIAS),
])
def test_validate_rejects(lib, kw, code):
    assert call(**kw) == code


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
