"""Checks on the compiled gfx950 code of the forward kernels (CPU only: hipcc emits the assembly).

The forward issues its K/V/mask buffer loads into LDS through inline asm that sets M0 itself
(attn_common.h, dma16); that is only sound while no compiler-generated code in those kernels
uses M0, and the point of the asm form is that the compiler inserts no vmcnt wait before the
transposed V reads. Both are properties of the generated code, checked here.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.fixture(scope="module")
def fwd_asm(tmp_path_factory):
    if not (os.path.exists(HIPCC) or shutil.which(HIPCC)):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("isa") / "attn_fwd.s"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature",
           "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I",
           os.path.join(ROOT, "scaled_dot_product_fwd_amd", "csrc"), "--cuda-device-only", "-S",
           os.path.join(ROOT, "scaled_dot_product_fwd_amd", "csrc", "attn_fwd.hip"), "-o",
           str(out)]
    subprocess.run(cmd, check=True, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    return out.read_text().splitlines()


def kernels(lines):
    """(name, body lines) of every attn_fwd_kernel instantiation."""
    out = []
    for i, line in enumerate(lines):
        m = re.match(r"^(_Z\S*attn_fwd_kernel\S*):", line)
        if m:
            j = i
            while "s_endpgm" not in lines[j]:
                j += 1
            out.append((m.group(1), lines[i:j]))
    return out


def test_m0_only_set_for_lds_dma(fwd_asm):
    ks = kernels(fwd_asm)
    assert len(ks) >= 30   # 2 types x 5 head dims x causal or not x 3 mask kinds
    for name, body in ks:
        if "ELi256E" in name:
            continue   # D = 256 keeps the builtin, whose M0 the compiler manages itself
        for i, line in enumerate(body):
            t = line.strip()
            if t.startswith(";") or "m0" not in t:
                continue
            assert t.startswith("s_mov_b32 m0,"), (name, t)
            assert re.search(r"buffer_load_dword(x4)? .* lds", body[i + 1]), (name, t, body[i + 1])


def test_no_dma_wait_before_transposed_reads(fwd_asm):
    # kernels up to D = 128 (the asm form): no vmcnt wait directly before a ds_read_b64_tr_b16
    for name, body in kernels(fwd_asm):
        if "ELi256E" in name:
            continue
        for i, line in enumerate(body[:-1]):
            if "s_waitcnt vmcnt" in line:
                assert "ds_read_b64_tr_b16" not in body[i + 1], (name, line, body[i + 1])
