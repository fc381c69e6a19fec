"""Checks on the compiled gfx950 code of the forward kernels (CPU only: hipcc emits the assembly).

The forward issues its K/V/mask buffer loads into LDS through inline asm (attn_common.h,
dma16_at): the compiler sets M0 for it (an operand constraint) but cannot see the load itself,
so the asm carries the wait states the hardware needs after a scalar write of M0 or a VALU write
of an SGPR the load reads; and the point of the asm form is that the compiler inserts no vmcnt
wait before the transposed V reads. Both are properties of the generated code, checked here,
as is the fp16 row sum's use of every weight register (a compiler pitfall seen once).
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


def test_lds_dma_carries_its_wait_states(fwd_asm):
    ks = kernels(fwd_asm)
    assert len(ks) >= 30   # 2 types x 5 head dims x causal or not x 3 mask kinds
    seen = 0
    for name, body in ks:
        if "ELi256E" in name:
            continue   # D = 256 keeps the builtin, whose wait states the compiler inserts
        for i, line in enumerate(body):
            if re.search(r"buffer_load_dword(x4)? .* lds", line):
                prev = [t.strip() for t in body[max(0, i - 3):i]
                        if t.strip() and not t.strip().startswith(";")]
                assert prev and prev[-1] == "s_nop 4", (name, body[max(0, i - 3):i + 1])
                seen += 1
    assert seen > 0


def test_m0_written_only_by_scalar_moves(fwd_asm):
    # M0 is the LDS destination of the DMA; nothing else in these kernels may rely on it, and
    # only scalar moves / adds / ors (the compiler's materialisation of the asm operand) write it.
    for name, body in kernels(fwd_asm):
        if "ELi256E" in name:
            continue
        for line in body:
            t = line.strip()
            if t.startswith(";") or not re.search(r"\bm0\b", t):
                continue
            assert re.match(r"s_(mov|add|or)_[bi]32 m0, ", t), (name, t)


def test_no_dma_wait_before_transposed_reads(fwd_asm):
    # kernels up to D = 128 (the asm form): no vmcnt wait directly before a ds_read_b64_tr_b16
    for name, body in kernels(fwd_asm):
        if "ELi256E" in name:
            continue
        for i, line in enumerate(body[:-1]):
            if "s_waitcnt vmcnt" in line:
                assert "ds_read_b64_tr_b16" not in body[i + 1], (name, line, body[i + 1])


def test_fp16_row_sum_reads_every_weight(fwd_asm):
    # fp16 kernels sum the rounded weights of a tile with v_dot2 (two per instruction): no dot2
    # may read the same register as the previous dot2 into its accumulator unless something
    # wrote that register in between (a bit cast of a vector element once compiled to a read
    # of element 0 for all four words of a weight fragment)
    seen = 0
    for name, body in kernels(fwd_asm):
        if "attn_fwd_kernelILi0E" not in name:   # ATTN_F16 = 0
            continue
        last = {}   # accumulator -> (source register, line index) within one basic block
        for i, line in enumerate(body):
            if re.match(r"^\.LBB|\s*s_(c?branch|setpc)", line):
                last = {}
                continue
            m = re.match(r"\s*v_dot2c?_f32_f16\S*\s+(v\d+),\s*\S+,\s*(v\d+)", line)
            if not m:
                continue
            acc, src = m.groups()
            seen += 1
            if acc in last and last[acc][0] == src:
                between = body[last[acc][1] + 1:i]
                wrote = any(re.match(r"\s*[vsd]\S*\s+%s\b" % src, t) or
                            re.match(r"\s*[vsd]\S*\s+v\[(\d+):(\d+)\]", t) and
                            int(re.match(r"\s*[vsd]\S*\s+v\[(\d+):(\d+)\]", t).group(1)) <=
                            int(src[1:]) <=
                            int(re.match(r"\s*[vsd]\S*\s+v\[(\d+):(\d+)\]", t).group(2))
                            for t in between)
                assert wrote, (name, line.strip())
            last[acc] = (src, i)
    assert seen > 0
