"""Build libattn.so (HIP, gfx950) in-tree with hipcc.

Usage: python -m scaled_dot_product_fwd_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRCS = [os.path.join(PKG, "csrc", name)
        for name in ("attn_fwd.hip", "attn_fwd_f32.hip", "attn_bwd.hip")]
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libattn.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed fp32 instructions are disabled on purpose: the kernels are written for plain fp32 VALU.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function"]


def build(out: str = LIB, extra_flags=()) -> str:
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, *extra_flags, "-I", INCLUDE, *SRCS, "-o", tmp]
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 target feature and says so; that is noise.
    lines = [ln for ln in proc.stdout.splitlines() if "packed-fp32-ops" not in ln]
    if proc.returncode != 0:
        sys.stderr.write("\n".join(lines) + "\n")
        raise RuntimeError("hipcc failed (%d): %s" % (proc.returncode, " ".join(cmd)))
    if lines:
        sys.stderr.write("\n".join(lines) + "\n")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
