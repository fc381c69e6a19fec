"""Build libattn.so (HIP, gfx950) in-tree with hipcc.

Usage: python -m scaled_dot_product_fwd_amd.build
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRCS = [os.path.join(PKG, "csrc", name)
        for name in ("attn_fwd.hip", "attn_fwd_f32.hip", "attn_bwd.hip", "attn_bwd_f32.hip",
                     "attn_api.hip")]
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libattn.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed fp32 instructions are disabled on purpose: the kernels are written for plain fp32 VALU.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function"]


def _run(cmd):
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 target feature and says so; that is noise.
    lines = [ln for ln in proc.stdout.splitlines() if "packed-fp32-ops" not in ln]
    if lines:
        sys.stderr.write("\n".join(lines) + "\n")
    if proc.returncode != 0:
        raise RuntimeError("hipcc failed (%d): %s" % (proc.returncode, " ".join(cmd)))


def build(out: str = LIB, extra_flags=()) -> str:
    """Compile every source to an object (in parallel, one hipcc per file) and link them."""
    with tempfile.TemporaryDirectory(prefix="attn_build_") as d:
        objs = [os.path.join(d, os.path.splitext(os.path.basename(src))[0] + ".o")
                for src in SRCS]
        cmds = [[HIPCC, *FLAGS, *extra_flags, "-I", INCLUDE, "-c", src, "-o", obj]
                for src, obj in zip(SRCS, objs)]
        with concurrent.futures.ThreadPoolExecutor(max_workers=len(cmds)) as pool:
            for f in [pool.submit(_run, c) for c in cmds]:
                f.result()
        tmp = out + ".tmp%d" % os.getpid()
        _run([HIPCC, "--offload-arch=gfx950", "-fPIC", "-shared", *objs, "-o", tmp])
        os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
