"""Compile the HIP library for gfx950, in-tree.

The library is three HIP translation units (attention; GEMM with a fused bias
+ GELU epilogue; row softmax and RMSNorm + SiLU) with the C ABI declared in
``include/fa.h``, ``include/gemm.h`` and ``include/rowwise.h``; it is built with hipcc for gfx950 only, with packed fp32
instructions disabled in device code.
"""

from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "fa_fwd.hip")
SRCS = [SRC, os.path.join(PKG, "csrc", "gemm_bias_gelu.hip"), os.path.join(PKG, "csrc", "rowwise.hip")]
LIB = os.path.join(PKG, "libfa_mi355x.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared",
    f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(extra=None, out=LIB) -> str:
    cmd = [hipcc(), *HIPCC_FLAGS, *(extra or []), *SRCS, "-o", out + ".tmp"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(sys.argv[1:]))
