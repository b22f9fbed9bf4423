"""Compile the HIP library for gfx950, in-tree.

The library is three HIP translation units (attention; GEMM with a fused bias
+ GELU epilogue; row softmax and RMSNorm + SiLU) with the C ABI declared in
``include/fa.h``, ``include/gemm.h`` and ``include/rowwise.h``; it is built with hipcc for gfx950 only, with packed fp32
instructions disabled in device code.  Each unit is compiled to its own object (in parallel, with its own device
options) and the objects are linked into one shared library.
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


# Device options of one translation unit.  The attention kernels keep every
# matrix-instruction accumulator in VGPRs: the instances with two key groups
# miss the two-waves-per-SIMD register budget, and the compiler would then
# give their products AGPR accumulators and copy every score tile between
# AGPRs and VGPRs around the softmax (hundreds of copies per launch, each
# waiting on a product).  With VGPR accumulators they need no copies and no
# scratch; every other attention kernel compiles to the same code either
# way.  The GEMM is left alone: its 256 accumulators live in AGPRs by design.
SRC_FLAGS = {SRC: ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def build(extra=None, out=LIB) -> str:
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    compile_flags = [f for f in HIPCC_FLAGS if f != "-shared"]
    jobs = []
    for src in SRCS:
        obj = os.path.join(objdir, os.path.splitext(os.path.basename(src))[0] + ".o")
        cmd = [hipcc(), *compile_flags, *SRC_FLAGS.get(src, []), *(extra or []), "-c", src, "-o", obj]
        jobs.append((subprocess.Popen(cmd), cmd, obj))
    failed = [cmd for proc, cmd, _ in jobs if proc.wait() != 0]
    if failed:
        raise subprocess.CalledProcessError(1, failed[0])
    subprocess.run([hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *[obj for _, _, obj in jobs],
                    "-o", out + ".tmp"], check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(sys.argv[1:]))
