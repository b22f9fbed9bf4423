"""Python driver for the float64 GEMM + bias + GELU oracle (oracle/gemm_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's cpu_baseline leg, never by the product package.  It shares no
code with the HIP library; both consume the same seeded bit patterns from
``fa_inputs``.  Rows of the output are independent and are fanned out over
host threads, each running the unchanged single-threaded C routine.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gemm_oracle.c")
_LIB = os.path.join(_HERE, "libgemm_oracle.so")
_lib = None
_lock = threading.Lock()
DTYPE_CODE = {"f16": 0, "bf16": 1}


def build() -> str:
    """Compile the oracle with gcc (plain -O2, no fast-math, no FP contraction)."""
    cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared",
           "-std=c11", "-Wall", "-Wextra", _SRC, "-o", _LIB + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        lib.gemm_oracle_gelu.restype = ctypes.c_double
        lib.gemm_oracle_gelu.argtypes = [ctypes.c_double]
        lib.gemm_oracle_rows.restype = ctypes.c_int
        lib.gemm_oracle_rows.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                         ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                         ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
        _lib = lib
        return lib


def gelu(x: float) -> float:
    """x * Phi(x) in double (the oracle's own routine)."""
    return float(_load().gemm_oracle_gelu(float(x)))


def gemm_rows(a, w, bias, dtype: str, rows=None, threads: int = 1, want_pre: bool = False):
    """Oracle rows of gelu(a @ w.T + bias).

    a: uint16 [M, K]; w: uint16 [N, K]; bias: uint16 [N] or None.  Returns
    c [n, N] float64 for the requested rows (all if None), and with
    ``want_pre`` also the pre-activation x [n, N].
    """
    lib = _load()
    a = np.ascontiguousarray(a, dtype=np.uint16)
    w = np.ascontiguousarray(w, dtype=np.uint16)
    M, K = a.shape
    N = w.shape[0]
    if w.shape != (N, K):
        raise ValueError("w must be [N, K] matching a [M, K]")
    b = None
    if bias is not None:
        b = np.ascontiguousarray(bias, dtype=np.uint16)
        if b.shape != (N,):
            raise ValueError("bias must be [N]")
    if rows is None:
        rows = np.arange(M, dtype=np.int64)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    n = rows.size
    c = np.empty((n, N), dtype=np.float64)
    pre = np.empty((n, N), dtype=np.float64) if want_pre else None

    def run(lo, hi):
        if hi <= lo:
            return 0
        return lib.gemm_oracle_rows(a.ctypes.data, w.ctypes.data, None if b is None else b.ctypes.data,
                                    DTYPE_CODE[dtype], M, N, K, rows[lo:].ctypes.data, hi - lo,
                                    None if pre is None else pre[lo:].ctypes.data, c[lo:].ctypes.data)

    threads = max(1, int(threads))
    if threads == 1 or n < 2 * threads:
        rcs = [run(0, n)]
    else:
        blk = max(1, n // (threads * 4))
        with ThreadPoolExecutor(max_workers=threads) as ex:
            rcs = list(ex.map(lambda lo: run(lo, min(n, lo + blk)), range(0, n, blk)))
    if any(rc != 0 for rc in rcs):
        raise RuntimeError("gemm_oracle_rows failed")
    return (c, pre) if want_pre else c
