"""Python driver for the float64 row-wise oracles (oracle/rowwise_oracle.c):
row softmax and fused RMSNorm + SiLU.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's cpu_baseline leg, never by the product package.  Rows are
independent and are fanned out over host threads, each running the
unchanged single-threaded C routine.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "rowwise_oracle.c")
_LIB = os.path.join(_HERE, "librowwise_oracle.so")
_lib = None
_lock = threading.Lock()
DTYPE_CODE = {"f16": 0, "bf16": 1}


def build() -> str:
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
        lib.rowwise_oracle_softmax.restype = ctypes.c_int
        lib.rowwise_oracle_softmax.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                               ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
        lib.rowwise_oracle_silu.restype = ctypes.c_double
        lib.rowwise_oracle_silu.argtypes = [ctypes.c_double]
        lib.rowwise_oracle_rmsnorm_silu.restype = ctypes.c_int
        lib.rowwise_oracle_rmsnorm_silu.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                                                    ctypes.c_int64, ctypes.c_double, ctypes.c_void_p,
                                                    ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
        _lib = lib
        return lib


def silu(z: float) -> float:
    return float(_load().rowwise_oracle_silu(float(z)))


def _fan(n, threads, run):
    threads = max(1, int(threads))
    if threads == 1 or n < 2 * threads:
        rcs = [run(0, n)]
    else:
        blk = max(1, n // (threads * 4))
        with ThreadPoolExecutor(max_workers=threads) as ex:
            rcs = list(ex.map(lambda lo: run(lo, min(n, lo + blk)), range(0, n, blk)))
    if any(rc != 0 for rc in rcs):
        raise RuntimeError("row-wise oracle failed")


def softmax_rows(x, dtype: str, rows=None, threads: int = 1):
    """Oracle softmax of rows of x (uint16 [R, C]); returns float64 [n, C]."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.uint16)
    R, C = x.shape
    rows = np.arange(R, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    y = np.empty((rows.size, C), dtype=np.float64)

    def run(lo, hi):
        if hi <= lo:
            return 0
        return lib.rowwise_oracle_softmax(x.ctypes.data, DTYPE_CODE[dtype], R, C, rows[lo:].ctypes.data, hi - lo,
                                          y[lo:].ctypes.data)

    _fan(rows.size, threads, run)
    return y


def rmsnorm_silu_rows(x, g, dtype: str, eps: float, rows=None, threads: int = 1, want_z: bool = False):
    """Oracle silu(x / rms(x) * g) of rows of x (uint16 [R, C]) with weight g
    (uint16 [C]); returns float64 [n, C] (and the pre-activation z)."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.uint16)
    g = np.ascontiguousarray(g, dtype=np.uint16)
    R, C = x.shape
    if g.shape != (C,):
        raise ValueError("g must be [C]")
    rows = np.arange(R, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    y = np.empty((rows.size, C), dtype=np.float64)
    z = np.empty((rows.size, C), dtype=np.float64) if want_z else None

    def run(lo, hi):
        if hi <= lo:
            return 0
        return lib.rowwise_oracle_rmsnorm_silu(x.ctypes.data, g.ctypes.data, DTYPE_CODE[dtype], R, C, float(eps),
                                               rows[lo:].ctypes.data, hi - lo,
                                               None if z is None else z[lo:].ctypes.data, y[lo:].ctypes.data)

    _fan(rows.size, threads, run)
    return (y, z) if want_z else y
