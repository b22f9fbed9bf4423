"""Python driver for the float64 attention oracle (oracle/fa_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's cpu_baseline leg, never by the product package.  It shares no code
with the HIP library; both consume the same seeded bit patterns from
``fa_inputs``.

The C routine evaluates any list of independent query rows single-threaded;
``attention_rows`` fans a row list out over host threads (ctypes releases the
GIL), each thread running the unchanged single-threaded routine on a disjoint
slice.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fa_oracle.c")
_LIB = os.path.join(_HERE, "libfa_oracle.so")

_lib = None
_lock = threading.Lock()

DTYPE_CODE = {"f16": 0, "bf16": 1}


def build() -> str:
    """Compile the oracles with gcc (plain -O2, no fast-math, no FP contraction):
    the attention oracle here, the GEMM + bias + GELU oracle of ``oracle.gemm``
    and the row-wise (softmax, RMSNorm + SiLU) oracles of ``oracle.rowwise``."""
    cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared",
           "-std=c11", "-Wall", "-Wextra", _SRC, "-o", _LIB + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    from . import gemm, rowwise

    gemm.build()
    rowwise.build()
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        lib.fa_oracle_init.restype = None
        lib.fa_oracle_init.argtypes = []
        lib.fa_oracle_decode.restype = None
        lib.fa_oracle_decode.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
        lib.fa_oracle_rows.restype = ctypes.c_int
        lib.fa_oracle_rows.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                       ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                       ctypes.c_int64, ctypes.c_double, ctypes.c_int,
                                       ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
        lib.fa_oracle_rows_range.restype = ctypes.c_int
        lib.fa_oracle_rows_range.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                             ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                             ctypes.c_int64, ctypes.c_double, ctypes.c_int,
                                             ctypes.c_int64, ctypes.c_int64,
                                             ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
        lib.fa_oracle_merge.restype = ctypes.c_int
        lib.fa_oracle_merge.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        lib.fa_oracle_init()
        _lib = lib
        return lib


def decode(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 values of fp16/bf16 bit patterns."""
    lib = _load()
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(b.shape, dtype=np.float64)
    lib.fa_oracle_decode(b.ctypes.data, b.size, DTYPE_CODE[dtype], out.ctypes.data)
    return out


def attention_rows(q, k, v, dtype: str, scale: float, causal: bool, rows=None, threads: int = 1,
                   key_range=None):
    """Oracle O rows and lse for flat query rows ``rows`` (all rows if None).

    q: uint16 [B,H,Sq,D]; k, v: uint16 [B,H,Sk,D].  Returns (o [n, D] float64,
    lse [n] float64) for the requested rows, in the order given.  With
    ``key_range=(a, b)`` only keys a <= j < b take part (causal mask on the
    global key index); rows that see none of them get lse -inf and o 0.
    """
    lib = _load()
    q = np.ascontiguousarray(q, dtype=np.uint16)
    k = np.ascontiguousarray(k, dtype=np.uint16)
    v = np.ascontiguousarray(v, dtype=np.uint16)
    B, H, Sq, D = q.shape
    Sk = k.shape[2]
    if k.shape != (B, H, Sk, D) or v.shape != (B, H, Sk, D):
        raise ValueError("k and v must be [B, H, Sk, D] matching q")
    if rows is None:
        rows = np.arange(B * H * Sq, dtype=np.int64)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    n = rows.size
    o = np.empty((n, D), dtype=np.float64)
    lse = np.empty(n, dtype=np.float64)

    k0, k1 = (0, Sk) if key_range is None else (int(key_range[0]), int(key_range[1]))
    if not 0 <= k0 < k1 <= Sk:
        raise ValueError("key_range must satisfy 0 <= a < b <= Sk")

    def run(a, b):
        if b <= a:
            return 0
        if key_range is None:
            return lib.fa_oracle_rows(q.ctypes.data, k.ctypes.data, v.ctypes.data, DTYPE_CODE[dtype],
                                      B, H, Sq, Sk, D, float(scale), int(bool(causal)),
                                      rows[a:].ctypes.data, b - a,
                                      o[a:].ctypes.data, lse[a:].ctypes.data)
        return lib.fa_oracle_rows_range(q.ctypes.data, k.ctypes.data, v.ctypes.data, DTYPE_CODE[dtype],
                                        B, H, Sq, Sk, D, float(scale), int(bool(causal)), k0, k1,
                                        rows[a:].ctypes.data, b - a,
                                        o[a:].ctypes.data, lse[a:].ctypes.data)

    threads = max(1, int(threads))
    if threads == 1 or n < 2 * threads:
        rc = run(0, n)
        if rc != 0:
            raise RuntimeError("fa_oracle_rows failed")
        return o, lse
    # interleaved blocks balance causal rows of different lengths
    blk = max(1, min(64, n // (threads * 8)))
    starts = list(range(0, n, blk))
    with ThreadPoolExecutor(max_workers=threads) as ex:
        rcs = list(ex.map(lambda a: run(a, min(n, a + blk)), starts))
    if any(rc != 0 for rc in rcs):
        raise RuntimeError("fa_oracle_rows failed")
    return o, lse


def attention(q, k, v, dtype: str, scale: float, causal: bool, threads: int = 1):
    """Full oracle output: (o [B,H,Sq,D] float64, lse [B,H,Sq] float64)."""
    B, H, Sq, D = q.shape
    o, lse = attention_rows(q, k, v, dtype, scale, causal, None, threads)
    return o.reshape(B, H, Sq, D), lse.reshape(B, H, Sq)


def merge(o_parts, lse_parts):
    """Log-sum-exp merge of partial results over disjoint key ranges.

    o_parts: float64 [G, ..., D]; lse_parts: float64 [G, ...] (the same
    leading shape).  Returns (o [..., D], lse [...]), see fa_oracle_merge.
    """
    lib = _load()
    o_parts = np.ascontiguousarray(o_parts, dtype=np.float64)
    lse_parts = np.ascontiguousarray(lse_parts, dtype=np.float64)
    G, D = o_parts.shape[0], o_parts.shape[-1]
    lead = lse_parts.shape[1:]
    if o_parts.shape != (G, *lead, D) or lse_parts.shape[0] != G:
        raise ValueError("o_parts must be [G, ..., D] and lse_parts [G, ...] with the same leading shape")
    nrows = int(np.prod(lead, dtype=np.int64))
    o = np.empty((nrows, D), dtype=np.float64)
    lse = np.empty(nrows, dtype=np.float64)
    rc = lib.fa_oracle_merge(G, nrows, D, o_parts.ctypes.data, lse_parts.ctypes.data,
                             o.ctypes.data, lse.ctypes.data)
    if rc != 0:
        raise RuntimeError("fa_oracle_merge failed")
    return o.reshape(*lead, D), lse.reshape(lead)
