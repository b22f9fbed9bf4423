"""ctypes binding of the C ABI in include/fa.h (argument marshalling only).

Every step of the attention forward pass runs in the HIP library
``libfa_mi355x.so``; this module only loads it, converts arguments and, in
:func:`fwd`, allocates the outputs with torch.  There is no fallback: if the
library is missing, importing the binding raises.
"""

from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfa_mi355x.so")

FA_F16 = 0
FA_BF16 = 1
FA_OK = 0
FA_ERR_INVALID_ARG = 1
FA_ERR_UNSUPPORTED = 2
FA_ERR_LAUNCH = 3


class FaError(RuntimeError):
    def __init__(self, status: int):
        super().__init__(f"fa_fwd failed: {fa_status_string(status)} (status {status})")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"HIP library {LIB_PATH} is not built; run __graft_entry__.build() "
            "(hipcc --offload-arch=gfx950) first")
    lib = ctypes.CDLL(LIB_PATH)
    lib.fa_fwd.restype = ctypes.c_int
    lib.fa_fwd.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                           ctypes.c_void_p,
                           ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                           ctypes.c_int64, ctypes.c_float, ctypes.c_int, ctypes.c_int,
                           ctypes.c_void_p]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_status_string.argtypes = [ctypes.c_int]
    return lib


_lib = _load()


def library() -> ctypes.CDLL:
    return _lib


def fa_fwd(q: int, k: int, v: int, o: int, lse: int, B: int, H: int, Sq: int, Sk: int, D: int,
           scale: float, causal: int, dtype: int, stream: int) -> int:
    """Direct call of the C entry point with raw device addresses; returns the status."""
    return int(_lib.fa_fwd(q, k, v, o, lse, B, H, Sq, Sk, D, scale, int(causal), int(dtype), stream))


def fa_status_string(status: int) -> str:
    return _lib.fa_status_string(int(status)).decode()


def fwd(q, k, v, causal: bool = False, scale: float | None = None, out=None, lse=None):
    """Attention forward on torch device tensors [B, H, S, D] (fp16 or bf16).

    Returns (o, lse): o like q, lse float32 [B, H, Sq].  Runs on torch's
    current stream and does not synchronise.
    """
    import math

    import torch

    if q.dtype not in (torch.float16, torch.bfloat16):
        raise TypeError("q, k, v must be float16 or bfloat16")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, S, D]")
    for t in (q, k, v):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("q, k, v must be contiguous device tensors")
    B, H, Sq, D = q.shape
    Sk = k.shape[2]
    if tuple(k.shape) != (B, H, Sk, D) or tuple(v.shape) != (B, H, Sk, D):
        raise ValueError("k and v must be [B, H, Sk, D] matching q")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    dt = FA_F16 if q.dtype == torch.float16 else FA_BF16
    stream = torch.cuda.current_stream(q.device).cuda_stream
    st = fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                B, H, Sq, Sk, D, float(scale), int(causal), dt, stream)
    if st != FA_OK:
        raise FaError(st)
    return out, lse
