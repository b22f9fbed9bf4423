"""ctypes binding of the C ABI in include/fa.h, include/gemm.h and
include/rowwise.h (argument marshalling only).

Every step of the attention forward pass, of the GEMM with its fused
bias + GELU epilogue and of the row-wise kernels runs in the HIP library
``libfa_mi355x.so``; this module
only loads it, converts arguments and, in the torch-level helpers, allocates
outputs (and the split workspace) with torch.  There is no fallback: if the
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
FA_ERR_SCRATCH_TOO_SMALL = 4
SPLIT_SCRATCH_BYTES = 32 * 1024 * 1024  # FA_SPLIT_SCRATCH_BYTES of include/fa.h


class FaError(RuntimeError):
    def __init__(self, status: int):
        super().__init__(f"attention call failed: {fa_status_string(status)} (status {status})")
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
    lib.fa_fwd_split_count.restype = ctypes.c_int64
    lib.fa_fwd_split_count.argtypes = [ctypes.c_int64] * 5
    lib.fa_fwd_split_workspace_size.restype = ctypes.c_size_t
    lib.fa_fwd_split_workspace_size.argtypes = [ctypes.c_int64] * 6
    lib.fa_fwd_split.restype = ctypes.c_int
    lib.fa_fwd_split.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                 ctypes.c_void_p,
                                 ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                 ctypes.c_int64, ctypes.c_float, ctypes.c_int, ctypes.c_int,
                                 ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.fa_fwd_split_noalloc.restype = ctypes.c_int
    lib.fa_fwd_split_noalloc.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_void_p,
                                         ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                         ctypes.c_int64, ctypes.c_float, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int64, ctypes.c_void_p]
    lib.fa_lse_merge.restype = ctypes.c_int
    lib.fa_lse_merge.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                 ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                 ctypes.c_void_p]
    lib.gemm_bias_gelu.restype = ctypes.c_int
    lib.gemm_bias_gelu.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
    lib.row_softmax.restype = ctypes.c_int
    lib.row_softmax.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                ctypes.c_void_p]
    lib.rmsnorm_silu.restype = ctypes.c_int
    lib.rmsnorm_silu.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                 ctypes.c_float, ctypes.c_int, ctypes.c_void_p]
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


def fa_fwd_split(q: int, k: int, v: int, o: int, lse: int, B: int, H: int, Sq: int, Sk: int, D: int,
                 scale: float, causal: int, dtype: int, n_split: int, workspace: int, workspace_bytes: int,
                 stream: int) -> int:
    """Direct call of the C entry point with raw device addresses; returns the status."""
    return int(_lib.fa_fwd_split(q, k, v, o, lse, B, H, Sq, Sk, D, scale, int(causal), int(dtype),
                                 int(n_split), workspace, int(workspace_bytes), stream))


def fa_fwd_split_noalloc(q: int, k: int, v: int, o: int, lse: int, B: int, H: int, Sq: int, Sk: int, D: int,
                         scale: float, causal: int, dtype: int, n_split: int, stream: int) -> int:
    """Direct call of the C entry point (partials in the library's fixed device
    buffer, no allocation) with raw device addresses; returns the status."""
    return int(_lib.fa_fwd_split_noalloc(q, k, v, o, lse, B, H, Sq, Sk, D, scale, int(causal), int(dtype),
                                         int(n_split), stream))


def fa_lse_merge(o_parts: int, lse_parts: int, n_part: int, rows: int, D: int, o: int, lse: int, dtype: int,
                 stream: int) -> int:
    """Direct call of the C entry point with raw device addresses; returns the status."""
    return int(_lib.fa_lse_merge(o_parts, lse_parts, n_part, rows, D, o, lse, int(dtype), stream))


def gemm_bias_gelu(a: int, w: int, bias: int, c: int, M: int, N: int, K: int, dtype: int, stream: int) -> int:
    """Direct call of the C entry point with raw device addresses (bias 0 = none); returns the status."""
    return int(_lib.gemm_bias_gelu(a, w, bias or None, c, M, N, K, int(dtype), stream))


def linear_gelu(a, w, bias=None, out=None):
    """gelu(a @ w.T + bias) on torch device tensors: a [M, K], w [N, K], bias [N]
    (or None), fp16 or bf16; returns c [M, N].  Runs on torch's current stream."""
    import torch

    if a.dtype not in (torch.float16, torch.bfloat16) or w.dtype != a.dtype:
        raise TypeError("a and w must share one dtype, float16 or bfloat16")
    if bias is not None and bias.dtype != a.dtype:
        raise TypeError("bias must have the dtype of a")
    if a.dim() != 2 or w.dim() != 2 or a.shape[1] != w.shape[1]:
        raise ValueError("a must be [M, K] and w [N, K]")
    M, K = a.shape
    N = w.shape[0]
    if bias is not None and tuple(bias.shape) != (N,):
        raise ValueError("bias must be [N]")
    for t in (a, w) + ((bias,) if bias is not None else ()):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("a, w, bias must be contiguous device tensors")
    _check_same_device(a.device, w, *((bias,) if bias is not None else ()))
    if out is None:
        out = torch.empty((M, N), dtype=a.dtype, device=a.device)
    _check_out(out, "out", (M, N), a.dtype, a.device)
    dt = FA_F16 if a.dtype == torch.float16 else FA_BF16
    stream = torch.cuda.current_stream(a.device).cuda_stream
    st = gemm_bias_gelu(a.data_ptr(), w.data_ptr(), 0 if bias is None else bias.data_ptr(), out.data_ptr(),
                        M, N, K, dt, stream)
    if st != FA_OK:
        raise FaError(st)
    return out


def row_softmax(x: int, y: int, R: int, C: int, dtype: int, stream: int) -> int:
    """Direct call of the C entry point with raw device addresses; returns the status."""
    return int(_lib.row_softmax(x, y, R, C, int(dtype), stream))


def rmsnorm_silu(x: int, g: int, y: int, R: int, C: int, eps: float, dtype: int, stream: int) -> int:
    """Direct call of the C entry point with raw device addresses; returns the status."""
    return int(_lib.rmsnorm_silu(x, g, y, R, C, float(eps), int(dtype), stream))


def _rows_call(x, extra, fn, out):
    import torch

    if x.dtype not in (torch.float16, torch.bfloat16) or x.dim() != 2:
        raise TypeError("x must be a [R, C] float16 or bfloat16 tensor")
    if not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous device tensor")
    if extra is not None:
        if not extra.is_cuda:
            raise ValueError("g must be a device tensor")
        _check_same_device(x.device, extra)
    if out is None:
        out = torch.empty_like(x)
    _check_out(out, "out", x.shape, x.dtype, x.device)
    dt = FA_F16 if x.dtype == torch.float16 else FA_BF16
    st = fn(x, out, dt, torch.cuda.current_stream(x.device).cuda_stream)
    if st != FA_OK:
        raise FaError(st)
    return out


def softmax(x, out=None):
    """Row softmax of a [R, C] device tensor (row_softmax); returns y like x."""
    return _rows_call(x, None, lambda t, o, dt, s: row_softmax(t.data_ptr(), o.data_ptr(), t.shape[0], t.shape[1],
                                                               dt, s), out)


def rmsnorm_silu_rows(x, g, eps: float = 1e-6, out=None):
    """silu(x / rms(x) * g) along the rows of a [R, C] device tensor; g [C]."""
    if x.dim() != 2 or g.dtype != x.dtype or tuple(g.shape) != (x.shape[1],) or not g.is_contiguous():
        raise ValueError("g must be a contiguous [C] tensor of x's dtype")
    return _rows_call(x, g, lambda t, o, dt, s: rmsnorm_silu(t.data_ptr(), g.data_ptr(), o.data_ptr(), t.shape[0],
                                                             t.shape[1], eps, dt, s), out)


def split_count(B: int, H: int, Sq: int, Sk: int, n_split: int = 0) -> int:
    return int(_lib.fa_fwd_split_count(B, H, Sq, Sk, n_split))


def split_workspace_size(B: int, H: int, Sq: int, Sk: int, D: int, n_split: int = 0) -> int:
    return int(_lib.fa_fwd_split_workspace_size(B, H, Sq, Sk, D, n_split))


def fa_status_string(status: int) -> str:
    return _lib.fa_status_string(int(status)).decode()


def _check(q, k, v):
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
    _check_same_device(q.device, k, v)
    B, H, Sq, D = q.shape
    Sk = k.shape[2]
    if tuple(k.shape) != (B, H, Sk, D) or tuple(v.shape) != (B, H, Sk, D):
        raise ValueError("k and v must be [B, H, Sk, D] matching q")
    return B, H, Sq, Sk, D


def _check_out(t, name, shape, dtype, device):
    """A caller-supplied output must match what the kernel writes exactly:
    the C ABI only sees a pointer, so a smaller, mistyped, strided or host
    tensor would be written past its end or fault the device."""
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must have dtype {dtype}, not {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, not {tuple(t.shape)}")
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be on {device}, not {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_same_device(device, *ts):
    for t in ts:
        if t.device != device:
            raise ValueError(f"all tensors must be on {device}; got one on {t.device}")


def fwd_split(q, k, v, causal: bool = False, scale: float | None = None, n_split: int = 0, out=None,
              lse=None, workspace=None):
    """Attention forward split over the keys (fa_fwd_split), for small Sq and
    long Sk.  ``workspace`` is a uint8 device tensor of at least
    :func:`split_workspace_size` bytes (allocated with torch when None).
    Returns (o, lse).  Runs on torch's current stream, no synchronisation.
    """
    import math

    import torch

    B, H, Sq, Sk, D = _check(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    _check_out(out, "out", q.shape, q.dtype, q.device)
    _check_out(lse, "lse", (B, H, Sq), torch.float32, q.device)
    need = split_workspace_size(B, H, Sq, Sk, D, n_split)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    if not isinstance(workspace, torch.Tensor) or not workspace.is_cuda or workspace.device != q.device:
        raise ValueError(f"workspace must be a tensor on {q.device}")
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    dt = FA_F16 if q.dtype == torch.float16 else FA_BF16
    stream = torch.cuda.current_stream(q.device).cuda_stream
    st = fa_fwd_split(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                      B, H, Sq, Sk, D, float(scale), int(causal), dt, int(n_split),
                      workspace.data_ptr(), workspace.numel() * workspace.element_size(), stream)
    if st != FA_OK:
        raise FaError(st)
    return out, lse


def lse_merge(o_parts, lse_parts, dtype):
    """Merge fp32 partials o_parts [G, ..., D] and lse_parts [G, ...] into
    (o [..., D] of torch dtype ``dtype``, lse float32 [...]) with fa_lse_merge."""
    import torch

    G, D = o_parts.shape[0], o_parts.shape[-1]
    lead = tuple(lse_parts.shape[1:])
    if o_parts.dtype != torch.float32 or lse_parts.dtype != torch.float32:
        raise TypeError("partials must be float32")
    if dtype not in (torch.float16, torch.bfloat16):
        raise TypeError("dtype must be torch.float16 or torch.bfloat16")
    if not o_parts.is_cuda or not lse_parts.is_cuda:
        raise ValueError("partials must be device tensors")
    _check_same_device(o_parts.device, lse_parts)
    if tuple(o_parts.shape) != (G, *lead, D) or lse_parts.shape[0] != G:
        raise ValueError("o_parts must be [G, ..., D] and lse_parts [G, ...]")
    if not (o_parts.is_contiguous() and lse_parts.is_contiguous()):
        raise ValueError("partials must be contiguous")
    rows = 1
    for x in lead:
        rows *= int(x)
    o = torch.empty((*lead, D), dtype=dtype, device=o_parts.device)
    lse = torch.empty(lead, dtype=torch.float32, device=o_parts.device)
    dt = FA_F16 if dtype == torch.float16 else FA_BF16
    stream = torch.cuda.current_stream(o_parts.device).cuda_stream
    st = fa_lse_merge(o_parts.data_ptr(), lse_parts.data_ptr(), G, rows, D, o.data_ptr(), lse.data_ptr(),
                      dt, stream)
    if st != FA_OK:
        raise FaError(st)
    return o, lse


def fwd(q, k, v, causal: bool = False, scale: float | None = None, out=None, lse=None):
    """Attention forward on torch device tensors [B, H, S, D] (fp16 or bf16).

    Returns (o, lse): o like q, lse float32 [B, H, Sq].  Runs on torch's
    current stream and does not synchronise.
    """
    import math

    import torch

    B, H, Sq, Sk, D = _check(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    _check_out(out, "out", q.shape, q.dtype, q.device)
    _check_out(lse, "lse", (B, H, Sq), torch.float32, q.device)
    dt = FA_F16 if q.dtype == torch.float16 else FA_BF16
    stream = torch.cuda.current_stream(q.device).cuda_stream
    st = fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                B, H, Sq, Sk, D, float(scale), int(causal), dt, stream)
    if st != FA_OK:
        raise FaError(st)
    return out, lse
