"""MI355X (gfx950) fused attention forward pass.

The compute path is the HIP library ``libfa_mi355x.so`` (C ABI in
``include/fa.h``, ``include/gemm.h`` and ``include/rowwise.h``); :mod:`tile_level_programming_amd.fa` is its ctypes binding.
"""

from .fa import (FA_BF16, FA_F16, FaError, fa_fwd, fa_fwd_split, fa_lse_merge, fa_status_string,  # noqa: F401
                 fwd, fwd_split, gemm_bias_gelu, linear_gelu, lse_merge, rmsnorm_silu, rmsnorm_silu_rows, row_softmax,
                 softmax, split_count, split_workspace_size)

__all__ = ["fa_fwd", "fa_fwd_split", "fa_lse_merge", "fa_status_string", "fwd", "fwd_split", "lse_merge",
           "split_count", "split_workspace_size", "gemm_bias_gelu", "linear_gelu", "row_softmax", "softmax",
           "rmsnorm_silu", "rmsnorm_silu_rows", "FaError", "FA_F16", "FA_BF16"]
