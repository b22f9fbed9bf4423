"""MI355X (gfx950) fused attention forward pass.

The compute path is the HIP library ``libfa_mi355x.so`` (C ABI in
``include/fa.h``); :mod:`tile_level_programming_amd.fa` is its ctypes binding.
"""

from .fa import FA_BF16, FA_F16, FaError, fa_fwd, fa_status_string, fwd  # noqa: F401

__all__ = ["fa_fwd", "fa_status_string", "fwd", "FaError", "FA_F16", "FA_BF16"]
