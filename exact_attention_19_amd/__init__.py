"""Exact FlashAttention-style attention for MI355X (gfx950).

The computation lives in libfa_mi355x.so (hand-written HIP kernels behind the
C ABI of include/fa.h); this package only marshals torch tensors into it.
"""
from ._lib import FaError, load
from .attention import (fa_bwd, fa_decode_kvcache, fa_decode_kvcache_ext, fa_decode_kvcache_noalloc, fa_fwd,
                        fa_fwd_blocksparse, fa_fwd_varlen, fa_fwd_window)

__all__ = ["fa_fwd", "fa_fwd_window", "fa_fwd_varlen", "fa_fwd_blocksparse", "fa_bwd", "fa_decode_kvcache",
           "fa_decode_kvcache_ext", "fa_decode_kvcache_noalloc", "FaError", "load"]
