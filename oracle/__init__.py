"""fp64 CPU oracle for exact attention (test infrastructure only).

Only ``tests/``, the smoke check and the benchmark's CPU-baseline leg import
this package; the HIP product path never does.
"""
from .attention import (attn_bwd, attn_bwd_dq_rows, attn_decode, attn_decode_paged, attn_fwd, attn_fwd_blocksparse, attn_fwd_rows,
                        attn_fwd_varlen, block_keep, gather_paged, head_probs)

__all__ = ["attn_fwd", "attn_bwd", "attn_bwd_dq_rows", "attn_decode", "attn_decode_paged", "attn_fwd_blocksparse", "attn_fwd_rows",
           "attn_fwd_varlen", "block_keep", "gather_paged", "head_probs"]
