"""Torch-facing binding of the C ABI: argument marshalling only.

Each function checks device, dtype, contiguity and shapes, allocates the
outputs (and workspace) with torch, and passes raw device pointers plus the
current HIP stream to the library. Every step of the computation runs in the
library's HIP kernels.

Layouts (as in include/fa.h): q, o, dout, dq ``[B, N, Hq, d]``;
k, v, dk, dv ``[B, N, Hkv, d]``; lse ``[B, Hq, N]`` float32.
"""
from __future__ import annotations

import math

import torch

from . import _lib

_DT = {torch.bfloat16: _lib.FA_BF16, torch.float32: _lib.FA_FP32}


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _check_tensor(name, t, dtype=None, ndim=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU device")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got {tuple(t.shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def fa_fwd(q, k, v, scale=None, causal=False, out=None, lse=None):
    """Attention forward. Returns (o, lse)."""
    _check_tensor("q", q, ndim=4)
    if q.dtype not in _DT:
        raise ValueError(f"unsupported dtype {q.dtype}")
    _check_tensor("k", k, q.dtype, 4, q.device)
    _check_tensor("v", v, q.dtype, 4, q.device)
    B, N, Hq, d = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[1] != N or k.shape[3] != d:
        raise ValueError(f"k/v shape {tuple(k.shape)} does not match q {tuple(q.shape)}")
    Hkv = k.shape[2]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    _check_tensor("out", out, q.dtype, 4, q.device)
    if lse is None:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    _check_tensor("lse", lse, torch.float32, 3, q.device)
    if out.shape != q.shape or tuple(lse.shape) != (B, Hq, N):
        raise ValueError("out/lse shapes do not match q")
    st = _lib.load().fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, N, d, scale,
                            int(bool(causal)), _DT[q.dtype], _stream(q.device))
    _lib.check(st)
    return out, lse


def fa_fwd_window(q, k, v, window, scale=None, causal=False, out=None, lse=None):
    """Sliding-window forward (bf16, d = 64 or 128): window = (left, right), -1 is
    unbounded on that side. Returns (o, lse) laid out as fa_fwd, written into
    out / lse when given."""
    _check_tensor("q", q, torch.bfloat16, 4)
    _check_tensor("k", k, torch.bfloat16, 4, q.device)
    _check_tensor("v", v, torch.bfloat16, 4, q.device)
    B, N, Hq, d = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[1] != N or k.shape[3] != d:
        raise ValueError(f"k/v shape {tuple(k.shape)} does not match q {tuple(q.shape)}")
    Hkv = k.shape[2]
    wl, wr = (int(x) for x in window)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device) if lse is None else lse
    _check_tensor("out", out, torch.bfloat16, 4, q.device)
    _check_tensor("lse", lse, torch.float32, 3, q.device)
    if out.shape != q.shape or tuple(lse.shape) != (B, Hq, N):
        raise ValueError("out/lse shapes do not match q")
    st = _lib.load().fa_fwd_window(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, N, d, scale,
                                   int(bool(causal)), wl, wr, _lib.FA_BF16, _stream(q.device))
    _lib.check(st)
    return out, lse


def fa_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, scale=None, causal=False,
                  window=(-1, -1)):
    """Forward over packed variable-length sequences (bf16, d = 64 or 128).

    q [total_q, Hq, d], k/v [total_k, Hkv, d]; cu_seqlens_q/k: int32 [B + 1]
    device prefix sums. Returns (o [total_q, Hq, d], lse [Hq, total_q])."""
    _check_tensor("q", q, torch.bfloat16, 3)
    dev = q.device
    _check_tensor("k", k, torch.bfloat16, 3, dev)
    _check_tensor("v", v, torch.bfloat16, 3, dev)
    _check_tensor("cu_seqlens_q", cu_seqlens_q, torch.int32, 1, dev)
    _check_tensor("cu_seqlens_k", cu_seqlens_k, torch.int32, 1, dev)
    total_q, Hq, d = q.shape
    total_k, Hkv = k.shape[0], k.shape[1]
    if k.shape != v.shape or k.shape[2] != d:
        raise ValueError(f"k/v shape {tuple(k.shape)} does not match q {tuple(q.shape)}")
    if cu_seqlens_q.shape != cu_seqlens_k.shape or cu_seqlens_q.numel() < 2:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both be [B + 1]")
    B = cu_seqlens_q.numel() - 1
    wl, wr = (int(x) for x in window)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out = torch.empty_like(q)
    lse = torch.empty((Hq, total_q), dtype=torch.float32, device=dev)
    st = _lib.load().fa_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(cu_seqlens_q),
                                   _ptr(cu_seqlens_k), B, int(max_seqlen_q), total_q, total_k, Hq, Hkv, d, scale,
                                   int(bool(causal)), wl, wr, _lib.FA_BF16, _stream(dev))
    _lib.check(st)
    return out, lse


def fa_fwd_blocksparse(q, k, v, block_mask, scale=None, causal=False):
    """Block-sparse forward (bf16, d = 64 or 128): block_mask is a uint8 device tensor
    of [nb, nb] (shared) or [B, Hq, nb, nb] bytes, nb = ceil(N / 128).
    Returns (o, lse) laid out as fa_fwd."""
    _check_tensor("q", q, torch.bfloat16, 4)
    dev = q.device
    _check_tensor("k", k, torch.bfloat16, 4, dev)
    _check_tensor("v", v, torch.bfloat16, 4, dev)
    _check_tensor("block_mask", block_mask, torch.uint8, None, dev)
    B, N, Hq, d = q.shape
    Hkv = k.shape[2]
    nb = (N + 127) // 128
    if block_mask.dim() == 2 and tuple(block_mask.shape) == (nb, nb):
        stride = 0
    elif block_mask.dim() == 4 and tuple(block_mask.shape) == (B, Hq, nb, nb):
        stride = nb * nb
    else:
        raise ValueError(f"block_mask must be [{nb}, {nb}] or [{B}, {Hq}, {nb}, {nb}]")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
    st = _lib.load().fa_fwd_blocksparse(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(block_mask), stride,
                                        B, Hq, Hkv, N, d, scale, int(bool(causal)), _lib.FA_BF16, _stream(dev))
    _lib.check(st)
    return out, lse


def fa_bwd(q, k, v, o, dout, lse, scale=None, causal=False, window=(-1, -1), dq=None, dk=None, dv=None,
           deterministic=True):
    """Attention backward from the forward's O and LSE. Returns (dq, dk, dv),
    written into the given tensors when passed. A window other than (-1, -1)
    calls fa_bwd_window (d = 64 or 128); deterministic=False calls fa_bwd_atomic
    (d = 128, no window: dQ accumulated with fp32 atomics)."""
    _check_tensor("q", q, torch.bfloat16, 4)
    dev = q.device
    for name, t in (("k", k), ("v", v), ("o", o), ("dout", dout)):
        _check_tensor(name, t, torch.bfloat16, 4, dev)
    _check_tensor("lse", lse, torch.float32, 3, dev)
    B, N, Hq, d = q.shape
    Hkv = k.shape[2]
    if o.shape != q.shape or dout.shape != q.shape or k.shape != v.shape or tuple(lse.shape) != (B, Hq, N):
        raise ValueError("inconsistent shapes for fa_bwd")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    lib = _lib.load()
    wl, wr = (int(x) for x in window)
    atomic = not deterministic
    if atomic and (wl >= 0 or wr >= 0):
        raise ValueError("the atomic backward has no window")
    ws_bytes = (lib.fa_bwd_atomic_workspace_bytes if atomic else lib.fa_bwd_workspace_bytes)(B, Hq, Hkv, N, d)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _check_tensor("dq", dq, torch.bfloat16, 4, dev)
    _check_tensor("dk", dk, torch.bfloat16, 4, dev)
    _check_tensor("dv", dv, torch.bfloat16, 4, dev)
    if dq.shape != q.shape or dk.shape != k.shape or dv.shape != v.shape:
        raise ValueError("dq/dk/dv must have the shapes of q/k/v")
    if atomic:
        st = lib.fa_bwd_atomic(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk),
                               _ptr(dv), _ptr(ws), ws_bytes, B, Hq, Hkv, N, d, scale, int(bool(causal)), _lib.FA_BF16,
                               _stream(dev))
    elif wl < 0 and wr < 0:
        st = lib.fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
                        _ptr(ws), ws_bytes, B, Hq, Hkv, N, d, scale, int(bool(causal)), _lib.FA_BF16, _stream(dev))
    else:
        st = lib.fa_bwd_window(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk),
                               _ptr(dv), _ptr(ws), ws_bytes, B, Hq, Hkv, N, d, scale, int(bool(causal)), wl, wr,
                               _lib.FA_BF16, _stream(dev))
    _lib.check(st)
    return dq, dk, dv


def fa_decode_kvcache(q, k_cache, v_cache, cache_seqlens, scale=None, causal=False, num_splits=0,
                      out=None, lse=None, workspace=None):
    """Decode one query token per sequence against a KV cache. Returns (o, lse).

    q: [B, Hq, d]; k_cache, v_cache: [B, N, Hkv, d]; cache_seqlens: int32 [B].
    """
    _check_tensor("q", q, torch.bfloat16, 3)
    dev = q.device
    _check_tensor("k_cache", k_cache, torch.bfloat16, 4, dev)
    _check_tensor("v_cache", v_cache, torch.bfloat16, 4, dev)
    _check_tensor("cache_seqlens", cache_seqlens, torch.int32, 1, dev)
    B, Hq, d = q.shape
    _, N, Hkv, _ = k_cache.shape
    if k_cache.shape != v_cache.shape or k_cache.shape[0] != B or k_cache.shape[3] != d or cache_seqlens.shape[0] != B:
        raise ValueError("inconsistent shapes for fa_decode_kvcache")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    lib = _lib.load()
    ws_bytes = lib.fa_decode_workspace_bytes(B, Hq, Hkv, N, d, int(num_splits))
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    st = lib.fa_decode_kvcache(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(cache_seqlens), _ptr(out), _ptr(lse),
                               _ptr(workspace), workspace.numel(), B, Hq, Hkv, N, d, scale, int(bool(causal)),
                               int(num_splits), _lib.FA_BF16, _stream(dev))
    _lib.check(st)
    return out, lse


def fa_decode_kvcache_noalloc(q, k_cache, v_cache, cache_seqlens, out, lse=None, scale=None, num_splits=0):
    """fa_decode_kvcache for callers that cannot allocate: no workspace is
    allocated (the library's per-device scratch array holds the partials) and
    the outputs are the caller's ``out`` [B, Hq, d] (and ``lse`` [B, Hq] or
    None). Calls that overlap on one device race. Returns (out, lse)."""
    _check_tensor("q", q, torch.bfloat16, 3)
    dev = q.device
    _check_tensor("k_cache", k_cache, torch.bfloat16, 4, dev)
    _check_tensor("v_cache", v_cache, torch.bfloat16, 4, dev)
    _check_tensor("cache_seqlens", cache_seqlens, torch.int32, 1, dev)
    _check_tensor("out", out, torch.bfloat16, 3, dev)
    B, Hq, d = q.shape
    _, N, Hkv, _ = k_cache.shape
    if (k_cache.shape != v_cache.shape or k_cache.shape[0] != B or k_cache.shape[3] != d
            or cache_seqlens.shape[0] != B or out.shape != q.shape):
        raise ValueError("inconsistent shapes for fa_decode_kvcache_noalloc")
    if lse is not None:
        _check_tensor("lse", lse, torch.float32, 2, dev)
        if tuple(lse.shape) != (B, Hq):
            raise ValueError("lse must be [B, Hq]")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    st = _lib.load().fa_decode_kvcache_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(cache_seqlens), _ptr(out),
                                               _ptr(lse), B, Hq, Hkv, N, d, scale, 0, int(num_splits), _lib.FA_BF16,
                                               _stream(dev))
    _lib.check(st)
    return out, lse


def fa_decode_kvcache_ext(q, k_cache, v_cache, cache_seqlens, block_table=None, k_new=None, v_new=None, scale=None,
                          num_splits=0):
    """Decode with an optional in-place append (k_new, v_new: [B, Hkv, d]) and
    an optional paged cache (k_cache, v_cache: [num_pages, page_size, Hkv, d],
    block_table: int32 [B, max_pages]). Returns (o [B, Hq, d], lse [B, Hq])."""
    _check_tensor("q", q, torch.bfloat16, 3)
    dev = q.device
    _check_tensor("k_cache", k_cache, torch.bfloat16, 4, dev)
    _check_tensor("v_cache", v_cache, torch.bfloat16, 4, dev)
    _check_tensor("cache_seqlens", cache_seqlens, torch.int32, 1, dev)
    B, Hq, d = q.shape
    if k_cache.shape != v_cache.shape or k_cache.shape[3] != d or cache_seqlens.shape[0] != B:
        raise ValueError("inconsistent shapes for fa_decode_kvcache_ext")
    Hkv = k_cache.shape[2]
    if block_table is not None:
        _check_tensor("block_table", block_table, torch.int32, 2, dev)
        if block_table.shape[0] != B:
            raise ValueError("block_table must be [B, max_pages]")
        num_pages, page_size = k_cache.shape[0], k_cache.shape[1]
        max_pages = block_table.shape[1]
        cap = max_pages * page_size
        rows = 0
    else:
        if k_cache.shape[0] != B:
            raise ValueError("a contiguous cache must be [B, rows, Hkv, d]")
        num_pages = page_size = max_pages = 0
        rows = cap = k_cache.shape[1]
    if (k_new is None) != (v_new is None):
        raise ValueError("k_new and v_new go together")
    if k_new is not None:
        _check_tensor("k_new", k_new, torch.bfloat16, 3, dev)
        _check_tensor("v_new", v_new, torch.bfloat16, 3, dev)
        if tuple(k_new.shape) != (B, Hkv, d) or k_new.shape != v_new.shape:
            raise ValueError("k_new/v_new must be [B, Hkv, d]")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    lib = _lib.load()
    ws_bytes = lib.fa_decode_workspace_bytes(B, Hq, Hkv, cap, d, num_splits)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    st = lib.fa_decode_kvcache_ext(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(cache_seqlens), _ptr(block_table),
                                   max_pages, num_pages, page_size, _ptr(k_new), _ptr(v_new), _ptr(o), _ptr(lse),
                                   _ptr(ws), ws_bytes, B, Hq, Hkv, rows, d, scale, 0, int(num_splits),
                                   _lib.FA_BF16, _stream(dev))
    _lib.check(st)
    return o, lse
