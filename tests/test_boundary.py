"""C ABI boundary checks that need no GPU: the library loads, exports every
function include/fa.h declares with the argument count the binding uses, and
rejects invalid arguments with the documented status before any HIP call."""
from __future__ import annotations

import ctypes
import os
import re

import pytest
import torch

from exact_attention_19_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "fa.h")
FAKE = 0x10000  # an aligned, never-dereferenced address: every case below fails validation first
MISALIGNED = 0x10002


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    decls = {}
    for m in re.finditer(r"\b(?:fa_status|size_t|const char\*)\s+(fa_\w+)\s*\(([^)]*)\)\s*;", text):
        args = [a for a in m.group(2).split(",") if a.strip() and a.strip() != "void"]
        decls[m.group(1)] = len(args)
    return decls


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_header_declares_the_entry_points():
    decls = _declared()
    for name in ("fa_fwd", "fa_bwd", "fa_decode_kvcache", "fa_bwd_workspace_bytes",
                 "fa_decode_workspace_bytes", "fa_last_error", "fa_version"):
        assert name in decls, name


def test_library_exports_every_declared_symbol(lib):
    for name, nargs in _declared().items():
        assert hasattr(lib, name), f"{name} not exported"
        assert name in _lib.SIGNATURES, f"{name} not bound"
        assert len(_lib.SIGNATURES[name][1]) == nargs, f"{name}: binding has wrong argument count"


def _fwd(lib, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, Hq=4, Hkv=2, N=16, d=128, scale=0.1, causal=0,
         dtype=_lib.FA_BF16):
    return lib.fa_fwd(q, k, v, o, lse, B, Hq, Hkv, N, d, scale, causal, dtype, None)


@pytest.mark.parametrize("kw, status", [
    (dict(q=None), _lib.FA_ERR_INVALID_ARG),
    (dict(lse=None), _lib.FA_ERR_INVALID_ARG),
    (dict(o=MISALIGNED), _lib.FA_ERR_INVALID_ARG),
    (dict(B=0), _lib.FA_ERR_INVALID_ARG),
    (dict(N=-3), _lib.FA_ERR_INVALID_ARG),
    (dict(Hq=6, Hkv=4), _lib.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), _lib.FA_ERR_INVALID_ARG),
    (dict(scale=float("inf")), _lib.FA_ERR_INVALID_ARG),
    (dict(scale=-1.0), _lib.FA_ERR_INVALID_ARG),
    (dict(d=96), _lib.FA_ERR_UNSUPPORTED),
    (dict(d=256), _lib.FA_ERR_UNSUPPORTED),
    (dict(dtype=7), _lib.FA_ERR_UNSUPPORTED),
])
def test_fwd_validation(lib, kw, status):
    assert _fwd(lib, **kw) == status
    assert lib.fa_last_error().decode().startswith("fa_fwd")


def test_bwd_validation(lib):
    args = [FAKE] * 10 + [1 << 20, 1, 4, 2, 64, 128, 0.1, 1, _lib.FA_BF16, None]
    bad_dtype = list(args)
    bad_dtype[18] = _lib.FA_FP32
    assert lib.fa_bwd(*bad_dtype) == _lib.FA_ERR_UNSUPPORTED
    no_ws = list(args)
    no_ws[9] = None
    assert lib.fa_bwd(*no_ws) == _lib.FA_ERR_WORKSPACE
    small = list(args)
    small[10] = lib.fa_bwd_workspace_bytes(1, 4, 2, 64, 128) - 1
    assert lib.fa_bwd(*small) == _lib.FA_ERR_WORKSPACE
    bad_heads = list(args)
    bad_heads[12], bad_heads[13] = 3, 2
    assert lib.fa_bwd(*bad_heads) == _lib.FA_ERR_INVALID_ARG
    assert "fa_bwd" in lib.fa_last_error().decode()


def test_window_validation(lib):
    args = [FAKE] * 5 + [1, 4, 2, 64, 128, 0.1, 0, 3, 0, _lib.FA_BF16, None]
    bad = list(args)
    bad[12] = -2  # window_left
    assert lib.fa_fwd_window(*bad) == _lib.FA_ERR_INVALID_ARG
    d96 = list(args)
    d96[9] = 96  # d = 64 and 128 are the head dims built
    assert lib.fa_fwd_window(*d96) == _lib.FA_ERR_UNSUPPORTED
    f32 = list(args)
    f32[14] = _lib.FA_FP32
    assert lib.fa_fwd_window(*f32) == _lib.FA_ERR_UNSUPPORTED
    null_lse = list(args)
    null_lse[4] = None
    assert lib.fa_fwd_window(*null_lse) == _lib.FA_ERR_INVALID_ARG
    assert lib.fa_last_error().decode().startswith("fa_fwd_window")


def test_bwd_window_validation(lib):
    args = [FAKE] * 10 + [1 << 20, 1, 4, 2, 64, 128, 0.1, 1, 16, 0, _lib.FA_BF16, None]
    bad = list(args)
    bad[18] = -3  # window_left
    assert lib.fa_bwd_window(*bad) == _lib.FA_ERR_INVALID_ARG
    d96 = list(args)
    d96[15] = 96
    assert lib.fa_bwd_window(*d96) == _lib.FA_ERR_UNSUPPORTED
    assert lib.fa_last_error().decode().startswith("fa_bwd_window")


def test_blocksparse_validation(lib):
    args = [FAKE] * 6 + [0, 1, 4, 2, 1000, 128, 0.1, 1, _lib.FA_BF16, None]
    for idx, val, status in ((5, None, _lib.FA_ERR_INVALID_ARG),      # block_mask
                             (6, 3, _lib.FA_ERR_INVALID_ARG),         # stride below nb*nb
                             (11, 96, _lib.FA_ERR_UNSUPPORTED),       # d
                             (10, 300000, _lib.FA_ERR_UNSUPPORTED),   # N too large
                             (14, _lib.FA_FP32, _lib.FA_ERR_UNSUPPORTED)):
        bad = list(args)
        bad[idx] = val
        assert lib.fa_fwd_blocksparse(*bad) == status, (idx, val)
        assert lib.fa_last_error().decode().startswith("fa_fwd_blocksparse")


def test_varlen_validation(lib):
    # q k v o lse cu_q cu_k, B, max_q, total_q, total_k, Hq, Hkv, d, scale, causal, wl, wr, dtype, stream
    args = [FAKE] * 7 + [3, 100, 200, 150, 4, 2, 128, 0.1, 1, -1, -1, _lib.FA_BF16, None]
    for idx, val, status in ((7, 0, _lib.FA_ERR_INVALID_ARG),       # B
                             (8, 0, _lib.FA_ERR_INVALID_ARG),       # max_seqlen_q
                             (9, 0, _lib.FA_ERR_INVALID_ARG),       # total_q
                             (10, -1, _lib.FA_ERR_INVALID_ARG),     # total_k
                             (11, 3, _lib.FA_ERR_INVALID_ARG),      # Hq not a multiple of Hkv
                             (13, 96, _lib.FA_ERR_UNSUPPORTED),     # d
                             (17, -5, _lib.FA_ERR_INVALID_ARG),     # window_right
                             (18, _lib.FA_FP32, _lib.FA_ERR_UNSUPPORTED),
                             (5, None, _lib.FA_ERR_INVALID_ARG),    # cu_seqlens_q
                             (6, FAKE + 2, _lib.FA_ERR_INVALID_ARG)):  # misaligned cu_seqlens_k
        bad = list(args)
        bad[idx] = val
        assert lib.fa_fwd_varlen(*bad) == status, (idx, val)
        assert lib.fa_last_error().decode().startswith("fa_fwd_varlen")


def test_decode_ext_validation(lib):
    # q kc vc seqlens table, max_pages, num_pages, page_size, k_new, v_new, o, lse, ws, ws_bytes,
    # B, Hq, Hkv, cache_rows, d, scale, causal, num_splits, dtype, stream
    # 40 pages of 64 rows: 2560 rows per sequence, so one split (a 2560-row chunk) is too few
    ws = lib.fa_decode_workspace_bytes(2, 8, 2, 64 * 40, 128, 0)
    args = [FAKE] * 5 + [40, 40, 64, FAKE, FAKE, FAKE, FAKE, FAKE, ws, 2, 8, 2, 0, 128, 0.1, 0, 0,
                         _lib.FA_BF16, None]
    for idx, val, status in ((7, 48, _lib.FA_ERR_INVALID_ARG),      # page_size not a power of two
                             (7, 8, _lib.FA_ERR_INVALID_ARG),       # page_size < 16
                             (5, 0, _lib.FA_ERR_INVALID_ARG),       # max_pages_per_seq
                             (6, 0, _lib.FA_ERR_INVALID_ARG),       # num_pages
                             (9, None, _lib.FA_ERR_INVALID_ARG),    # v_new without k_new
                             (21, 1, _lib.FA_ERR_INVALID_ARG),      # too few splits for pages
                             (13, ws - 4, _lib.FA_ERR_WORKSPACE),
                             (22, _lib.FA_FP32, _lib.FA_ERR_UNSUPPORTED)):
        bad = list(args)
        bad[idx] = val
        assert lib.fa_decode_kvcache_ext(*bad) == status, (idx, val)
        assert lib.fa_last_error().decode().startswith("fa_decode_kvcache_ext")


def test_decode_validation(lib):
    ws = lib.fa_decode_workspace_bytes(2, 8, 2, 1000, 128, 0)
    args = [FAKE] * 7 + [ws, 2, 8, 2, 1000, 128, 0.1, 0, 0, _lib.FA_BF16, None]
    neg = list(args)
    neg[15] = -1  # num_splits
    assert lib.fa_decode_kvcache(*neg) == _lib.FA_ERR_INVALID_ARG
    small = list(args)
    small[7] = ws - 4
    assert lib.fa_decode_kvcache(*small) == _lib.FA_ERR_WORKSPACE
    nolse_bad = list(args)
    nolse_bad[3] = None  # cache_seqlens
    assert lib.fa_decode_kvcache(*nolse_bad) == _lib.FA_ERR_INVALID_ARG
    fp32 = list(args)
    fp32[16] = _lib.FA_FP32  # dtype
    assert lib.fa_decode_kvcache(*fp32) == _lib.FA_ERR_UNSUPPORTED


def test_workspace_sizes(lib):
    assert lib.fa_bwd_workspace_bytes(1, 96, 96, 8192, 128) == 2 * 96 * 8192 * 4  # D and LSE*log2(e)
    assert lib.fa_bwd_workspace_bytes(0, 1, 1, 1, 64) == 0
    # default split: 1024-row chunks -> 32 splits for a 32768-row cache
    o_bytes = 64 * 32 * 32 * 128 * 4
    lse_bytes = 64 * 32 * 32 * 4
    assert lib.fa_decode_workspace_bytes(64, 32, 8, 32768, 128, 0) == o_bytes + lse_bytes
    # one split
    assert lib.fa_decode_workspace_bytes(2, 4, 2, 100, 64, 1) == (2 * 4 * 64 * 4 + 255) // 256 * 256 + 256


def test_binding_rejects_host_tensors():
    import exact_attention_19_amd as fa

    x = torch.zeros(1, 8, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.fa_fwd(x, x, x)


def test_error_message_is_per_call(lib):
    assert _fwd(lib, d=80) == _lib.FA_ERR_UNSUPPORTED
    assert "d=80" in lib.fa_last_error().decode()
    assert _fwd(lib, B=0) == _lib.FA_ERR_INVALID_ARG
    assert "sizes" in lib.fa_last_error().decode()
    assert isinstance(lib.fa_version(), bytes) and ctypes.sizeof(ctypes.c_size_t) == 8


def test_noalloc_decode_rejects_sizes_beyond_its_scratch(lib):
    """Partials larger than the 64 MiB scratch array: FA_ERR_WORKSPACE before
    any HIP call (an explicit split count plans without querying a device)."""
    B, Hq, Hkv, N, d, ns = 512, 64, 8, 65536, 128, 64
    assert lib.fa_decode_workspace_bytes(B, Hq, Hkv, N, d, ns) > (64 << 20)
    st = lib.fa_decode_kvcache_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, None, B, Hq, Hkv, N, d, 0.1, 0, ns,
                                       _lib.FA_BF16, None)
    assert st == _lib.FA_ERR_WORKSPACE
    assert lib.fa_last_error().decode().startswith("fa_decode_kvcache_noalloc")
    assert lib.fa_decode_kvcache_noalloc(None, FAKE, FAKE, FAKE, FAKE, None, 2, 4, 2, 64, 128, 0.1, 0, 0,
                                         _lib.FA_BF16, None) == _lib.FA_ERR_INVALID_ARG
