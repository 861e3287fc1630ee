"""Plain fp64 CPU oracle for exact scaled-dot-product attention.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module. The product path (the HIP
library and its Python binding) never calls it and shares no code with it.

What is computed, and where the pages define it:

* Forward: ``O = softmax(Q K^T * scale) V`` per (batch, query head).
  Qiita FlashAttention tutorial (GeneLab_999), section 2.2 gives
  ``softmax(QK^T / sqrt(d)) V``; the hysenlabs digest of the flash-attention
  README ("FlashAttentionで見る出力と運用記録") gives the same with an explicit
  ``softmax_scale``. The "standard attention" of tutorial section 4.1 (and
  "基本アイデア" in the abeam.tech summary of the FlashAttention paper) is
  computed literally: S is materialised, softmax is taken row by row, then
  P V. FlashAttention is exact (abeam summary, "Softmax をブロック単位で正しく
  計算する"): only the order of evaluation differs, so the plain definition is
  the oracle for every tiled GPU result.
* Causal masking keeps key j for query i iff j <= i + (Nk - Nq): the mask is
  aligned to the bottom-right corner when the query and key lengths differ
  (hysenlabs digest, "制約を切り分ける確認", v2.1 entry). With Nq == Nk this is
  the usual j <= i.
* MQA/GQA: Hq must be a multiple of Hkv (hysenlabs digest, "出力と運用記録").
  Query head h reads key/value head h // (Hq // Hkv) (consecutive groups); the
  pages only fix divisibility, so this grouping is a stated reading.
* Logsumexp: the per-row normalisation statistic the forward keeps for the
  recompute backward (abeam summary, "用語解説: Recomputation" and
  "学習時の backward では再計算を使う") is taken to be the natural-log
  logsumexp of the scaled, masked scores, ``LSE_i = log sum_j exp(S_ij)``.
* Backward: the gradient of ``L = sum(O * dO)`` through the definition above,
  i.e. the textbook softmax Jacobian (the pages say only that the backward
  recomputes attention from the saved statistics):
  ``dV = P^T dO``, ``dP = dO V^T``, ``D_i = sum_j P_ij dP_ij``,
  ``dS = P * (dP - D)``, ``dQ = scale dS K``, ``dK = scale dS^T Q``;
  dK and dV of a key/value head sum over the query heads of its group.
* Decode with a KV cache (hysenlabs digest, ``flash_attn_with_kvcache``): one
  query row per (sequence, head) attends keys 0 .. L_b - 1 of its cache
  (with one query the bottom-right causal mask keeps every cached key).
  The same function updates k_cache / v_cache in place (outputs section),
  and the v2.5 changelog entry adds a paged KV cache. The readings taken:
  with new rows k_new, v_new ([B, Hkv, d], one token per sequence) the token
  is written at row L_b and attention covers rows 0 .. L_b; a paged cache is
  a pool of pages [P, page_size, Hkv, d] and a block table [B, max_pages]
  maps logical row t of sequence b to row t % page_size of page
  table[b, t // page_size].

* Sliding window (hysenlabs digest: ``window_size`` among the arguments in
  "出力と運用記録", sliding-window attention in the v2.3 entry of
  "制約を切り分ける確認"). The pages give no formula; the reading taken is a
  band about the bottom-right-aligned diagonal: with window (wl, wr), query i
  keeps key j iff ``i + off - wl <= j <= i + off + wr`` where
  ``off = Nk - Nq``, and a negative side is unbounded. Causal masking is
  applied on top (it equals wr = 0).
* Variable-length batches (the v2.0 entry of the same changelog: the
  "unpadded" functions became "varlen"): sequences are packed along the row
  axis and delimited by prefix sums ``cu_q`` / ``cu_k`` (``[B + 1]``,
  ``cu[0] = 0``); sequence b is an independent attention problem on rows
  ``cu_q[b]:cu_q[b+1]`` of Q and ``cu_k[b]:cu_k[b+1]`` of K and V, with the
  bottom-right causal alignment inside each sequence. This packing is a
  stated reading (the pages only name the functions).

* Block-sparse attention (abeam summary, "Block-sparse への拡張"): blocks of
  the score matrix known to be zero are left out and FlashAttention runs on
  the rest. Reading taken: a 0/1 block mask over ``block`` x ``block`` tiles
  of (query, key) positions; positions in a 0 block are excluded exactly
  like masked ones (score -inf), on top of any causal mask.

A fully masked row (possible when causal and Nq > Nk, with a window that
leaves a row no keys, or with a block mask) has O = 0 and LSE = -inf by
convention.

Inputs are numpy arrays of any float dtype; they are converted exactly to
float64. Layouts: q, o, do, dq ``[B, Nq, Hq, d]``; k, v, dk, dv
``[B, Nk, Hkv, d]``; lse ``[B, Hq, Nq]``.
"""
from __future__ import annotations

import numpy as np


def _check_heads(hq: int, hkv: int) -> int:
    if hkv <= 0 or hq % hkv != 0:
        raise ValueError(f"Hq={hq} must be a positive multiple of Hkv={hkv}")
    return hq // hkv


def head_probs(q: np.ndarray, k: np.ndarray, scale: float, causal: bool, rows=None, nq=None, window=(-1, -1),
               keep_extra=None):
    """Scores, probabilities and logsumexp for one (batch, head).

    q: [R, d] query rows, k: [Nk, d] (float64). ``rows`` gives the absolute
    index of each query row among ``nq`` queries (default: all rows,
    0 .. R-1 of R), which the causal mask and the window need. ``window`` is
    (wl, wr), a negative side being unbounded. Returns (S, P, lse) where S
    holds -inf at masked positions, P = softmax(S) row-wise (0 where
    masked) and lse = log sum_j exp(S_ij) (-inf for a fully masked row).
    """
    nk = k.shape[0]
    if rows is None:
        rows = np.arange(q.shape[0])
        nq = q.shape[0]
    s = scale * (q @ k.T)
    diag = np.asarray(rows)[:, None] + (nk - nq)   # the bottom-right-aligned diagonal of each row
    j = np.arange(nk)[None, :]
    if causal:
        keep = j <= diag
        s = np.where(keep, s, -np.inf)
    wl, wr = window
    if wl >= 0:
        s = np.where(j >= diag - wl, s, -np.inf)
    if wr >= 0:
        s = np.where(j <= diag + wr, s, -np.inf)
    if keep_extra is not None:               # [R, Nk] booleans (block-sparse pattern)
        s = np.where(keep_extra, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    e = np.exp(s - m_safe)
    l = e.sum(axis=1, keepdims=True)
    with np.errstate(divide="ignore", invalid="ignore"):
        p = np.where(empty, 0.0, e / np.where(empty, 1.0, l))
        lse = np.where(empty[:, 0], -np.inf, m_safe[:, 0] + np.log(np.where(empty[:, 0], 1.0, l[:, 0])))
    return s, p, lse


def attn_fwd(q, k, v, scale: float, causal: bool, window=(-1, -1)):
    """O = softmax(Q K^T * scale [+ causal mask] [+ window]) V and the per-row
    logsumexp.

    q: [B, Nq, Hq, d]; k, v: [B, Nk, Hkv, d]. Returns (o [B, Nq, Hq, d],
    lse [B, Hq, Nq]) in float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    b_, nq, hq, d = q.shape
    _, nk, hkv, _ = k.shape
    g = _check_heads(hq, hkv)
    o = np.zeros((b_, nq, hq, d))
    lse = np.zeros((b_, hq, nq))
    for b in range(b_):
        for h in range(hq):
            kh = h // g
            _, p, lse_bh = head_probs(q[b, :, h, :], k[b, :, kh, :], scale, causal, window=window)
            o[b, :, h, :] = p @ v[b, :, kh, :]
            lse[b, h, :] = lse_bh
    return o, lse


def attn_bwd(q, k, v, do, scale: float, causal: bool, window=(-1, -1)):
    """Gradients of L = sum(O * dO) with respect to Q, K and V.

    P is recomputed from Q and K (nothing from a forward pass is reused).
    Returns (dq [B, Nq, Hq, d], dk [B, Nk, Hkv, d], dv [B, Nk, Hkv, d]) and
    D = rowsum(P * dP) = rowsum(dO * O), shaped [B, Hq, Nq].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    b_, nq, hq, d = q.shape
    _, nk, hkv, _ = k.shape
    g = _check_heads(hq, hkv)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dd = np.zeros((b_, hq, nq))
    for b in range(b_):
        for h in range(hq):
            kh = h // g
            qh, kk, vv, doh = q[b, :, h, :], k[b, :, kh, :], v[b, :, kh, :], do[b, :, h, :]
            _, p, _ = head_probs(qh, kk, scale, causal, window=window)
            dv[b, :, kh, :] += p.T @ doh
            dp = doh @ vv.T
            drow = (p * dp).sum(axis=1, keepdims=True)
            ds = p * (dp - drow)
            dq[b, :, h, :] = scale * (ds @ kk)
            dk[b, :, kh, :] += scale * (ds.T @ qh)
            dd[b, h, :] = drow[:, 0]
    return dq, dk, dv, dd


def attn_decode(q, k_cache, v_cache, cache_seqlens, scale: float):
    """One query row per (sequence, head) against that sequence's cache.

    q: [B, Hq, d]; k_cache, v_cache: [B, Lmax, Hkv, d] (only rows
    < cache_seqlens[b] are read); cache_seqlens: [B] ints in [1, Lmax].
    Returns (o [B, Hq, d], lse [B, Hq]) in float64.
    """
    q = np.asarray(q, dtype=np.float64)
    b_, hq, d = q.shape
    hkv = k_cache.shape[2]
    g = _check_heads(hq, hkv)
    o = np.zeros((b_, hq, d))
    lse = np.zeros((b_, hq))
    for b in range(b_):
        n = int(cache_seqlens[b])
        if n < 1 or n > k_cache.shape[1]:
            raise ValueError(f"cache_seqlens[{b}]={n} outside [1, {k_cache.shape[1]}]")
        kb = np.asarray(k_cache[b, :n], dtype=np.float64)
        vb = np.asarray(v_cache[b, :n], dtype=np.float64)
        for h in range(hq):
            kh = h // g
            _, p, lse_h = head_probs(q[b, h][None, :], kb[:, kh, :], scale, causal=False)
            o[b, h] = (p @ vb[:, kh, :])[0]
            lse[b, h] = lse_h[0]
    return o, lse


def attn_fwd_varlen(q, k, v, cu_q, cu_k, scale: float, causal: bool, window=(-1, -1)):
    """Forward over packed variable-length sequences.

    q: [total_q, Hq, d]; k, v: [total_k, Hkv, d]; cu_q, cu_k: [B + 1]
    prefix sums of the query and key lengths. Sequence b is the forward of
    ``attn_fwd`` on rows cu_q[b]:cu_q[b+1] and cu_k[b]:cu_k[b+1].
    Returns (o [total_q, Hq, d], lse [Hq, total_q]) in float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    cu_q = np.asarray(cu_q, dtype=np.int64)
    cu_k = np.asarray(cu_k, dtype=np.int64)
    if cu_q.shape != cu_k.shape or cu_q[0] != 0 or cu_k[0] != 0:
        raise ValueError("cu_q and cu_k must be [B + 1] prefix sums starting at 0")
    if np.any(np.diff(cu_q) < 0) or np.any(np.diff(cu_k) < 0):
        raise ValueError("sequence lengths must be non-negative")
    if cu_q[-1] != q.shape[0] or cu_k[-1] != k.shape[0]:
        raise ValueError("cu_q[-1] / cu_k[-1] must equal the packed row counts")
    hq = q.shape[1]
    o = np.zeros_like(q)
    lse = np.full((hq, q.shape[0]), -np.inf)
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        if q1 == q0:
            continue
        if k1 == k0:            # no keys: every row is empty (O = 0, LSE = -inf)
            continue
        ob, lb = attn_fwd(q[None, q0:q1], k[None, k0:k1], v[None, k0:k1], scale, causal, window)
        o[q0:q1] = ob[0]
        lse[:, q0:q1] = lb[0]
    return o, lse


def block_keep(block_mask, block: int, nq: int, nk: int):
    """Expand a [ceil(nq/block), ceil(nk/block)] 0/1 block mask to [nq, nk]."""
    bm = np.asarray(block_mask).astype(bool)
    return bm[np.arange(nq)[:, None] // block, np.arange(nk)[None, :] // block]


def attn_fwd_blocksparse(q, k, v, block_mask, block: int, scale: float, causal: bool):
    """Forward restricted to the 1-blocks of ``block_mask``.

    q: [B, N, Hq, d]; k, v: [B, N, Hkv, d]; block_mask: [nbq, nbk] shared by
    every (batch, head), or [B, Hq, nbq, nbk]. Returns (o, lse) as attn_fwd.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    b_, nq, hq, d = q.shape
    nk, hkv = k.shape[1], k.shape[2]
    g = _check_heads(hq, hkv)
    bm = np.asarray(block_mask)
    o = np.zeros((b_, nq, hq, d))
    lse = np.zeros((b_, hq, nq))
    for b in range(b_):
        for h in range(hq):
            kh = h // g
            mask_bh = bm if bm.ndim == 2 else bm[b, h]
            _, p, lse_bh = head_probs(q[b, :, h, :], k[b, :, kh, :], scale, causal,
                                      keep_extra=block_keep(mask_bh, block, nq, nk))
            o[b, :, h, :] = p @ v[b, :, kh, :]
            lse[b, h, :] = lse_bh
    return o, lse


def gather_paged(pages, block_table, b: int, n: int):
    """Logical rows 0 .. n-1 of sequence b from a paged cache: row t is row
    t % page_size of page block_table[b, t // page_size]."""
    page_size = pages.shape[1]
    t = np.arange(n)
    return pages[np.asarray(block_table)[b, t // page_size], t % page_size]


def attn_decode_paged(q, k_pages, v_pages, block_table, cache_seqlens, scale: float, k_new=None, v_new=None):
    """Decode against a paged cache, optionally appending one new token.

    q: [B, Hq, d]; k_pages, v_pages: [P, page_size, Hkv, d];
    block_table: [B, max_pages] ints; cache_seqlens: [B]. With k_new/v_new
    ([B, Hkv, d]) the new token is written at logical row L_b of copies of
    the caches and attention covers L_b + 1 rows. Returns (o [B, Hq, d],
    lse [B, Hq], k_pages', v_pages') with the updated copies.
    """
    k_pages = np.array(k_pages, dtype=np.float64)
    v_pages = np.array(v_pages, dtype=np.float64)
    page_size = k_pages.shape[1]
    table = np.asarray(block_table)
    lens = np.asarray(cache_seqlens).astype(np.int64)
    if k_new is not None:
        for b in range(len(lens)):
            t = int(lens[b])
            pg, r = table[b, t // page_size], t % page_size
            k_pages[pg, r] = np.asarray(k_new[b], dtype=np.float64)
            v_pages[pg, r] = np.asarray(v_new[b], dtype=np.float64)
        lens = lens + 1
    b_ = len(lens)
    n_max = int(lens.max())
    kc = np.zeros((b_, n_max) + k_pages.shape[2:])
    vc = np.zeros_like(kc)
    for b in range(b_):
        kc[b, :lens[b]] = gather_paged(k_pages, table, b, int(lens[b]))
        vc[b, :lens[b]] = gather_paged(v_pages, table, b, int(lens[b]))
    o, lse = attn_decode(q, kc, vc, lens, scale)
    return o, lse, k_pages, v_pages


def attn_fwd_rows(q, k, v, scale: float, causal: bool, b: int, h: int, rows):
    """Forward for selected query rows of one (batch, head) only.

    Used to check large problems on sampled outputs: the cost is
    O(len(rows) * Nk * d). Returns (o [len(rows), d], lse [len(rows)]).
    """
    hq, hkv = q.shape[2], k.shape[2]
    kh = h // _check_heads(hq, hkv)
    rows = np.asarray(rows)
    qh = np.asarray(q[b, rows, h, :], dtype=np.float64)
    kk = np.asarray(k[b, :, kh, :], dtype=np.float64)
    vv = np.asarray(v[b, :, kh, :], dtype=np.float64)
    _, p, lse = head_probs(qh, kk, scale, causal, rows=rows, nq=q.shape[1])
    return p @ vv, lse


def attn_bwd_dq_rows(q, k, v, do, scale: float, causal: bool, b: int, h: int, rows):
    """dQ and D for selected query rows of one (batch, query head).

    Row i of dQ depends only on row i of P and of dP (the backward formulas
    in the module docstring: D_i = sum_j P_ij dP_ij, dS_i = P_i (dP_i - D_i),
    dQ_i = scale dS_i K), so sampled rows cost O(len(rows) * Nk * d) and
    check problems too large for the full backward. Returns
    (dq [len(rows), d], D [len(rows)]).
    """
    hq, hkv = q.shape[2], k.shape[2]
    kv_head = h // _check_heads(hq, hkv)
    rows = np.asarray(rows)
    qr = np.asarray(q[b, rows, h, :], dtype=np.float64)
    dor = np.asarray(do[b, rows, h, :], dtype=np.float64)
    kk = np.asarray(k[b, :, kv_head, :], dtype=np.float64)
    vv = np.asarray(v[b, :, kv_head, :], dtype=np.float64)
    _, pr, _ = head_probs(qr, kk, scale, causal, rows=rows, nq=q.shape[1])
    dpr = dor @ vv.T
    dr = (pr * dpr).sum(axis=1)
    dsr = pr * (dpr - dr[:, None])
    return scale * (dsr @ kk), dr
