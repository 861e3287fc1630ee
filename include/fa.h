/*
 * fa.h - C ABI of the MI355X (gfx950) exact-attention library (libfa_mi355x.so).
 *
 * Every entry point computes exact scaled-dot-product attention
 *     O = softmax(Q K^T * scale [+ causal mask]) V
 * as defined in the Qiita FlashAttention tutorial (GeneLab_999), section 2.2,
 * and in the hysenlabs digest of the flash-attention README (section on
 * outputs: softmax(Q @ K^T * softmax_scale) @ V, with MQA/GQA when the number
 * of query heads is a multiple of the number of key/value heads). The scores
 * S and probabilities P are never written to device memory: Q, K and V tiles
 * are staged on chip and an online softmax (tutorial section 4.3) carries the
 * per-row running maximum and sum (abeam.tech summary of the FlashAttention
 * paper, "Softmax をブロック単位で正しく計算する").
 *
 * Conventions shared by all entry points
 * --------------------------------------
 * Layouts (row-major, last dimension contiguous, no padding between rows):
 *   q, o, dout, dq : [B, N, Hq,  d]
 *   k, v, dk, dv   : [B, N, Hkv, d]
 *   lse            : [B, Hq, N] float32, natural-log logsumexp of the scaled,
 *                    masked scores of each query row: log sum_j exp(S_ij).
 * GQA grouping: query head h reads key/value head h / (Hq / Hkv).
 * Causal masking keeps key j for query i iff j <= i (queries and keys have
 *   the same length N here, where bottom-right and top-left alignment agree).
 * dtype: FA_BF16 (bfloat16 storage, float32 accumulation; outputs rounded to
 *   nearest even) or FA_FP32 (float32 throughout; fa_fwd only).
 * Supported head dims: d = 64 or 128.
 *
 * Ownership: every pointer is device memory owned by the caller (including
 *   workspaces). The library allocates and frees nothing, never synchronises
 *   the device, and keeps no state except a thread-local error message.
 * Asynchrony: work is enqueued on `stream` (a hipStream_t; NULL is the
 *   default stream) and the call returns after enqueueing. Results are valid
 *   once the stream has reached that point.
 * Errors: arguments are validated before any HIP call; on failure nothing is
 *   launched and a non-zero fa_status is returned. fa_last_error() then
 *   returns a message for the calling thread. No C++ exception crosses the
 *   ABI. NaN or Inf in the inputs propagate to the outputs; they are not
 *   detected.
 */
#ifndef FA_MI355X_FA_H
#define FA_MI355X_FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = 1, /* null/misaligned pointer, non-positive size, Hq % Hkv != 0,
                             non-finite or non-positive scale, bad cache length range */
  FA_ERR_UNSUPPORTED = 2, /* head dim or dtype not implemented for this entry point */
  FA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than the *_workspace_bytes query */
  FA_ERR_HIP = 4          /* a HIP launch failed; fa_last_error() has hipGetErrorString */
} fa_status;

typedef enum { FA_BF16 = 0, FA_FP32 = 1 } fa_dtype;

/*
 * Forward pass: O and the per-row logsumexp.
 * Defined by the attention formula above; the forward keeps only the
 * normalisation statistic (LSE) needed to recompute attention in the backward
 * pass (abeam summary, "用語解説: Recomputation").
 *   q [B,N,Hq,d], k/v [B,N,Hkv,d] in: dtype;  o [B,N,Hq,d] out: dtype;
 *   lse [B,Hq,N] float32 out (may not be NULL).
 * Pointers must be 16-byte aligned (lse: 4-byte).
 */
fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int Hq, int Hkv, int N, int d, float scale, int causal,
                 int dtype, void* stream);

/*
 * Forward pass with a sliding window (sliding-window attention: hysenlabs
 * digest, `window_size` among the arguments in the outputs section and the
 * v2.3 entry of the changelog in the constraints section). Query i keeps key
 * j iff i - window_left <= j <= i + window_right (a side of -1 is unbounded;
 * causal = 1 additionally keeps only j <= i). With both sides -1 this is
 * fa_fwd. Layouts, alignment and outputs as fa_fwd.
 * A row that sees no key has O = 0 and LSE = -inf.
 * Errors: FA_ERR_INVALID_ARG as fa_fwd, or a window side < -1;
 *   FA_ERR_UNSUPPORTED for a window with dtype != FA_BF16 (d = 64 or 128).
 */
fa_status fa_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse,
                        int B, int Hq, int Hkv, int N, int d, float scale, int causal,
                        int window_left, int window_right, int dtype, void* stream);

/*
 * Forward pass over packed variable-length sequences (the "varlen"
 * functions of the v2.0 changelog entry, hysenlabs digest, constraints
 * section), optionally causal and/or windowed. The B sequences are packed
 * along the row axis:
 *   q, o [total_q, Hq, d] bf16;  k, v [total_k, Hkv, d] bf16;
 *   lse  [Hq, total_q] float32 out;
 *   cu_seqlens_q, cu_seqlens_k: device int32 [B + 1] prefix sums of the query
 *   and key lengths (cu[0] = 0, non-decreasing, cu_q[B] = total_q,
 *   cu_k[B] = total_k). Sequence b is an independent attention problem on
 *   rows cu_q[b] .. cu_q[b+1]-1 of q/o and cu_k[b] .. cu_k[b+1]-1 of k/v.
 * Causal masking and the window are aligned to the bottom-right corner of each
 *   sequence (v2.1 entry): with Nq, Nk the lengths and off = Nk - Nq, query i
 *   keeps key j iff j <= i + off (causal) and
 *   i + off - window_left <= j <= i + off + window_right (a side of -1 is
 *   unbounded). A row that sees no key (e.g. causal with Nq > Nk) has O = 0,
 *   LSE = -inf.
 * max_seqlen_q must be >= every query length: it sizes the launch, and rows of
 *   a longer sequence past max_seqlen_q are left unwritten. Prefix sums are
 *   read on the device and clamped to [0, total], so malformed values cannot
 *   cause accesses outside the tensors (their results are unspecified).
 * d = 64 or 128, FA_BF16 only. Pointers 16-byte aligned (lse, cu_*: 4-byte).
 * Errors: FA_ERR_INVALID_ARG for NULL/misaligned pointers, B, Hq, Hkv,
 *   max_seqlen_q or total_q <= 0, total_k < 0, Hq % Hkv != 0, a bad scale or a
 *   window side < -1; FA_ERR_UNSUPPORTED for d not 64 or 128, or dtype != FA_BF16.
 */
fa_status fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                        const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                        int B, int max_seqlen_q, int total_q, int total_k,
                        int Hq, int Hkv, int d, float scale, int causal,
                        int window_left, int window_right, int dtype, void* stream);

/*
 * Block-sparse forward (the block-sparse FlashAttention of the abeam.tech
 * summary, "Block-sparse への拡張": blocks known to be zero are skipped and the
 * rest is computed as usual). block_mask holds one byte per 128 x 128 block of
 * (query, key) positions, nb = ceil(N / 128) rows of nb bytes, row-major;
 * (b, hq) uses block_mask + (b * Hq + hq) * mask_head_stride (stride 0: one
 * mask for every batch entry and head). Positions in a zero block are excluded
 * like masked ones; causal = 1 applies the causal mask as well. A row that
 * keeps no key has O = 0, LSE = -inf. Skipped blocks cost neither loads nor
 * arithmetic. Layouts, alignment and outputs as fa_fwd.
 * Errors: as fa_fwd (d = 64 or 128), plus FA_ERR_UNSUPPORTED for dtype != FA_BF16 or
 * N > 262144; FA_ERR_INVALID_ARG for a NULL mask or a stride that is neither 0
 * nor >= nb * nb.
 */
fa_status fa_fwd_blocksparse(const void* q, const void* k, const void* v, void* o, float* lse,
                             const uint8_t* block_mask, long long mask_head_stride,
                             int B, int Hq, int Hkv, int N, int d, float scale, int causal,
                             int dtype, void* stream);

/* Bytes of device workspace fa_bwd needs for these sizes (256-byte aligned). */
size_t fa_bwd_workspace_bytes(int B, int Hq, int Hkv, int N, int d);

/*
 * Backward pass: gradients of L = sum(O * dout) with respect to Q, K and V,
 * recomputing the attention tiles from Q, K and the saved LSE instead of
 * storing S or P (abeam summary, "学習時の backward では再計算を使う").
 *   q, k, v: as in fa_fwd; o [B,N,Hq,d] and lse: the outputs of fa_fwd for
 *   the same inputs; dout [B,N,Hq,d]: upstream gradient.
 *   dq [B,N,Hq,d], dk/dv [B,N,Hkv,d] out (dk/dv sum over the query heads of
 *   each group). bf16 only. The result is deterministic (no atomics).
 *   workspace: device memory of at least fa_bwd_workspace_bytes(...) bytes,
 *   256-byte aligned; its contents on entry do not matter.
 */
fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                 const float* lse, void* dq, void* dk, void* dv,
                 void* workspace, size_t workspace_bytes,
                 int B, int Hq, int Hkv, int N, int d, float scale, int causal,
                 int dtype, void* stream);

/*
 * One stage of fa_bwd, for callers that schedule or time the stages
 * separately. fa_bwd is exactly stage 0, then 1, then 2 on one stream, with
 * the same arguments and workspace (stage 0 writes D = rowsum(dO * O) and the
 * logsumexp in log2 units into the workspace, stages 1 and 2 read them):
 *   stage 0: D;  stage 1: dK and dV;  stage 2: dQ.
 * Pointers a stage does not use may be NULL (stage 0 reads only o, dout, lse;
 * stage 1 writes only dk, dv; stage 2 writes only dq). Any other stage
 * number returns FA_ERR_INVALID_ARG.
 */
fa_status fa_bwd_stage(int stage, const void* q, const void* k, const void* v, const void* o,
                       const void* dout, const float* lse, void* dq, void* dk, void* dv,
                       void* workspace, size_t workspace_bytes,
                       int B, int Hq, int Hkv, int N, int d, float scale, int causal,
                       int dtype, void* stream);

/*
 * Backward pass of the sliding-window forward (fa_fwd_window): the same
 * gradients as fa_bwd with attention restricted to the band
 * i - window_left <= j <= i + window_right (a side of -1 is unbounded;
 * causal additionally keeps j <= i). Deterministic: no atomics, every sum is
 * taken in a fixed order (the deterministic backward of the v2.4 changelog
 * entry, hysenlabs digest, constraints section, holds for every backward
 * here). Arguments, layouts, workspace and errors as fa_bwd (d = 64 or 128),
 * plus FA_ERR_INVALID_ARG for a window side < -1. With both sides -1 this is
 * fa_bwd.
 */
fa_status fa_bwd_window(const void* q, const void* k, const void* v, const void* o, const void* dout,
                        const float* lse, void* dq, void* dk, void* dv, void* workspace,
                        size_t workspace_bytes, int B, int Hq, int Hkv, int N, int d, float scale,
                        int causal, int window_left, int window_right, int dtype, void* stream);

/*
 * Non-deterministic backward with the same inputs, outputs and layouts as
 * fa_bwd: one fused kernel per (batch, kv head, 128 keys) computes dK and
 * dV as fa_bwd does and also dQ, which it accumulates in fp32 with atomic
 * adds (the recompute backward of the abeam summary, "学習時の backward では
 * 再計算を使う", with the S and dP products done once for all three
 * gradients). The flash-attention API takes a `deterministic` flag and its
 * changelog adds the deterministic backward in v2.4 (hysenlabs digest,
 * "出力と運用記録" and "制約を切り分ける確認"); here fa_bwd is that
 * deterministic backward and this is the other one. dK and dV are bitwise
 * equal to fa_bwd's; dQ may differ from run to run in its last bits (the
 * order of the fp32 additions).
 *   workspace: at least fa_bwd_atomic_workspace_bytes(...) bytes (D and
 *   LSE*log2(e) as for fa_bwd, then a [B,N,Hq,d] float32 dQ accumulator),
 *   256-byte aligned.
 * d = 128, bf16 only (FA_ERR_UNSUPPORTED otherwise); errors as fa_bwd.
 */
size_t fa_bwd_atomic_workspace_bytes(int B, int Hq, int Hkv, int N, int d);
fa_status fa_bwd_atomic(const void* q, const void* k, const void* v, const void* o, const void* dout,
                        const float* lse, void* dq, void* dk, void* dv,
                        void* workspace, size_t workspace_bytes,
                        int B, int Hq, int Hkv, int N, int d, float scale, int causal,
                        int dtype, void* stream);
/* fa_bwd_atomic one launch at a time (for timing): stage 0 computes D and
 * LSE*log2(e) and zeroes the dQ accumulator, stage 1 runs the fused kernel,
 * stage 2 writes dq from the accumulator. */
fa_status fa_bwd_atomic_stage(int stage, const void* q, const void* k, const void* v, const void* o,
                              const void* dout, const float* lse, void* dq, void* dk, void* dv,
                              void* workspace, size_t workspace_bytes,
                              int B, int Hq, int Hkv, int N, int d, float scale, int causal,
                              int dtype, void* stream);

/* Bytes of device workspace fa_decode_kvcache needs (num_splits as passed to it).
 * With num_splits = 0 the size depends on the current device (the balanced
 * split described below sizes its partials by the device's resident
 * workgroups): query it with the device current that will run the call. */
size_t fa_decode_workspace_bytes(int B, int Hq, int Hkv, int N, int d, int num_splits);

/*
 * Decode against a KV cache: one new query token per sequence attends the
 * first cache_seqlens[b] rows of that sequence's cache (the inference path
 * of flash_attn_with_kvcache in the hysenlabs digest, "出力と運用記録"; the
 * v2.2 changelog entry adds it for short queries). The cache is read in
 * splits along the sequence, each split producing a partial (O, LSE), and a
 * second kernel merges the partials with LSE weights.
 *   q [B,Hq,d] in; k_cache/v_cache [B,N,Hkv,d] in (N = cache capacity;
 *   rows >= cache_seqlens[b] are never read); cache_seqlens: int32 [B] in
 *   device memory, each in [1, N] (a value outside that range makes that
 *   sequence's output O = 0, LSE = -inf rather than reading out of range);
 *   o [B,Hq,d] out; lse [B,Hq] float32 out, or NULL.
 *   causal: accepted for symmetry; with one query aligned to the bottom-right
 *   corner every cached key is visible, so it does not change the result.
 *   num_splits: number of sequence splits (0 = chosen by the library). With
 *     0, when Hkv is a multiple of 512 / d and B <= 1024, the valid rows of
 *     all sequences, concatenated, are cut into equal ranges (as many as the
 *     device has resident workgroup slots, per block of kv heads) and the
 *     partials of each sequence are merged; otherwise each sequence is cut
 *     into chunks of up to 1024 rows. A positive value cuts each sequence
 *     into that many equal chunks.
 *   workspace: at least fa_decode_workspace_bytes(..., num_splits) bytes.
 * bf16 only.
 */
fa_status fa_decode_kvcache(const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* cache_seqlens, void* o, float* lse,
                            void* workspace, size_t workspace_bytes,
                            int B, int Hq, int Hkv, int N, int d, float scale, int causal,
                            int num_splits, int dtype, void* stream);

/*
 * fa_decode_kvcache without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). Same arguments, results and errors as
 * fa_decode_kvcache, whose kernels it launches; the split partials go to a
 * file-scope device array of FA_NOALLOC_SCRATCH_BYTES (64 MiB) that each
 * device the library runs on holds until the process ends. The call itself
 * allocates and frees nothing; its first call on a device looks up the
 * array's address there.
 *   Sizes whose partials exceed the array (fa_decode_workspace_bytes(...,
 *   num_splits) > FA_NOALLOC_SCRATCH_BYTES) return FA_ERR_WORKSPACE before any
 *   launch; the 64-sequence, Hq=32, Hkv=8, d=128, 32k-row cache decode needs
 *   about a sixth of it.
 * Every call on one device shares that device's array, and the array keeps
 * the last call's contents (nothing in it needs to start at zero): calls
 * that overlap on one device, on different streams or threads, race.
 * Serialise them (one stream, or synchronise between calls).
 */
#define FA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
fa_status fa_decode_kvcache_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                    const int32_t* cache_seqlens, void* o, float* lse,
                                    int B, int Hq, int Hkv, int N, int d, float scale, int causal,
                                    int num_splits, int dtype, void* stream);

/*
 * Decode with an in-place cache append and/or a paged KV cache
 * (flash_attn_with_kvcache updates k_cache/v_cache in place: hysenlabs
 * digest, outputs section; paged KV cache: v2.5 entry of the changelog in
 * the constraints section). One query per sequence as fa_decode_kvcache.
 *   block_table == NULL: contiguous cache k_cache, v_cache [B, cache_rows, Hkv, d];
 *     each sequence holds N = cache_rows rows.
 *   block_table != NULL: paged cache k_cache, v_cache [num_pages, page_size, Hkv, d]
 *     (page_size a power of two >= 16) and block_table: device int32
 *     [B, max_pages_per_seq]; logical row t of sequence b is row
 *     t % page_size of page block_table[b][t / page_size]. Each sequence
 *     holds N = max_pages_per_seq * page_size rows; cache_rows is ignored.
 *     Page ids are clamped to [0, num_pages) on the device, so a bad table
 *     cannot cause accesses outside the pool (results are then unspecified).
 *   k_new, v_new (both NULL or both given): device bf16 [B, Hkv, d], one new
 *     token per sequence, written in place at logical row cache_seqlens[b]
 *     before attention; attention then covers cache_seqlens[b] + 1 rows.
 *     cache_seqlens itself is not modified. A position outside [0, N) is not
 *     written.
 * Attention covers L_b = cache_seqlens[b] (+ 1 with an append) rows; an L_b
 * outside [1, N] gives O = 0 and LSE = -inf for that sequence.
 * Workspace: fa_decode_workspace_bytes(B, Hq, Hkv, N, d, num_splits) with the
 *   N above. With a paged cache num_splits must be 0 (automatic) or at least
 *   ceil(N / 1024) (chunks of at most 1024 rows).
 * Errors: as fa_decode_kvcache, plus FA_ERR_INVALID_ARG for a bad page_size,
 *   max_pages_per_seq or num_pages <= 0 (paged), only one of k_new/v_new,
 *   misaligned block_table/k_new/v_new, or too few splits for a paged cache.
 */
fa_status fa_decode_kvcache_ext(const void* q, void* k_cache, void* v_cache,
                                const int32_t* cache_seqlens, const int32_t* block_table,
                                int max_pages_per_seq, int num_pages, int page_size,
                                const void* k_new, const void* v_new, void* o, float* lse,
                                void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv,
                                int cache_rows, int d, float scale, int causal, int num_splits,
                                int dtype, void* stream);

/* Message for the last non-FA_OK status returned on this thread ("" if none). */
const char* fa_last_error(void);

/* Library version string. */
const char* fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_FA_H */
