// C ABI of the gfx950 attention library: argument validation, workspace
// layout and kernel launches. Every check runs before any HIP call, so an
// invalid call launches nothing. Declarations and argument documentation are
// in include/fa.h.
#include "../../include/fa.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "fa_internal.h"

namespace {

thread_local char g_err[512] = "";

fa_status fail(fa_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

fa_status ok() {
  g_err[0] = '\0';
  return FA_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

fa_status check_sizes(const char* fn, int B, int Hq, int Hkv, int N, int d, float scale) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || N <= 0)
    return fail(FA_ERR_INVALID_ARG, "%s: sizes must be positive (B=%d Hq=%d Hkv=%d N=%d)", fn, B, Hq, Hkv, N);
  if (Hq % Hkv != 0)
    return fail(FA_ERR_INVALID_ARG, "%s: Hq=%d is not a multiple of Hkv=%d", fn, Hq, Hkv);
  if (!std::isfinite(scale) || !(scale > 0.f))
    return fail(FA_ERR_INVALID_ARG, "%s: scale must be finite and positive", fn);
  if (d != 64 && d != 128) return fail(FA_ERR_UNSUPPORTED, "%s: head dim d=%d is not 64 or 128", fn, d);
  // Element offsets are 64-bit, but one tensor must stay below 2^62 bytes.
  const double elems = (double)B * N * Hq * d;
  if (elems > 4.0e18) return fail(FA_ERR_INVALID_ARG, "%s: tensor too large", fn);
  return FA_OK;
}

fa_status check_ptr(const char* fn, const char* name, const void* p, size_t align) {
  if (!p) return fail(FA_ERR_INVALID_ARG, "%s: %s is NULL", fn, name);
  if (!aligned(p, align)) return fail(FA_ERR_INVALID_ARG, "%s: %s is not %zu-byte aligned", fn, name, align);
  return FA_OK;
}

#define FA_TRY(expr)                 \
  do {                               \
    fa_status _st = (expr);          \
    if (_st != FA_OK) return _st;    \
  } while (0)

fa_status hip_status(const char* fn, hipError_t e) {
  if (e != hipSuccess) return fail(FA_ERR_HIP, "%s: %s", fn, hipGetErrorString(e));
  return ok();
}

// D and LSE * log2(e), each [B, Hq, N] float32.
size_t bwd_ws_bytes(int B, int Hq, int N) { return 2 * fa::bwd_vec_stride(B, Hq, N) * sizeof(float); }

void decode_ws_layout(int B, int Hq, int N, int d, int num_splits, int* chunk, int* nsplit, size_t* o_bytes,
                      size_t* lse_bytes) {
  fa::decode_split_plan(N, num_splits, chunk, nsplit);
  *o_bytes = round_up((size_t)B * Hq * (size_t)(*nsplit) * d * sizeof(float), 256);
  *lse_bytes = round_up((size_t)B * Hq * (size_t)(*nsplit) * sizeof(float), 256);
}

// How a decode call splits the cache: balanced row ranges (P > 0, automatic
// split count on a device where they apply) or fixed chunks.
struct DecodePlan {
  int P = 0;
  int chunk = 0, nsplit = 0;
  size_t o_bytes = 0, lse_bytes = 0;
  size_t bytes() const { return o_bytes + lse_bytes; }
};

DecodePlan decode_plan(int B, int Hq, int Hkv, int N, int d, int num_splits) {
  DecodePlan p;
  p.P = fa::decode_balanced_ranges(B, Hq, Hkv, d, num_splits);
  if (p.P > 0) {
    const fa::DecodeBalLayout l = fa::decode_bal_layout(B, Hq, d, p.P);
    p.lse_bytes = l.cum_bytes + l.lse_bytes;
    p.o_bytes = l.o_bytes;
  } else {
    decode_ws_layout(B, Hq, N, d, num_splits, &p.chunk, &p.nsplit, &p.o_bytes, &p.lse_bytes);
  }
  return p;
}

fa_status bwd_common(const char* fn, int stage, const void* q, const void* k, const void* v, const void* o,
                     const void* dout, const float* lse, void* dq, void* dk, void* dv, void* workspace,
                     size_t workspace_bytes, int B, int Hq, int Hkv, int N, int d, float scale, int causal,
                     int dtype, void* stream, int window_left = -1, int window_right = -1, bool atomic = false) {
  FA_TRY(check_sizes(fn, B, Hq, Hkv, N, d, scale));
  if (dtype != FA_BF16) return fail(FA_ERR_UNSUPPORTED, "%s: only bf16 is implemented (dtype %d)", fn, dtype);
  if (atomic && d != 128) return fail(FA_ERR_UNSUPPORTED, "%s: the atomic backward needs d = 128 (got %d)", fn, d);
  if (window_left < -1 || window_right < -1)
    return fail(FA_ERR_INVALID_ARG, "%s: window (%d, %d): each side must be >= -1", fn, window_left, window_right);
  const bool all = stage < 0;
  if (all || stage == 0) {
    FA_TRY(check_ptr(fn, "o", o, 16));
    FA_TRY(check_ptr(fn, "dout", dout, 16));
    FA_TRY(check_ptr(fn, "lse", lse, 4));
  }
  if (all || stage >= 1) {
    FA_TRY(check_ptr(fn, "q", q, 16));
    FA_TRY(check_ptr(fn, "k", k, 16));
    FA_TRY(check_ptr(fn, "v", v, 16));
    FA_TRY(check_ptr(fn, "dout", dout, 16));
    FA_TRY(check_ptr(fn, "lse", lse, 4));
  }
  if (all || stage == 1) {
    FA_TRY(check_ptr(fn, "dk", dk, 16));
    FA_TRY(check_ptr(fn, "dv", dv, 16));
  }
  if (all || stage == 2) FA_TRY(check_ptr(fn, "dq", dq, 16));
  const size_t need = atomic ? fa::bwd_atomic_ws_bytes(B, Hq, N, d) : bwd_ws_bytes(B, Hq, N);
  if (!workspace || workspace_bytes < need)
    return fail(FA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned(workspace, 256)) return fail(FA_ERR_INVALID_ARG, "%s: workspace is not 256-byte aligned", fn);
  fa::BwdArgs a{q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, N, d, scale, causal ? 1 : 0,
                reinterpret_cast<hipStream_t>(stream), window_left, window_right};
  if (atomic) a.dq_acc = reinterpret_cast<float*>(static_cast<char*>(workspace) + fa::bwd_atomic_acc_offset(B, Hq, N));
  float* delta = static_cast<float*>(workspace);
  return hip_status(fn, all ? fa::launch_bwd(a, delta) : fa::launch_bwd_stage(a, delta, stage));
}

// Decode without append or paging. With use_scratch the partials go to the
// library's per-device scratch array instead of the caller's workspace.
fa_status decode_common(const char* fn, const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* cache_seqlens, void* o, float* lse, void* workspace, size_t workspace_bytes,
                        bool use_scratch, int B, int Hq, int Hkv, int N, int d, float scale, int num_splits,
                        int dtype, void* stream) {
  FA_TRY(check_sizes(fn, B, Hq, Hkv, N, d, scale));
  if (dtype != FA_BF16) return fail(FA_ERR_UNSUPPORTED, "%s: only bf16 is implemented (dtype %d)", fn, dtype);
  if (num_splits < 0) return fail(FA_ERR_INVALID_ARG, "%s: num_splits must be >= 0", fn);
  FA_TRY(check_ptr(fn, "q", q, 16));
  FA_TRY(check_ptr(fn, "k_cache", k_cache, 16));
  FA_TRY(check_ptr(fn, "v_cache", v_cache, 16));
  FA_TRY(check_ptr(fn, "cache_seqlens", cache_seqlens, 4));
  FA_TRY(check_ptr(fn, "o", o, 16));
  if (lse && !aligned(lse, 4)) return fail(FA_ERR_INVALID_ARG, "%s: lse is not 4-byte aligned", fn);
  const DecodePlan plan = decode_plan(B, Hq, Hkv, N, d, num_splits);
  if (use_scratch) {
    if (plan.bytes() > fa::kNoAllocScratchBytes)
      return fail(FA_ERR_WORKSPACE, "%s: these sizes need %zu bytes of partials, more than the %zu-byte scratch "
                  "array; use fa_decode_kvcache with a workspace", fn, plan.bytes(), fa::kNoAllocScratchBytes);
    hipError_t e = hipSuccess;
    workspace = fa::decode_noalloc_scratch(&e);
    if (!workspace) return hip_status(fn, e);
    workspace_bytes = fa::kNoAllocScratchBytes;
  }
  if (!workspace || workspace_bytes < plan.bytes())
    return fail(FA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, plan.bytes(),
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned(workspace, 256)) return fail(FA_ERR_INVALID_ARG, "%s: workspace is not 256-byte aligned", fn);
  fa::DecodeArgs a{q, k_cache, v_cache, cache_seqlens, o, lse, B, Hq, Hkv, N, d, scale,
                   reinterpret_cast<hipStream_t>(stream)};
  if (plan.P > 0) return hip_status(fn, fa::launch_decode_balanced(a, workspace, plan.P));
  float* part_o = static_cast<float*>(workspace);
  float* part_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) + plan.o_bytes);
  return hip_status(fn, fa::launch_decode(a, part_o, part_lse, plan.chunk, plan.nsplit));
}

}  // namespace

extern "C" {

const char* fa_last_error(void) { return g_err; }

const char* fa_version(void) { return "fa_mi355x 0.1 (gfx950)"; }

fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv, int N,
                 int d, float scale, int causal, int dtype, void* stream) {
  static const char* fn = "fa_fwd";
  FA_TRY(check_sizes(fn, B, Hq, Hkv, N, d, scale));
  if (dtype != FA_BF16 && dtype != FA_FP32) return fail(FA_ERR_UNSUPPORTED, "%s: dtype %d not supported", fn, dtype);
  FA_TRY(check_ptr(fn, "q", q, 16));
  FA_TRY(check_ptr(fn, "k", k, 16));
  FA_TRY(check_ptr(fn, "v", v, 16));
  FA_TRY(check_ptr(fn, "o", o, 16));
  FA_TRY(check_ptr(fn, "lse", lse, 4));
  fa::FwdArgs a{q, k, v, o, lse, B, Hq, Hkv, N, d, scale, causal ? 1 : 0, dtype,
                reinterpret_cast<hipStream_t>(stream)};
  return hip_status(fn, fa::launch_fwd(a));
}

fa_status fa_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
                        int N, int d, float scale, int causal, int window_left, int window_right, int dtype,
                        void* stream) {
  static const char* fn = "fa_fwd_window";
  FA_TRY(check_sizes(fn, B, Hq, Hkv, N, d, scale));
  if (window_left < -1 || window_right < -1)
    return fail(FA_ERR_INVALID_ARG, "%s: window (%d, %d): each side must be >= -1", fn, window_left, window_right);
  if (window_left < 0 && window_right < 0) return fa_fwd(q, k, v, o, lse, B, Hq, Hkv, N, d, scale, causal, dtype, stream);
  if (dtype != FA_BF16) return fail(FA_ERR_UNSUPPORTED, "%s: only bf16 supports a window", fn);
  FA_TRY(check_ptr(fn, "q", q, 16));
  FA_TRY(check_ptr(fn, "k", k, 16));
  FA_TRY(check_ptr(fn, "v", v, 16));
  FA_TRY(check_ptr(fn, "o", o, 16));
  FA_TRY(check_ptr(fn, "lse", lse, 4));
  fa::FwdArgs a{q, k, v, o, lse, B, Hq, Hkv, N, d, scale, causal ? 1 : 0, dtype,
                reinterpret_cast<hipStream_t>(stream)};
  fa::FwdSeq seq;
  seq.win_left = window_left;
  seq.win_right = window_right;
  return hip_status(fn, fa::launch_fwd_seq(a, seq));
}

fa_status fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                        const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int B, int max_seqlen_q,
                        int total_q, int total_k, int Hq, int Hkv, int d, float scale, int causal, int window_left,
                        int window_right, int dtype, void* stream) {
  static const char* fn = "fa_fwd_varlen";
  FA_TRY(check_sizes(fn, B, Hq, Hkv, max_seqlen_q, d, scale));
  if (total_q <= 0 || total_k < 0)
    return fail(FA_ERR_INVALID_ARG, "%s: total_q %d must be > 0 and total_k %d >= 0", fn, total_q, total_k);
  if (window_left < -1 || window_right < -1)
    return fail(FA_ERR_INVALID_ARG, "%s: window (%d, %d): each side must be >= -1", fn, window_left, window_right);
  if (dtype != FA_BF16) return fail(FA_ERR_UNSUPPORTED, "%s: only bf16 is supported", fn);
  FA_TRY(check_ptr(fn, "q", q, 16));
  FA_TRY(check_ptr(fn, "k", k, 16));
  FA_TRY(check_ptr(fn, "v", v, 16));
  FA_TRY(check_ptr(fn, "o", o, 16));
  FA_TRY(check_ptr(fn, "lse", lse, 4));
  FA_TRY(check_ptr(fn, "cu_seqlens_q", cu_seqlens_q, 4));
  FA_TRY(check_ptr(fn, "cu_seqlens_k", cu_seqlens_k, 4));
  if ((int64_t)(max_seqlen_q + 127) / 128 * B * Hq > 0x7fffffff)
    return fail(FA_ERR_INVALID_ARG, "%s: launch grid too large", fn);
  fa::FwdArgs a{q, k, v, o, lse, B, Hq, Hkv, max_seqlen_q, d, scale, causal ? 1 : 0, dtype,
                reinterpret_cast<hipStream_t>(stream)};
  fa::FwdSeq seq;
  seq.cu_q = cu_seqlens_q;
  seq.cu_k = cu_seqlens_k;
  seq.total_q = total_q;
  seq.total_k = total_k;
  seq.max_q = max_seqlen_q;
  seq.win_left = window_left;
  seq.win_right = window_right;
  return hip_status(fn, fa::launch_fwd_seq(a, seq));
}

fa_status fa_fwd_blocksparse(const void* q, const void* k, const void* v, void* o, float* lse,
                             const uint8_t* block_mask, long long mask_head_stride, int B, int Hq, int Hkv, int N,
                             int d, float scale, int causal, int dtype, void* stream) {
  static const char* fn = "fa_fwd_blocksparse";
  FA_TRY(check_sizes(fn, B, Hq, Hkv, N, d, scale));
  if (dtype != FA_BF16) return fail(FA_ERR_UNSUPPORTED, "%s: only bf16 is supported", fn);
  const int nb = (N + fa::kBlockSparseBlock - 1) / fa::kBlockSparseBlock;
  if (nb > fa::kBlockSparseMaxBlocks)
    return fail(FA_ERR_UNSUPPORTED, "%s: N = %d exceeds %d", fn, N, fa::kBlockSparseMaxBlocks * fa::kBlockSparseBlock);
  if (mask_head_stride != 0 && mask_head_stride < (long long)nb * nb)
    return fail(FA_ERR_INVALID_ARG, "%s: mask_head_stride %lld is neither 0 nor >= %d", fn, mask_head_stride, nb * nb);
  FA_TRY(check_ptr(fn, "q", q, 16));
  FA_TRY(check_ptr(fn, "k", k, 16));
  FA_TRY(check_ptr(fn, "v", v, 16));
  FA_TRY(check_ptr(fn, "o", o, 16));
  FA_TRY(check_ptr(fn, "lse", lse, 4));
  FA_TRY(check_ptr(fn, "block_mask", block_mask, 1));
  fa::FwdArgs a{q, k, v, o, lse, B, Hq, Hkv, N, d, scale, causal ? 1 : 0, dtype,
                reinterpret_cast<hipStream_t>(stream)};
  fa::FwdSeq seq;
  seq.block_mask = block_mask;
  seq.mask_stride = mask_head_stride;
  seq.nbk = nb;
  return hip_status(fn, fa::launch_fwd_blocksparse(a, seq));
}

size_t fa_bwd_workspace_bytes(int B, int Hq, int Hkv, int N, int d) {
  (void)Hkv;
  (void)d;
  if (B <= 0 || Hq <= 0 || N <= 0) return 0;
  return bwd_ws_bytes(B, Hq, N);
}

fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                 void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv,
                 int N, int d, float scale, int causal, int dtype, void* stream) {
  return bwd_common("fa_bwd", -1, q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, Hq, Hkv, N, d,
                    scale, causal, dtype, stream);
}

fa_status fa_bwd_stage(int stage, const void* q, const void* k, const void* v, const void* o, const void* dout,
                       const float* lse, void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                       int B, int Hq, int Hkv, int N, int d, float scale, int causal, int dtype, void* stream) {
  if (stage < 0 || stage > 2) return fail(FA_ERR_INVALID_ARG, "fa_bwd_stage: stage %d is not 0, 1 or 2", stage);
  return bwd_common("fa_bwd_stage", stage, q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, Hq,
                    Hkv, N, d, scale, causal, dtype, stream);
}

size_t fa_bwd_atomic_workspace_bytes(int B, int Hq, int Hkv, int N, int d) {
  (void)Hkv;
  if (B <= 0 || Hq <= 0 || N <= 0 || d <= 0) return 0;
  return fa::bwd_atomic_ws_bytes(B, Hq, N, d);
}

fa_status fa_bwd_atomic(const void* q, const void* k, const void* v, const void* o, const void* dout,
                        const float* lse, void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                        int B, int Hq, int Hkv, int N, int d, float scale, int causal, int dtype, void* stream) {
  return bwd_common("fa_bwd_atomic", -1, q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, Hq, Hkv,
                    N, d, scale, causal, dtype, stream, -1, -1, true);
}

fa_status fa_bwd_atomic_stage(int stage, const void* q, const void* k, const void* v, const void* o,
                              const void* dout, const float* lse, void* dq, void* dk, void* dv, void* workspace,
                              size_t workspace_bytes, int B, int Hq, int Hkv, int N, int d, float scale, int causal,
                              int dtype, void* stream) {
  if (stage < 0 || stage > 2)
    return fail(FA_ERR_INVALID_ARG, "fa_bwd_atomic_stage: stage %d is not 0, 1 or 2", stage);
  return bwd_common("fa_bwd_atomic_stage", stage, q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B,
                    Hq, Hkv, N, d, scale, causal, dtype, stream, -1, -1, true);
}

fa_status fa_bwd_window(const void* q, const void* k, const void* v, const void* o, const void* dout,
                        const float* lse, void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                        int B, int Hq, int Hkv, int N, int d, float scale, int causal, int window_left,
                        int window_right, int dtype, void* stream) {
  return bwd_common("fa_bwd_window", -1, q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, Hq, Hkv,
                    N, d, scale, causal, dtype, stream, window_left, window_right);
}

size_t fa_decode_workspace_bytes(int B, int Hq, int Hkv, int N, int d, int num_splits) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || N <= 0 || d <= 0 || num_splits < 0) return 0;
  return decode_plan(B, Hq, Hkv, N, d, num_splits).bytes();
}

fa_status fa_decode_kvcache(const void* q, const void* k_cache, const void* v_cache, const int32_t* cache_seqlens,
                            void* o, float* lse, void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv,
                            int N, int d, float scale, int causal, int num_splits, int dtype, void* stream) {
  return decode_common("fa_decode_kvcache", q, k_cache, v_cache, cache_seqlens, o, lse, workspace, workspace_bytes,
                       false, B, Hq, Hkv, N, d, scale, num_splits, dtype, stream);
}

fa_status fa_decode_kvcache_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                    const int32_t* cache_seqlens, void* o, float* lse, int B, int Hq, int Hkv, int N,
                                    int d, float scale, int causal, int num_splits, int dtype, void* stream) {
  (void)causal;  // one query aligned to the bottom-right corner sees every cached key
  return decode_common("fa_decode_kvcache_noalloc", q, k_cache, v_cache, cache_seqlens, o, lse, nullptr, 0, true,
                       B, Hq, Hkv, N, d, scale, num_splits, dtype, stream);
}

fa_status fa_decode_kvcache_ext(const void* q, void* k_cache, void* v_cache, const int32_t* cache_seqlens,
                                const int32_t* block_table, int max_pages_per_seq, int num_pages, int page_size,
                                const void* k_new, const void* v_new, void* o, float* lse, void* workspace,
                                size_t workspace_bytes, int B, int Hq, int Hkv, int cache_rows, int d, float scale,
                                int causal, int num_splits, int dtype, void* stream) {
  static const char* fn = "fa_decode_kvcache_ext";
  (void)causal;  // one query aligned to the bottom-right corner sees every cached key
  int N = cache_rows;
  int shift = 0;
  if (block_table) {
    if (page_size < 16 || (page_size & (page_size - 1)) != 0)
      return fail(FA_ERR_INVALID_ARG, "%s: page_size %d must be a power of two >= 16", fn, page_size);
    if (max_pages_per_seq <= 0 || num_pages <= 0)
      return fail(FA_ERR_INVALID_ARG, "%s: max_pages_per_seq %d and num_pages %d must be > 0", fn,
                  max_pages_per_seq, num_pages);
    if ((int64_t)max_pages_per_seq * page_size > 0x7fffffff)
      return fail(FA_ERR_INVALID_ARG, "%s: max_pages_per_seq * page_size overflows", fn);
    N = max_pages_per_seq * page_size;
    while ((1 << shift) < page_size) ++shift;
  }
  FA_TRY(check_sizes(fn, B, Hq, Hkv, N, d, scale));
  if (dtype != FA_BF16) return fail(FA_ERR_UNSUPPORTED, "%s: only bf16 is implemented (dtype %d)", fn, dtype);
  if (num_splits < 0) return fail(FA_ERR_INVALID_ARG, "%s: num_splits must be >= 0", fn);
  if ((k_new == nullptr) != (v_new == nullptr))
    return fail(FA_ERR_INVALID_ARG, "%s: k_new and v_new must be given together", fn);
  FA_TRY(check_ptr(fn, "q", q, 16));
  FA_TRY(check_ptr(fn, "k_cache", k_cache, 16));
  FA_TRY(check_ptr(fn, "v_cache", v_cache, 16));
  FA_TRY(check_ptr(fn, "cache_seqlens", cache_seqlens, 4));
  FA_TRY(check_ptr(fn, "o", o, 16));
  if (block_table && !aligned(block_table, 4)) return fail(FA_ERR_INVALID_ARG, "%s: block_table misaligned", fn);
  if (k_new) {
    FA_TRY(check_ptr(fn, "k_new", k_new, 16));
    FA_TRY(check_ptr(fn, "v_new", v_new, 16));
  }
  if (lse && !aligned(lse, 4)) return fail(FA_ERR_INVALID_ARG, "%s: lse is not 4-byte aligned", fn);
  const DecodePlan plan = decode_plan(B, Hq, Hkv, N, d, num_splits);
  if (block_table && plan.P == 0 && plan.chunk > fa::kDecodeDefaultChunk)
    return fail(FA_ERR_INVALID_ARG, "%s: with a paged cache num_splits must be 0 or >= %d", fn,
                (N + fa::kDecodeDefaultChunk - 1) / fa::kDecodeDefaultChunk);
  if (!workspace || workspace_bytes < plan.bytes())
    return fail(FA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, plan.bytes(),
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned(workspace, 256)) return fail(FA_ERR_INVALID_ARG, "%s: workspace is not 256-byte aligned", fn);
  float* part_o = static_cast<float*>(workspace);
  float* part_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) + plan.o_bytes);
  fa::DecodeArgs a{q, k_cache, v_cache, cache_seqlens, o, lse, B, Hq, Hkv, N, d, scale,
                   reinterpret_cast<hipStream_t>(stream)};
  a.block_table = block_table;
  a.page_shift = shift;
  a.max_pages = max_pages_per_seq;
  a.num_pages = num_pages;
  a.k_new = k_new;
  a.v_new = v_new;
  if (plan.P > 0) return hip_status(fn, fa::launch_decode_balanced(a, workspace, plan.P));
  return hip_status(fn, fa::launch_decode(a, part_o, part_lse, plan.chunk, plan.nsplit));
}

}  // extern "C"
