// Host-side interfaces between the C ABI (fa_api.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

namespace fa {

// Devices the library keeps per-device set-up state for (kernel attributes,
// the balanced decode's slot count, the address of the no-alloc scratch).
constexpr int kMaxDevices = 64;

// Raises a kernel's dynamic-LDS limit once per device, on the first launch
// there: one flag per kernel and device (the library's only state besides the
// thread-local error text and the per-device values named above). The kernel
// is a template argument, so every kernel instantiation has flags of its own
// (kernels that differ only in template arguments share a function-pointer
// type). Racing first calls may both set the attribute, which is harmless.
template <auto KERN>
hipError_t set_smem_once(size_t bytes) {
  static std::atomic<unsigned char> done[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < kMaxDevices && done[dev].load(std::memory_order_acquire)) return hipSuccess;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(KERN), hipFuncAttributeMaxDynamicSharedMemorySize,
                          (int)bytes);
  if (e == hipSuccess && dev >= 0 && dev < kMaxDevices) done[dev].store(1, std::memory_order_release);
  return e;
}

constexpr int kDtypeBf16 = 0;
constexpr int kDtypeF32 = 1;

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, Hq, Hkv, N, d;
  float scale;
  int causal;
  int dtype;
  hipStream_t stream;
};

// Sequence geometry for the d = 128 bf16 forward beyond dense batches.
// Varlen: sequences packed along the row axis, cu_q / cu_k are device
// [B + 1] prefix sums (rows cu_q[b] .. cu_q[b+1] - 1 of Q, O and of the LSE
// column range; likewise cu_k for K, V); LSE is laid out [Hq, total_q].
// Window: query i keeps key j iff i + off - win_left <= j <= i + off + win_right,
// off = Nk - Nq, a negative bound meaning unbounded on that side.
struct FwdSeq {
  const int* cu_q = nullptr;
  const int* cu_k = nullptr;
  int total_q = 0;
  int total_k = 0;
  int max_q = 0;
  int win_left = -1;
  int win_right = -1;
  // Block-sparse: 0/1 bytes over kBlockSparseBlock x kBlockSparseBlock tiles,
  // [ceil(N/128)] x [nbk] per (b, hq) at block_mask + (b*Hq + hq)*mask_stride
  // (stride 0: one mask shared by all).
  const uint8_t* block_mask = nullptr;
  int64_t mask_stride = 0;
  int nbk = 0;
};

constexpr int kModeVarlen = 1;
constexpr int kModeWindow = 2;
constexpr int kModeBlockSparse = 4;
constexpr int kBlockSparseBlock = 128;
constexpr int kBlockSparseMaxBlocks = 2048;  // N <= 262144

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  int B, Hq, Hkv, N, d;
  float scale;
  int causal;
  hipStream_t stream;
  int win_left = -1;   // sliding window (d = 128 only); -1 = unbounded side
  int win_right = -1;
  // Atomic backward (d = 128, no window): fp32 dQ accumulator [B, N, Hq, d];
  // stage 0 also zeroes it, stage 1 is the fused dK/dV/dQ kernel, stage 2
  // converts it to dq. NULL: the deterministic three-kernel backward.
  float* dq_acc = nullptr;
};

struct DecodeArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* seqlens;
  void* o;
  float* lse;
  int B, Hq, Hkv, N, d;  // N: rows each sequence can hold (paged: max_pages << page_shift)
  float scale;
  hipStream_t stream;
  // Paged cache: k_cache/v_cache are [num_pages, 1 << page_shift, Hkv, d] and
  // block_table [B, max_pages] maps logical page p of sequence b to a page
  // (ids are clamped to [0, num_pages)). NULL block_table: [B, N, Hkv, d].
  const int32_t* block_table = nullptr;
  int page_shift = 0;
  int max_pages = 0;
  int num_pages = 0;
  // Append: one new K/V row per sequence ([B, Hkv, d]) written at row
  // seqlens[b] before attention, which then covers seqlens[b] + 1 rows.
  const void* k_new = nullptr;
  const void* v_new = nullptr;
};

// Decode splits the cache into chunks of this many rows unless told otherwise.
constexpr int kDecodeDefaultChunk = 1024;
// Query heads that one decode workgroup serves from a single read of K/V.
constexpr int kDecodeMaxHeadsPerGroup = 4;
// Balanced decode split (automatic split count): at most this many sequences
// (their prefix sums live in LDS), and this many equal row ranges per
// resident workgroup slot of the device.
constexpr int kDecBalMaxB = 1024;
constexpr int kDecBalRounds = 1;

hipError_t launch_fwd(const FwdArgs& a);
// Varlen and/or windowed forward (bf16, d = 128). a.N is ignored; a.B is
// the number of sequences.
hipError_t launch_fwd_seq(const FwdArgs& a, const FwdSeq& seq);
// Block-sparse forward (bf16, d = 128, dense batch).
hipError_t launch_fwd_blocksparse(const FwdArgs& a, const FwdSeq& seq);

// Backward workspace: D = rowsum(dO * O) at `delta` ([B, Hq, N] float32),
// then LSE * log2(e) at delta + bwd_vec_stride(...) (same shape).
// Stage 0 computes both, stage 1 dK and dV, stage 2 dQ; launch_bwd runs all three.
inline size_t bwd_vec_stride(int B, int Hq, int N) {
  return ((size_t)B * Hq * N + 63) / 64 * 64;  // floats; keeps the second vector 256-byte aligned
}
// Atomic backward workspace: the two vectors above, then the fp32 dQ
// accumulator (256-byte aligned).
inline size_t bwd_atomic_acc_offset(int B, int Hq, int N) { return 2 * bwd_vec_stride(B, Hq, N) * sizeof(float); }
inline size_t bwd_atomic_ws_bytes(int B, int Hq, int N, int d) {
  return bwd_atomic_acc_offset(B, Hq, N) + (size_t)B * N * Hq * d * sizeof(float);
}
hipError_t launch_bwd_stage(const BwdArgs& a, float* delta, int stage);
hipError_t launch_bwd(const BwdArgs& a, float* delta);

int decode_heads_per_group(int Hq, int Hkv);
void decode_split_plan(int N, int num_splits, int* chunk, int* nsplit);
hipError_t launch_decode(const DecodeArgs& a, float* part_o, float* part_lse, int chunk, int nsplit);
// Balanced split: number of row ranges P per kv-head block for these sizes on
// the current device, or 0 when the chunked split is used instead (explicit
// num_splits, B > kDecBalMaxB, or Hkv not a multiple of 512 / d).
int decode_balanced_ranges(int B, int Hq, int Hkv, int d, int num_splits);
// Workspace of the balanced split: prefix sums (B + 1 int64), then LSE and O
// partials for P + B - 1 slots.
struct DecodeBalLayout {
  size_t cum_bytes, lse_bytes, o_bytes;
};
DecodeBalLayout decode_bal_layout(int B, int Hq, int d, int P);
hipError_t launch_decode_balanced(const DecodeArgs& a, void* workspace, int P);

// The no-allocation decode entry point keeps its partials in a file-scope
// device array of this many bytes (one copy per device, held until the
// process ends).
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
// Device address of that array on the current device, looked up with
// hipGetSymbolAddress on the first call on each device; nullptr (and *err
// set) when the lookup fails.
void* decode_noalloc_scratch(hipError_t* err);

}  // namespace fa
