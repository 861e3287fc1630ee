// Host-side interfaces between the C ABI (fa_api.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

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
};

struct DecodeArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* seqlens;
  void* o;
  float* lse;
  int B, Hq, Hkv, N, d;
  float scale;
  hipStream_t stream;
};

// Decode splits the cache into chunks of this many rows unless told otherwise.
constexpr int kDecodeDefaultChunk = 512;
// Query heads that one decode workgroup serves from a single read of K/V.
constexpr int kDecodeMaxHeadsPerGroup = 4;

hipError_t launch_fwd(const FwdArgs& a);

// Backward workspace: D = rowsum(dO * O) at `delta` ([B, Hq, N] float32),
// then LSE * log2(e) at delta + bwd_vec_stride(...) (same shape).
// Stage 0 computes both, stage 1 dK and dV, stage 2 dQ; launch_bwd runs all three.
inline size_t bwd_vec_stride(int B, int Hq, int N) {
  return ((size_t)B * Hq * N + 63) / 64 * 64;  // floats; keeps the second vector 256-byte aligned
}
hipError_t launch_bwd_stage(const BwdArgs& a, float* delta, int stage);
hipError_t launch_bwd(const BwdArgs& a, float* delta);

int decode_heads_per_group(int Hq, int Hkv);
void decode_split_plan(int N, int num_splits, int* chunk, int* nsplit);
hipError_t launch_decode(const DecodeArgs& a, float* part_o, float* part_lse, int chunk, int nsplit);

}  // namespace fa
