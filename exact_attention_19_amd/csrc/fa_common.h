// Device helpers shared by the gfx950 attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

// 32x32x16 bf16 MFMA (gfx950): D[32x32] += A[32x16] * B[16x32].
// Lane l supplies A row (l % 32), k = 8*(l/32) .. +7 and B column (l % 32),
// k = 8*(l/32) .. +7; it receives D column (l % 32), rows
// 8*j + 4*(l/32) + i in element 4*j + i.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two floats -> packed bf16x2 (round to nearest even, v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 r;
  r[0] = (__bf16)lo;
  r[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, r);
}

// Low 16 bits of a and of b into one dword: (a.lo, b.lo).
__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
// High 16 bits of a and of b into one dword: (a.hi, b.hi).
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

template <typename T>
__device__ __forceinline__ T max3(T a, T b, T c) { return fmaxf(fmaxf(a, b), c); }

// Value of lane (l ^ 32): exchange between the two halves of the wave.
// Max and sum of x over the lane pair (l, l ^ 32), the same value in both
// lanes. v_permlane32_swap with x as both operands hands every lane the
// lower-half value in the first result and the upper-half value in the
// second, in the VALU (no LDS round trip as with a shuffle).
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Sum over LPT consecutive lanes (LPT = 8 or 16); every lane of the group
// receives the same total (each pairing adds two equal-order partial sums).
template <int LPT>
__device__ __forceinline__ float row_group_sum(float x) {
  x += dpp_f<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp_f<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp_f<0x141>(x);  // row_half_mirror: pairs the two quads of each 8 lanes
  if (LPT == 16) x += dpp_f<0x140>(x);  // row_mirror: pairs the two halves of 16 lanes
  return x;
}

__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t w) { return __builtin_bit_cast(bf16x2, w); }

// 8-element bf16 dot product accumulated in fp32 (v_dot2_f32_bf16). Each
// vector element is copied into a scalar before the bit cast: casting the
// indexed element in place made hipcc (ROCm 7.2) load element 0 only.
__device__ __forceinline__ float dot8_bf16(const u32x4& a, const u32x4& b, float acc) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t x = a[w], y = b[w];
    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(x), as_bf16x2(y), acc, false);
  }
  return acc;
}

// Transposed 64-wide tiles in LDS (V^T in the forward, Q^T / dO^T / K^T in
// the backward): D rows of 64 bf16 (128 bytes) each, holding one head-dim
// index per row and 64 sequence positions along the row.
//
// Position of sequence group kg (4 consecutive positions, kg = 0..15) inside
// the row. Within each group of 16 positions, groups of 4 are stored in the
// order 0, 2, 1, 3: the order in which a 32x32 MFMA accumulator hands them to
// one 16-deep MFMA step (lanes 0-31 hold positions 0-3 and 8-11, lanes 32-63
// hold 4-7 and 12-15). A lane reading the 16 bytes at logical offset
// 16*step + 8*(l/32) then gets exactly the 8 positions its accumulator half
// holds, so the permutation cancels in the product.
__device__ __forceinline__ int tr_pos_of_group4(int kg) {
  const int in16 = kg & 3;
  const int perm = (in16 == 1) ? 2 : (in16 == 2 ? 1 : in16);
  return (kg >> 2) * 16 + perm * 4;
}

// XOR swizzle of the eight 16-byte units of a transposed row, so that both
// the transposing writes (rows 8 apart) and the MFMA operand reads
// (consecutive rows) spread over the LDS banks.
__device__ __forceinline__ int tr_swz(int d) { return (d & 7) ^ ((d >> 3) & 7); }

// Write the 4 (positions) x 8 (head dims) block held in `rows` (four 16-byte
// rows, one per position) transposed into a 64-wide tile `tr`: 8 rows
// (dims 8*dc .. 8*dc+7) of 4 positions each.
__device__ __forceinline__ void store_transposed_4x8(__bf16* tr, int kg, int dc, const u32x4 (&rows)[4]) {
  const int pos = tr_pos_of_group4(kg);
  const int unit = pos >> 3, half = (pos >> 2) & 1;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int d = dc * 8 + j;
    const int w = j >> 1;
    const uint32_t a0 = rows[0][w], a1 = rows[1][w], a2 = rows[2][w], a3 = rows[3][w];
    u32x2 out;
    if (j & 1) {
      out[0] = (a0 >> 16) | (a1 & 0xffff0000u);
      out[1] = (a2 >> 16) | (a3 & 0xffff0000u);
    } else {
      out[0] = (a0 & 0xffffu) | (a1 << 16);
      out[1] = (a2 & 0xffffu) | (a3 << 16);
    }
    const int u = unit ^ tr_swz(d);
    *reinterpret_cast<u32x2*>(tr + d * 64 + u * 8 + half * 4) = out;
  }
}

// MFMA A operand from a transposed tile: row d, logical 16-byte unit
// 2*step + half.
__device__ __forceinline__ bf16x8 load_tr_operand(const __bf16* tr, int d, int step, int half) {
  const int u = (2 * step + half) ^ tr_swz(d);
  return *reinterpret_cast<const bf16x8*>(tr + d * 64 + u * 8);
}

// Workgroup order for a launch of nh x T workgroups (nh heads, a multiple of
// 8, each with T tiles; rank 0 is a head's heaviest tile). Workgroups are
// dealt round-robin to the 8 XCDs, so workgroup bid runs on XCD bid % 8; that
// XCD takes heads xcd, xcd + 8, ..., so its L2 only ever holds their tiles.
// It visits them in groups of `group` heads, rank-major inside a group (the
// heaviest tile of every head in the group first), so that the heaviest tile
// of the last head is not dispatched when little other work is left.
// group = 1 is plain head-major order.
__device__ __forceinline__ void xcd_order(int bid, int nh, int T, int group, int& h, int& rank) {
  const int xcd = bid & 7, slot = bid >> 3;
  const int grp = slot / (group * T);
  const int g = min(group, (nh >> 3) - grp * group);  // heads in this group
  const int w = slot - grp * group * T;
  rank = w / g;
  h = (grp * group + (w - rank * g)) * 8 + xcd;
}

// Heads per group in xcd_order, per kernel.
constexpr int kFwdHeadGroup = 4;
constexpr int kDkdvHeadGroup = 4;
constexpr int kDqHeadGroup = 8;

// ---------------------------------------------------------------------------
// Row-major 64 x 128 bf16 tiles in LDS (256 bytes per row), filled straight
// from global memory with global_load_lds_dwordx4: one wave instruction
// writes 1 KB (4 rows) contiguously, lane i landing at byte 16 i. The 16-byte
// units of row r are stored XOR-permuted by tile_swz(r), which is free of
// LDS bank conflicts both for 16-byte MFMA operand reads down 16 consecutive
// rows and for ds_read_b64_tr_b16 transposed reads of 4-row x 32-byte blocks
// (measured on gfx950).
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((ext_vector_type(4))) short i16x4;

__device__ __forceinline__ int tile_swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// The same tiles for d = 64: 128-byte rows of eight 16-byte units. With
// m = r / 2, unit u of row r lands at u ^ (4 (m & 1) + (m / 2) % 4). Over
// eight consecutive rows of one parity this is a permutation of 0..7, so
// 16-byte operand reads down 16 consecutive rows meet 16 distinct bank
// groups (odd rows sit in the other half of the 256-byte bank line); over
// rows c, c + 2, c + 4, c + 6 its bit 2 alternates, so a transposed read of
// a 4-row block uses both halves of the row evenly.
__device__ __forceinline__ int tile_swz8(int r) { return (((r >> 1) & 1) << 2) | ((r >> 2) & 3); }
template <int D>
__device__ __forceinline__ int row_swz(int r) {
  static_assert(D == 64 || D == 128, "d = 64 or 128");
  return D == 128 ? tile_swz(r) : tile_swz8(r);
}

// Scalar (wave-uniform) copy of a value the compiler cannot prove uniform,
// e.g. the result of an integer division of uniform operands.
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ const unsigned char* uniform(const unsigned char* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const unsigned char*>(((uint64_t)hi << 32) | lo);
}

// Buffer resource over the byte range [base, base + bytes): loads at offsets
// past `bytes` return zero. (Raw buffer, stride 0, 32-bit data format.)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Per-lane byte offset of a tile DMA chunk (constant for every chunk the
// wave issues): row lane/16 of the chunk, 16-byte unit (lane%16) XOR the
// row's swizzle. Chunks issued by one wave are c = first + STEP*i with STEP a
// multiple of 4, so (4c + row) % 16 is the same for all of them.
__device__ __forceinline__ uint32_t dma_lane_offset(int lane, int first, uint32_t stride_bytes) {
  const int lr = lane >> 4;
  return (uint32_t)lr * stride_bytes + 16u * (uint32_t)((lane & 15) ^ tile_swz(4 * first + lr));
}

// The same for tiles of D-dim rows: a 1 KB chunk holds 1024 / (2 D) rows
// (4 at d = 128, 8 at d = 64); for d = 64 the chunks a wave issues,
// c = first + 4 i, share the swizzle phase of rows 8 c + (0..7).
template <int D>
__device__ __forceinline__ uint32_t dma_lane_offset_d(int lane, int first, uint32_t stride_bytes) {
  if constexpr (D == 128) return dma_lane_offset(lane, first, stride_bytes);
  const int lr = lane >> 3;
  return (uint32_t)lr * stride_bytes + 16u * (uint32_t)((lane & 7) ^ tile_swz8(8 * first + lr));
}

// Tile DMA: rows [0, 64) below `tile_base` (row stride `stride_bytes`) go
// into a swizzled LDS tile; rows at or past `nrows` arrive as zeros. The
// calling wave issues chunks c = first + step*i (4 rows each, i < nchunk,
// step a multiple of 4, so every chunk of a lane has the same swizzle phase:
// lane_off, from dma_lane_offset, is the lane's offset inside its chunk, and
// chunk c starts 4*c*stride_bytes into the tile). One buffer
// resource spans the tile's valid rows, so a tile costs a few scalar
// instructions, one add per chunk and one load per chunk. tile_base and
// nrows must be wave-uniform; first, step and nchunk are compile-time
// constants at every call site (the loop unrolls after inlining).
__device__ __forceinline__ void dma_rows64(const unsigned char* tile_base, uint32_t stride_bytes, int nrows,
                                           unsigned char* lds_tile, int first, int step, int nchunk,
                                           uint32_t lane_off) {
  const uint32_t rows = (uint32_t)uniform(min(max(nrows, 0), 64));
  const __amdgpu_buffer_rsrc_t r = make_rsrc(uniform(tile_base), rows * stride_bytes);
  const uint32_t chunk_stride = (uint32_t)(4 * step) * stride_bytes;
  const uint32_t first_off = lane_off + (uint32_t)(4 * first) * stride_bytes;
#pragma unroll
  for (int i = 0; i < nchunk; ++i) {
    const int c = first + step * i;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(lds_tile + c * 1024), 16, first_off + i * chunk_stride,
                                             0, 0, 0);
  }
}

// dma_rows64 for tiles of D-dim rows (1024 / (2 D) rows per chunk).
template <int D>
__device__ __forceinline__ void dma_rows64_d(const unsigned char* tile_base, uint32_t stride_bytes, int nrows,
                                             unsigned char* lds_tile, int first, int step, int nchunk,
                                             uint32_t lane_off) {
  constexpr int RPC = 1024 / (2 * D);
  const uint32_t rows = (uint32_t)uniform(min(max(nrows, 0), 64));
  const __amdgpu_buffer_rsrc_t r = make_rsrc(uniform(tile_base), rows * stride_bytes);
  const uint32_t chunk_stride = (uint32_t)(RPC * step) * stride_bytes;
  const uint32_t first_off = lane_off + (uint32_t)(RPC * first) * stride_bytes;
#pragma unroll
  for (int i = 0; i < nchunk; ++i) {
    const int c = first + step * i;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(lds_tile + c * 1024), 16, first_off + i * chunk_stride,
                                             0, 0, 0);
  }
}

// DMA 64 consecutive floats src[i0 + lane] (indices clamped to `last`) into
// LDS dst[lane]: one wave instruction.
__device__ __forceinline__ void dma_vec64_f32(const float* src, int i0, int last, unsigned char* lds_dst, int lane) {
  const uint32_t idx = (uint32_t)min(i0 + lane, last);
  const __amdgpu_buffer_rsrc_t r =
      make_rsrc(uniform(reinterpret_cast<const unsigned char*>(src)), (uint32_t)uniform(4 * (last + 1)));
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_dst, 4, 4u * idx, 0, 0, 0);
}

// Wait until at most N vector-memory operations of this wave are in flight
// (s_waitcnt vmcnt(N); expcnt and lgkmcnt left unconstrained). N <= 63.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier without the memory fence of __syncthreads(): LDS reads
// are complete (lgkmcnt 0), but vector-memory operations (in-flight tile
// DMAs) may stay outstanding; callers wait for those with wait_vmcnt first.
__device__ __forceinline__ void barrier_keep_dma() {
  __builtin_amdgcn_s_waitcnt((15 & 15) | ((63 >> 4) << 14) | (7 << 4) | (0 << 8));  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

// Transposed read of 4 consecutive rows x 1 column per lane from a swizzled
// d=128 tile: within each group of 16 lanes, lane j addresses row
// r0 + j/4, columns 16*cg + 4*(j%4) .. +3 (cg picks the 16-column half of a
// 32-column block), and receives the 4 rows of column 16*cg + j.
__device__ __forceinline__ i16x4 tr_read(const unsigned char* lds_tile_byte_addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)lds_tile_byte_addr);
}

}  // namespace fa
