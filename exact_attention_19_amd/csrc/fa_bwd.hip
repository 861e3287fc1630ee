// Backward attention kernels for gfx950 (MI355X).
//
// The backward pass recomputes the attention tiles from Q, K and the row
// logsumexp saved by the forward instead of reading a stored S or P
// (abeam.tech summary of the FlashAttention paper, "用語解説: Recomputation"
// and "学習時の backward では再計算を使う"). With P_ij = exp(S_ij - LSE_i)
// recomputed on chip, the gradients of L = sum(O * dO) are
//   dV = P^T dO,  dP = dO V^T,  D_i = sum_c dO_ic O_ic,  dS = P * (dP - D),
//   dQ = scale dS K,  dK = scale dS^T Q.
//
// Three launches on one stream:
//   1. preprocess: D = rowsum(dO * O) per (b, head, row), float32, and the
//      logsumexp rescaled to log2 units (LSE * log2 e) for the exp2 below.
//   2. dK/dV: one workgroup per (b, kv head, 128-key tile). Each wave keeps
//      32 keys' K and V fragments and their dK^T, dV^T accumulators in
//      registers and sweeps every query head of the GQA group and every
//      64-row query tile that the causal mask leaves visible (S = Q K^T,
//      dP = dO V^T, dV^T += dO^T P, dK^T += Q^T dS). dK and dV of a group
//      are summed in registers, so nothing is accumulated in memory.
//   3. dQ: one workgroup per (b, query head, 128-row query tile), shaped like
//      the forward (S^T = K Q^T, dP^T = V dO^T, dQ^T += K^T dS^T).
// No atomics: the result is bit-reproducible. dS is recomputed in both
// kernels (seven tile products per tile pair instead of five).
#include <type_traits>

#include "fa_common.h"
#include "fa_internal.h"

namespace fa {

// Query rows per step of the dK/dV kernel (64 or 128). 128 halves the
// barriers per FLOP but measured 36% slower (4.9 vs 3.6 ms at B=1, N=8192,
// H=96; the kernel's code grows from 35 to 60 KB), so 64 is used.
#ifndef KV_QTILE
#define KV_QTILE 64
#endif
constexpr int kDkdvQueryTile = KV_QTILE;

// VALU instructions placed after each MFMA in the pinned dQ schedule.
#ifndef DQ_SGB_VALU0
#define DQ_SGB_VALU0 3
#endif
#ifndef DQ_SGB_VALU1
#define DQ_SGB_VALU1 6
#endif

namespace {

constexpr int kBwdThreads = 256;

// ---------------------------------------------------------------------------
// 1. D_i = sum_c dO_ic O_ic
template <int D>
__global__ __launch_bounds__(256) void bwd_preprocess_kernel(const __bf16* __restrict__ o,
                                                             const __bf16* __restrict__ dout,
                                                             const float* __restrict__ lse,
                                                             float* __restrict__ delta, float* __restrict__ lse2,
                                                             int B, int Hq, int N, float* __restrict__ dq_acc) {
  constexpr int LPT = D / 8;
  const int64_t rows = (int64_t)B * N * Hq;
  const int64_t gt = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t r = gt / LPT;
  const int dl = (int)(gt % LPT);
  const bool ok = r < rows;
  const int64_t rr = ok ? r : 0;
  if (dq_acc && ok) {  // the atomic backward's fp32 dQ accumulator starts at zero
    f32x4* z = reinterpret_cast<f32x4*>(dq_acc + rr * D + dl * 8);
    z[0] = f32x4{};
    z[1] = f32x4{};
  }
  const u32x4 a = *reinterpret_cast<const u32x4*>(o + rr * D + dl * 8);
  const u32x4 g = *reinterpret_cast<const u32x4*>(dout + rr * D + dl * 8);
  const float tot = row_group_sum<LPT>(dot8_bf16(a, g, 0.f));
  if (ok && dl == 0) {
    const int64_t per_b = (int64_t)N * Hq;
    const int64_t b = rr / per_b;
    const int64_t rem = rr - b * per_b;
    const int64_t i = rem / Hq;
    const int64_t h = rem - i * Hq;
    const int64_t idx = (b * Hq + h) * N + i;
    delta[idx] = tot;
    lse2[idx] = lse[idx] * kLog2e;  // exponent reference in log2 units
  }
}

// dQ = bf16(scale * dQacc), 8 elements per thread (the atomic backward).
__global__ __launch_bounds__(256) void bwd_dq_finalize_kernel(const float* __restrict__ acc, __bf16* __restrict__ dq,
                                                              int64_t n8, float scale) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const f32x4* a = reinterpret_cast<const f32x4*>(acc + 8 * i);
  const f32x4 x = a[0], y = a[1];
  u32x4 w;
  w[0] = pack_bf16x2(x[0] * scale, x[1] * scale);
  w[1] = pack_bf16x2(x[2] * scale, x[3] * scale);
  w[2] = pack_bf16x2(y[0] * scale, y[1] * scale);
  w[3] = pack_bf16x2(y[2] * scale, y[3] * scale);
  *reinterpret_cast<u32x4*>(dq + 8 * i) = w;
}

// ---------------------------------------------------------------------------
// 2. dK, dV and 3. dQ. Row-major 64 x d tiles (rows of 2 d bytes, swizzled by
// row_swz) go from global memory straight into LDS (global_load_lds_dwordx4);
// transposed MFMA operands (Q^T, dO^T, K^T) are read from the same tiles with
// ds_read_b64_tr_b16, so no tile is stored twice and nothing passes through
// staging registers.
// For a 16-row step st of a 64-row tile, a transposed read at row offset
// 4*hh + j/4 (+8) yields, for the lane's column, the rows the score
// accumulator pairs with it: 16*st + 4*hh + {0..3} and 16*st + 8 + 4*hh + {0..3}.

// Per-lane byte offsets inside a swizzled tile for a transposed operand read
// (second read at index 1), for column block 0; column block db is reached by
// XOR with 64*db, 16-row step st by adding 16 rows (32*D bytes) per step.
template <int D = 128>
__device__ __forceinline__ void tr_offsets(int lane, int (&off)[2]) {
  const int j = lane & 15, g = lane >> 4, hh = lane >> 5;
#pragma unroll
  for (int rd = 0; rd < 2; ++rd) {
    const int r = 4 * hh + (j >> 2) + 8 * rd;
    const int unit = 2 * (g & 1) + ((j & 3) >> 1);
    off[rd] = r * 2 * D + 16 * (unit ^ row_swz<D>(r)) + 8 * (j & 1);
  }
}

template <int D = 128>
__device__ __forceinline__ bf16x8 tr_operand(const unsigned char* tile, int st, int db, const int (&off)[2]) {
  const i16x4 lo = tr_read(tile + st * 32 * D + (off[0] ^ (64 * db)));
  const i16x4 hi = tr_read(tile + st * 32 * D + (off[1] ^ (64 * db)));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Row operand (16 bytes of row r0 + l32, 16-deep step s) from a swizzled
// tile: byte offset (roff ^ (32*s)) + 8192 * (r0 / 32), roff from row_offset.
template <int D = 128>
__device__ __forceinline__ int row_offset(int lane) {
  const int l32 = lane & 31, hh = lane >> 5;
  return l32 * 2 * D + 16 * (hh ^ row_swz<D>(l32));
}

// dK, dV, four waves: one workgroup per (b, kv head, 128 keys); wave w keeps
// keys k0 + 32w .. +31 (K, V fragments and dK^T, dV^T accumulators in
// registers) and sweeps the visible 64-row query tiles of every query head
// in the GQA group. Launched for d = 64, where the fragments and
// accumulators take half the registers (248 in all) so two workgroups share
// a CU, and for the fused dQ below at d = 128 (one wave per SIMD); the
// deterministic d = 128 backward runs bwd_dkdv8_kernel.
//
// FUSED (the atomic backward) also produces dQ, so that the backward runs
// the five N x N x d products once each instead of recomputing S and dP in a
// separate dQ kernel: every wave writes its dS block to an LDS tile
// [64 queries x 128 keys], and during the next step wave w adds
// dQ[:, 32w .. 32w+31] += dS K over the workgroup's 128 keys (K kept in LDS)
// into an fp32 accumulator with atomic adds (so dQ's last bits depend on the
// order in which workgroups arrive).
template <bool CAUSAL, bool WINDOW, int BQ, bool FUSED = false, int D = 128>
__global__ __launch_bounds__(kBwdThreads, D == 64 ? 2 : 1) void bwd_dkdv_d128_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const __bf16* __restrict__ dout, const float* __restrict__ lse2, const float* __restrict__ delta,
    __bf16* __restrict__ dk, __bf16* __restrict__ dv, int B, int Hq, int Hkv, int N, float scale,
    float scale_log2, int win_left, int win_right, float* __restrict__ dq_acc) {
  constexpr int DS = D / 16, DB = D / 32, BKV = 128;
  constexpr int ROWB = 2 * D;                  // bytes of one tile row
  constexpr int QBLK = 32 * ROWB;              // 32 rows of a tile
  constexpr int NQB = BQ / 32;                 // 32-query blocks per query tile
  static_assert(BQ == 64 || BQ == 128, "query tiles of 64 or 128 rows");
  static_assert(D == 128 || (D == 64 && !FUSED), "d = 128, or d = 64 without the fused dQ");
  static_assert(!FUSED || (BQ == 64 && !WINDOW), "fused dQ: 64-query tiles, no window");
  // Key j is visible to query i iff j <= i (causal), i - wl <= j <= i + wr
  // (window, a negative side unbounded) and both are < N.
  const int wl = WINDOW ? win_left : -1;
  const int wr = WINDOW ? win_right : -1;
  constexpr int TILE = BQ * ROWB;              // one BQ x D bf16 tile (Q, then dO)
  constexpr int VEC_OFF = 2 * TILE;            // lse2 (BQ floats) then delta (BQ floats)
  constexpr int STAGE = 2 * TILE + 8 * BQ;
  constexpr int KT_OFF = 2 * STAGE;            // FUSED: the workgroup's 128 K rows (two 64-row tiles)
  constexpr int DSB_OFF = KT_OFF + 2 * 16384;  // FUSED: two [64 x 128] dS tiles, by step parity
  extern __shared__ __align__(1024) unsigned char smem[];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, hh = lane >> 5;

  const int BHK = B * Hkv;
  const int nkt = (N + BKV - 1) / BKV;
  int bhk, kt;
  if (BHK % 8 == 0) {
    // Workgroups are dealt round-robin to the 8 XCDs: keep every key tile of
    // kv head h on XCD h % 8, so the query tiles they all stream share its L2.
    xcd_order(blockIdx.x, BHK, nkt, kDkdvHeadGroup, bhk, kt);
  } else {
    bhk = blockIdx.x % BHK;
    kt = blockIdx.x / BHK;  // low key tiles see the most query tiles: launched first
  }
  const int b = uniform(bhk / Hkv);
  const int hk = uniform(bhk - b * Hkv);
  const int G = Hq / Hkv;

  const int64_t q_rs = (int64_t)Hq * D;
  const int64_t kv_rs = (int64_t)Hkv * D;
  const int k0 = kt * BKV;
  const int kw0 = k0 + wave * 32;
  const int my_key = kw0 + l32;
  const bool wave_active = kw0 < N;

  bf16x8 kf[DS], vf[DS];
  {
    const int64_t off = ((int64_t)b * N + min(my_key, N - 1)) * kv_rs + (int64_t)hk * D + 8 * hh;
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      kf[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(k + off + 16 * s));
      vf[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(v + off + 16 * s));
    }
  }

  // Query tiles of each head in the group, in two phases: first every tile
  // that needs masking for some wave of the workgroup (the causal diagonal,
  // the window's edges, a ragged last tile), for all heads; then all full
  // tiles. Each phase is a loop with its own body, so the full tiles run a
  // branch-free body. Per head the visited tiles are [qlo, qhi), the full
  // ones [f_lo, f_hi).
  const int nqt = (N + BQ - 1) / BQ;
  const int k_last = k0 + BKV - 1;
  int q_lo_row = 0, q_hi_row = N - 1;  // queries that see some key of the workgroup
  if (CAUSAL) q_lo_row = k0;
  if (WINDOW && wr >= 0) q_lo_row = max(q_lo_row, k0 - wr);
  if (WINDOW && wl >= 0) q_hi_row = min(q_hi_row, k_last + wl);
  const int qlo = min(max(q_lo_row, 0), N) / BQ;
  const int qhi = q_hi_row >= max(q_lo_row, 0) ? q_hi_row / BQ + 1 : qlo;
  int f_lo = qlo, f_hi = qhi;
  if (CAUSAL) f_lo = max(f_lo, (k_last + BQ - 1) / BQ);
  if (WINDOW && wr >= 0) f_lo = max(f_lo, (max(k_last - wr, 0) + BQ - 1) / BQ);
  if (WINDOW && wl >= 0) f_hi = min(f_hi, k0 + wl - (BQ - 1) >= 0 ? (k0 + wl - (BQ - 1)) / BQ + 1 : 0);
  if (N % BQ != 0) f_hi = min(f_hi, nqt - 1);
  f_lo = min(f_lo, qhi);
  f_hi = max(f_hi, f_lo);
  const int n_lo = f_lo - qlo;
  const int n_m = n_lo + (qhi - f_hi);  // masked tiles per head
  const int n_u = f_hi - f_lo;          // full tiles per head
  const int n1 = G * n_m;
  const int n_iter = n1 + G * n_u;
  // Iteration it is tile j of head h within its phase: it = h * n_m + j in
  // the first phase, n1 + h * n_u + j in the second. The loops visit it in
  // order, so (h, j) is carried along and advanced by one (no divisions).
  struct Cursor { int h, j; };
  auto tile_at = [&](int it, Cursor c, int& hq, int& q0) __attribute__((always_inline)) {
    hq = hk * G + c.h;
    if (it < n1) q0 = (c.j < n_lo ? qlo + c.j : f_hi + (c.j - n_lo)) * BQ;
    else q0 = (f_lo + c.j) * BQ;
  };
  auto advance = [&](int it, Cursor c) __attribute__((always_inline)) {  // cursor of it + 1
    if (it + 1 == n1) return Cursor{0, 0};
    const int n = it < n1 ? n_m : n_u;
    return c.j + 1 < n ? Cursor{c.h, c.j + 1} : Cursor{c.h + 1, 0};
  };
  Cursor cur{0, 0};

  const int roff = row_offset<D>(lane);
  int toff[2];
  tr_offsets<D>(lane, toff);
  const uint32_t q_rs_bytes = (uint32_t)(q_rs * 2);
  const uint32_t dma_off = dma_lane_offset_d<D>(lane, wave, q_rs_bytes);
  constexpr int CPW = 64 * ROWB / 1024 / 4;  // 1 KB chunks per wave of a 64-row tile

  f32x16 dkacc[DB], dvacc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) { dkacc[i] = f32x16{}; dvacc[i] = f32x16{}; }

  auto issue = [&](int it, Cursor c, int stage) __attribute__((always_inline)) {
    int hq, q0;
    tile_at(it, c, hq, q0);
    unsigned char* st = smem + stage * STAGE;
#pragma unroll
    for (int h = 0; h < BQ / 64; ++h) {
      const int64_t off = ((int64_t)b * N + q0 + 64 * h) * q_rs * 2 + (int64_t)hq * D * 2;
      dma_rows64_d<D>(reinterpret_cast<const unsigned char*>(q) + off, q_rs_bytes, N - q0 - 64 * h,
                      st + h * 64 * ROWB, wave, 4, CPW, dma_off);
      dma_rows64_d<D>(reinterpret_cast<const unsigned char*>(dout) + off, q_rs_bytes, N - q0 - 64 * h,
                      st + TILE + h * 64 * ROWB, wave, 4, CPW, dma_off);
    }
    const int64_t vb = ((int64_t)b * Hq + hq) * N;
    // lse2 then delta, 64 floats per wave instruction, spread over the waves
#pragma unroll
    for (int h = 0; h < BQ / 64; ++h) {
      if (wave == 2 * h % 4) dma_vec64_f32(lse2 + vb, q0 + 64 * h, N - 1, st + VEC_OFF + 256 * h, lane);
      if (wave == (2 * h + 1) % 4) dma_vec64_f32(delta + vb, q0 + 64 * h, N - 1, st + VEC_OFF + 4 * BQ + 256 * h, lane);
    }
  };

  // The tile's two 32-query blocks are skewed so that independent work sits
  // side by side for the scheduler: S/dP of block 1 next to the softmax
  // algebra of block 0, and the dV/dK products of block 0 next to the
  // algebra of block 1.
  //   scores(qb):  S = Q K^T and dP = dO V^T for the 32 queries of block qb
  //   algebra(qb): P = exp2(S*c - LSE2), dS = P * (dP - D), both to bf16
  //   update(qb):  dV^T += dO^T P, dK^T += Q^T dS
  struct Scores { f32x16 s, dp; };
  struct Probs { bf16x8 p[2], ds[2]; };
  auto scores = [&](const unsigned char* st, int qb) __attribute__((always_inline)) {
    const unsigned char* qs = st;
    const unsigned char* ds_ = st + TILE;
    Scores r{f32x16{}, f32x16{}};
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      r.s = mfma32(*reinterpret_cast<const bf16x8*>(qs + qb * QBLK + (roff ^ (32 * s))), kf[s], r.s);
      r.dp = mfma32(*reinterpret_cast<const bf16x8*>(ds_ + qb * QBLK + (roff ^ (32 * s))), vf[s], r.dp);
    }
    return r;
  };
  // Element e of a block is query q0 + 32*qb + 4*hh + c(e), c(e) = 8*(e/4) +
  // e%4. It is masked (score set to -inf, so P = dS = 0) when the query
  // precedes the key (causal) or lies past N. Called under a wave-uniform
  // branch on diagonal and ragged tiles only.
  auto apply_mask = [&](Scores& sc, int q0, int qb) __attribute__((always_inline)) {
    const int qbase = q0 + 32 * qb + 4 * hh;
    int lo = CAUSAL ? my_key - qbase : -1;                        // masked iff c(e) < lo
    if (WINDOW && wr >= 0) lo = max(lo, my_key - wr - qbase);
    int hi = N - 1 - qbase;                                       // masked iff c(e) > hi
    if (WINDOW && wl >= 0) hi = min(hi, my_key + wl - qbase);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int c = 8 * (e >> 2) + (e & 3);
      sc.s[e] = (c < lo || c > hi) ? kNegInf : sc.s[e];
    }
  };
  auto algebra = [&](const unsigned char* st, int qb, const Scores& sc) __attribute__((always_inline)) {
    const float* lse_s = reinterpret_cast<const float*>(st + VEC_OFF);
    const float* dlt_s = lse_s + BQ;
    Probs r;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(lse_s + 32 * qb + 8 * jj + 4 * hh);
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(dlt_s + 32 * qb + 8 * jj + 4 * hh);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = 4 * jj + i;
        const float p = fast_exp2(fmaf(sc.s[e], scale_log2, -l4[i]));
        r.p[e >> 3][e & 7] = (__bf16)p;
        r.ds[e >> 3][e & 7] = (__bf16)(p * (sc.dp[e] - d4[i]));
      }
    }
    return r;
  };
  auto update = [&](const unsigned char* st, int qb, const Probs& pr) __attribute__((always_inline)) {
    const unsigned char* qs = st;
    const unsigned char* ds_ = st + TILE;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int stp = 2 * qb + tt;
        dvacc[db] = mfma32(tr_operand<D>(ds_, stp, db, toff), pr.p[tt], dvacc[db]);
        dkacc[db] = mfma32(tr_operand<D>(qs, stp, db, toff), pr.ds[tt], dkacc[db]);
      }
    }
  };
  // FUSED: dS of block qb into the LDS tile dsb, row = query within the tile,
  // 16-byte units swizzled as the Q tiles. Within each 16-key group, keys
  // 4-7 and 8-11 trade places (bits 2 and 3 of the key swapped), so that one
  // 16-byte row read yields keys {0-3, 8-11} (lanes 0-31) or {4-7, 12-15}
  // (lanes 32-63): the order in which the transposed K operand pairs them.
  // A key past N (its K row, loaded clamped, stands in for the last key) gets
  // dS = 0 here, so it adds nothing to dQ whatever its scores were.
  auto store_ds = [&](unsigned char* dsb, int qb, const Probs& pr) __attribute__((always_inline)) {
    const int kl = 32 * wave + l32;
    const int pos = (kl & ~15) | (kl & 3) | ((kl & 4) << 1) | ((kl & 8) >> 1);
    const int unit = pos >> 3, byte = 2 * (pos & 7);
    const bool valid = my_key < N;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int row = 32 * qb + 8 * (e >> 2) + 4 * hh + (e & 3);
      *reinterpret_cast<__bf16*>(dsb + row * 256 + 16 * (unit ^ tile_swz(row)) + byte) =
          valid ? pr.ds[e >> 3][e & 7] : (__bf16)0.f;
    }
  };
  // FUSED: dQ rows q0 .. q0+63, columns 32w .. 32w+31 of query head hq from
  // the dS tile of that step: 16 MFMAs over the 128 keys (16-key steps of
  // waves whose keys the tile skipped are left out), then one atomic add per
  // element.
  auto dq_pass = [&](const unsigned char* dsb, int hq, int q0, int skipmask) __attribute__((always_inline)) {
    f32x16 acc[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      if (skipmask & (1 << (ks >> 1))) continue;
      const bf16x8 kop = tr_operand(smem + KT_OFF, ks, wave, toff);
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
        acc[qb] = mfma32(*reinterpret_cast<const bf16x8*>(dsb + qb * 8192 + (roff ^ (32 * ks))), kop, acc[qb]);
    }
    if (skipmask == 15) return;
    float* base = dq_acc + ((int64_t)b * N + q0) * q_rs + (int64_t)hq * D + 32 * wave + l32;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = 32 * qb + 8 * (e >> 2) + 4 * hh + (e & 3);
        if (q0 + row < N) unsafeAtomicAdd(base + (int64_t)row * q_rs, acc[qb][e]);
      }
    }
  };
  // Waves whose 32 keys see no query of the tile at q0 (bit w set).
  auto skip_mask = [&](int q0) __attribute__((always_inline)) {
    int m = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int kw = k0 + 32 * w;
      if (kw >= N || (CAUSAL && q0 + BQ - 1 < kw)) m |= 1 << w;
    }
    return m;
  };
  int prev_hq = 0, prev_q0 = 0, prev_skip = 15;

  // MASK is a compile-time tag: tiles without masking (all but the causal
  // diagonal and the ragged end) run a branch-free body, one scheduling
  // region. (Pinning its issue order as in the dQ kernel measured slower
  // here, with one wave per SIMD; the compiler's order is kept.)
  auto tile_body = [&](const unsigned char* st, int q0, auto mask_tag, unsigned char* dsb)
                       __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    // Skewed over the NQB blocks: the scores of block qb + 1 are issued
    // before the algebra and products of block qb.
    Scores sa = scores(st, 0);
    if constexpr (MASK) apply_mask(sa, q0, 0);
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      Scores sb;
      if (qb + 1 < NQB) sb = scores(st, qb + 1);
      const Probs p = algebra(st, qb, sa);
      if (qb + 1 < NQB) {
        if constexpr (MASK) apply_mask(sb, q0, qb + 1);
      }
      update(st, qb, p);
      if constexpr (FUSED) store_ds(dsb, qb, p);
      if (qb + 1 < NQB) sa = sb;
    }
  };

  auto step = [&](int it, auto stage_tag, auto mask_tag) __attribute__((always_inline)) {
    constexpr int STG = decltype(stage_tag)::value;
    const Cursor nxt = advance(it, cur);
    // FUSED: dQ of the previous step (its dS tile completed at the barrier
    // that ended it); the atomics go out before this step's DMA, and the
    // wait below covers both.
    if constexpr (FUSED) {
      if (it > 0) dq_pass(smem + DSB_OFF + (STG ^ 1) * 16384, prev_hq, prev_q0, prev_skip);
    }
    if (it + 1 < n_iter) issue(it + 1, nxt, STG ^ 1);
    int hq_cur, q0;
    tile_at(it, cur, hq_cur, q0);
    cur = nxt;
    bool skip = !wave_active || (CAUSAL && q0 + BQ - 1 < kw0);
    if (WINDOW && wr >= 0) skip = skip || q0 + BQ - 1 < kw0 - wr;
    if (WINDOW && wl >= 0) skip = skip || q0 > kw0 + 31 + wl;
    if (!skip) tile_body(smem + STG * STAGE, q0, mask_tag, smem + DSB_OFF + STG * 16384);
    if constexpr (FUSED) {
      prev_hq = hq_cur;
      prev_q0 = q0;
      prev_skip = skip_mask(q0);
    }
    wait_vmcnt<0>();
    barrier_keep_dma();
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;

  if (n_iter > 0) issue(0, cur, 0);
  if constexpr (FUSED) {
    const uint32_t kv_rs_bytes = (uint32_t)(kv_rs * 2);
    const uint32_t kdma_off = dma_lane_offset(lane, wave, kv_rs_bytes);
    const unsigned char* kt = reinterpret_cast<const unsigned char*>(k) + ((int64_t)b * N + k0) * kv_rs * 2 +
                              (int64_t)hk * D * 2;
    dma_rows64(kt, kv_rs_bytes, N - k0, smem + KT_OFF, wave, 4, 4, kdma_off);
    dma_rows64(kt + (int64_t)64 * kv_rs * 2, kv_rs_bytes, N - k0 - 64, smem + KT_OFF + 16384, wave, 4, 4, kdma_off);
  }
  wait_vmcnt<0>();
  barrier_keep_dma();
  int it = 0;
  for (; it < n1; ++it) {
    if ((it & 1) == 0) step(it, S0{}, std::true_type{});
    else step(it, S1{}, std::true_type{});
  }
  if (it < n_iter && (it & 1)) step(it++, S1{}, std::false_type{});
  for (; it + 1 < n_iter; it += 2) {
    step(it, S0{}, std::false_type{});
    step(it + 1, S1{}, std::false_type{});
  }
  if (it < n_iter) step(it, S0{}, std::false_type{});
  if constexpr (FUSED) {
    if (n_iter > 0) dq_pass(smem + DSB_OFF + ((n_iter - 1) & 1) * 16384, prev_hq, prev_q0, prev_skip);
  }

  if (!wave_active || my_key >= N) return;
  const int64_t off = ((int64_t)b * N + my_key) * kv_rs + (int64_t)hk * D;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d = db * 32 + 8 * j + 4 * hh;
      u32x2 wk, wv;
      wk[0] = pack_bf16x2(dkacc[db][4 * j + 0] * scale, dkacc[db][4 * j + 1] * scale);
      wk[1] = pack_bf16x2(dkacc[db][4 * j + 2] * scale, dkacc[db][4 * j + 3] * scale);
      wv[0] = pack_bf16x2(dvacc[db][4 * j + 0], dvacc[db][4 * j + 1]);
      wv[1] = pack_bf16x2(dvacc[db][4 * j + 2], dvacc[db][4 * j + 3]);
      *reinterpret_cast<u32x2*>(dk + off + d) = wk;
      *reinterpret_cast<u32x2*>(dv + off + d) = wv;
    }
  }
}

// dK, dV at d = 128 (no window): one workgroup per (b, kv head, 128 keys) as
// above, but with 8 waves so that two share each SIMD. Waves w and w + 4 (one
// SIMD) take keys k0 + 32 (w % 4) .. +31 and query half w / 4 (rows 32 (w / 4)
// .. +31) of every 64-query tile. K and V of the workgroup's 128 keys sit in
// LDS and are read as MFMA operands like the Q and dO tiles, so a wave holds
// only its dK^T, dV^T accumulators (128 registers) and one block's scores,
// about 210 registers in all, where the four-wave kernel needs ~480 and runs
// one wave per SIMD. The cost is one more 16-byte LDS read per S and dP MFMA;
// in exchange the two waves of a SIMD hide each other's exponentials, LDS
// latency and barrier waits. The tiles are visited in the same two phases,
// each unrolled over the two ring stages. At the end the waves of query half
// 1 pass their partial dK, dV to their partners through LDS.
template <bool CAUSAL, bool WINDOW>
__global__ __launch_bounds__(512, 1) void bwd_dkdv8_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const __bf16* __restrict__ dout, const float* __restrict__ lse2, const float* __restrict__ delta,
    __bf16* __restrict__ dk, __bf16* __restrict__ dv, int B, int Hq, int Hkv, int N, float scale,
    float scale_log2, int win_left, int win_right) {
  constexpr int D = 128, DS = 8, DB = 4, BKV = 128, BQ = 64;
  const int wl = WINDOW ? win_left : -1;
  const int wr = WINDOW ? win_right : -1;
  constexpr int ROWB = 2 * D;
  constexpr int QBLK = 32 * ROWB;
  constexpr int TILE = BQ * ROWB;
  constexpr int VEC_OFF = 2 * TILE;
  constexpr int STAGE = 2 * TILE + 8 * BQ;
  constexpr int KT_OFF = 2 * STAGE;            // K rows k0 .. k0 + 127 (two 64-row tiles)
  constexpr int VT_OFF = KT_OFF + 2 * TILE;    // V rows likewise
  extern __shared__ __align__(1024) unsigned char smem[];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kb = wave & 3, qh = wave >> 2;
  const int l32 = lane & 31, hh = lane >> 5;

  const int BHK = B * Hkv;
  const int nkt = (N + BKV - 1) / BKV;
  int bhk, kt;
  if (BHK % 8 == 0) {
    xcd_order(blockIdx.x, BHK, nkt, kDkdvHeadGroup, bhk, kt);
  } else {
    bhk = blockIdx.x % BHK;
    kt = blockIdx.x / BHK;
  }
  const int b = uniform(bhk / Hkv);
  const int hk = uniform(bhk - b * Hkv);
  const int G = Hq / Hkv;

  const int64_t q_rs = (int64_t)Hq * D;
  const int64_t kv_rs = (int64_t)Hkv * D;
  const int k0 = kt * BKV;
  const int kw0 = k0 + kb * 32;
  const int my_key = kw0 + l32;
  const bool wave_active = kw0 < N;

  const int nqt = (N + BQ - 1) / BQ;
  const int k_last = k0 + BKV - 1;
  int q_lo_row = 0, q_hi_row = N - 1;  // queries that see some key of the workgroup
  if (CAUSAL) q_lo_row = k0;
  if (WINDOW && wr >= 0) q_lo_row = max(q_lo_row, k0 - wr);
  if (WINDOW && wl >= 0) q_hi_row = min(q_hi_row, k_last + wl);
  const int qlo = min(max(q_lo_row, 0), N) / BQ;
  const int qhi = q_hi_row >= max(q_lo_row, 0) ? q_hi_row / BQ + 1 : qlo;
  int f_lo = qlo, f_hi = qhi;
  if (CAUSAL) f_lo = max(f_lo, (k_last + BQ - 1) / BQ);
  if (WINDOW && wr >= 0) f_lo = max(f_lo, (max(k_last - wr, 0) + BQ - 1) / BQ);
  if (WINDOW && wl >= 0) f_hi = min(f_hi, k0 + wl - (BQ - 1) >= 0 ? (k0 + wl - (BQ - 1)) / BQ + 1 : 0);
  if (N % BQ != 0) f_hi = min(f_hi, nqt - 1);
  f_lo = min(f_lo, qhi);
  f_hi = max(f_hi, f_lo);
  const int n_lo = f_lo - qlo;
  const int n_m = n_lo + (qhi - f_hi);
  const int n_u = f_hi - f_lo;
  const int n1 = G * n_m;
  const int n_iter = n1 + G * n_u;
  struct Cursor { int h, j; };
  auto tile_at = [&](int it, Cursor c, int& hq, int& q0) __attribute__((always_inline)) {
    hq = hk * G + c.h;
    if (it < n1) q0 = (c.j < n_lo ? qlo + c.j : f_hi + (c.j - n_lo)) * BQ;
    else q0 = (f_lo + c.j) * BQ;
  };
  auto advance = [&](int it, Cursor c) __attribute__((always_inline)) {
    if (it + 1 == n1) return Cursor{0, 0};
    const int n = it < n1 ? n_m : n_u;
    return c.j + 1 < n ? Cursor{c.h, c.j + 1} : Cursor{c.h + 1, 0};
  };
  Cursor cur{0, 0};

  const int roff = row_offset<D>(lane);
  int toff[2];
  tr_offsets<D>(lane, toff);
  const uint32_t q_rs_bytes = (uint32_t)(q_rs * 2);
  const uint32_t kv_rs_bytes = (uint32_t)(kv_rs * 2);
  const uint32_t dma_off = dma_lane_offset(lane, wave, q_rs_bytes);

  f32x16 dkacc[DB], dvacc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) { dkacc[i] = f32x16{}; dvacc[i] = f32x16{}; }

  // Q and dO tiles: 16 chunks of 1 KB each, two per wave; LSE2 and D by waves 0, 1.
  auto issue = [&](int it, Cursor c, int stage) __attribute__((always_inline)) {
    int hq, q0;
    tile_at(it, c, hq, q0);
    unsigned char* st = smem + stage * STAGE;
    const int64_t off = ((int64_t)b * N + q0) * q_rs * 2 + (int64_t)hq * D * 2;
    dma_rows64(reinterpret_cast<const unsigned char*>(q) + off, q_rs_bytes, N - q0, st, wave, 8, 2, dma_off);
    dma_rows64(reinterpret_cast<const unsigned char*>(dout) + off, q_rs_bytes, N - q0, st + TILE, wave, 8, 2, dma_off);
    const int64_t vb = ((int64_t)b * Hq + hq) * N;
    if (wave == 0) dma_vec64_f32(lse2 + vb, q0, N - 1, st + VEC_OFF, lane);
    if (wave == 1) dma_vec64_f32(delta + vb, q0, N - 1, st + VEC_OFF + 4 * BQ, lane);
  };

  struct Scores { f32x16 s, dp; };
  struct Probs { bf16x8 p[2], ds[2]; };
  const unsigned char* ks = smem + KT_OFF + kb * QBLK;
  const unsigned char* vs = smem + VT_OFF + kb * QBLK;
  auto scores = [&](const unsigned char* st) __attribute__((always_inline)) {
    const unsigned char* qs = st + qh * QBLK;
    const unsigned char* ds_ = st + TILE + qh * QBLK;
    Scores r{f32x16{}, f32x16{}};
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      const int o = roff ^ (32 * s);
      r.s = mfma32(*reinterpret_cast<const bf16x8*>(qs + o), *reinterpret_cast<const bf16x8*>(ks + o), r.s);
      r.dp = mfma32(*reinterpret_cast<const bf16x8*>(ds_ + o), *reinterpret_cast<const bf16x8*>(vs + o), r.dp);
    }
    return r;
  };
  auto apply_mask = [&](Scores& sc, int q0) __attribute__((always_inline)) {
    const int qbase = q0 + 32 * qh + 4 * hh;
    int lo = CAUSAL ? my_key - qbase : -1;                        // masked iff c(e) < lo
    if (WINDOW && wr >= 0) lo = max(lo, my_key - wr - qbase);
    int hi = N - 1 - qbase;                                       // masked iff c(e) > hi
    if (WINDOW && wl >= 0) hi = min(hi, my_key + wl - qbase);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int c = 8 * (e >> 2) + (e & 3);
      sc.s[e] = (c < lo || c > hi) ? kNegInf : sc.s[e];
    }
  };
  auto algebra = [&](const unsigned char* st, const Scores& sc) __attribute__((always_inline)) {
    const float* lse_s = reinterpret_cast<const float*>(st + VEC_OFF);
    const float* dlt_s = lse_s + BQ;
    Probs r;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(lse_s + 32 * qh + 8 * jj + 4 * hh);
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(dlt_s + 32 * qh + 8 * jj + 4 * hh);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = 4 * jj + i;
        const float p = fast_exp2(fmaf(sc.s[e], scale_log2, -l4[i]));
        r.p[e >> 3][e & 7] = (__bf16)p;
        r.ds[e >> 3][e & 7] = (__bf16)(p * (sc.dp[e] - d4[i]));
      }
    }
    return r;
  };
  auto update = [&](const unsigned char* st, const Probs& pr) __attribute__((always_inline)) {
    const unsigned char* qs = st;
    const unsigned char* ds_ = st + TILE;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int stp = 2 * qh + tt;
        dvacc[db] = mfma32(tr_operand<D>(ds_, stp, db, toff), pr.p[tt], dvacc[db]);
        dkacc[db] = mfma32(tr_operand<D>(qs, stp, db, toff), pr.ds[tt], dkacc[db]);
      }
    }
  };
  auto step = [&](int it, auto stage_tag, auto mask_tag) __attribute__((always_inline)) {
    constexpr int STG = decltype(stage_tag)::value;
    constexpr bool MASK = decltype(mask_tag)::value;
    const Cursor nxt = advance(it, cur);
    if (it + 1 < n_iter) issue(it + 1, nxt, STG ^ 1);
    int hq_cur, q0;
    tile_at(it, cur, hq_cur, q0);
    cur = nxt;
    const int qw = q0 + 32 * qh;  // this wave's 32 queries
    bool skip = !wave_active || (CAUSAL && qw + 31 < kw0);
    if (WINDOW && wr >= 0) skip = skip || qw + 31 < kw0 - wr;
    if (WINDOW && wl >= 0) skip = skip || qw > kw0 + 31 + wl;
    if (!skip) {
      const unsigned char* st = smem + STG * STAGE;
      Scores sc = scores(st);
      if constexpr (MASK) apply_mask(sc, q0);
      const Probs p = algebra(st, sc);
      // Issue priority while the wave feeds its dV/dK products: when both
      // waves of the SIMD are ready, the one holding the matrix pipe keeps it
      // (measured 0.5 % faster, bitwise equal).
      __builtin_amdgcn_s_setprio(1);
      update(st, p);
      __builtin_amdgcn_s_setprio(0);
    }
    wait_vmcnt<0>();
    barrier_keep_dma();
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;

  {
    const unsigned char* kt0 = reinterpret_cast<const unsigned char*>(k) + ((int64_t)b * N + k0) * kv_rs * 2 +
                               (int64_t)hk * D * 2;
    const unsigned char* vt0 = reinterpret_cast<const unsigned char*>(v) + ((int64_t)b * N + k0) * kv_rs * 2 +
                               (int64_t)hk * D * 2;
    const uint32_t kdma_off = dma_lane_offset(lane, wave, kv_rs_bytes);
    dma_rows64(kt0, kv_rs_bytes, N - k0, smem + KT_OFF, wave, 8, 2, kdma_off);
    dma_rows64(kt0 + (int64_t)64 * kv_rs * 2, kv_rs_bytes, N - k0 - 64, smem + KT_OFF + TILE, wave, 8, 2, kdma_off);
    dma_rows64(vt0, kv_rs_bytes, N - k0, smem + VT_OFF, wave, 8, 2, kdma_off);
    dma_rows64(vt0 + (int64_t)64 * kv_rs * 2, kv_rs_bytes, N - k0 - 64, smem + VT_OFF + TILE, wave, 8, 2, kdma_off);
  }
  if (n_iter > 0) issue(0, cur, 0);
  wait_vmcnt<0>();
  barrier_keep_dma();
  int it = 0;
  for (; it + 1 < n1; it += 2) {
    step(it, S0{}, std::true_type{});
    step(it + 1, S1{}, std::true_type{});
  }
  if (it < n1) step(it++, S0{}, std::true_type{});
  if (it < n_iter && (it & 1)) step(it++, S1{}, std::false_type{});
  for (; it + 1 < n_iter; it += 2) {
    step(it, S0{}, std::false_type{});
    step(it + 1, S1{}, std::false_type{});
  }
  if (it < n_iter) step(it, S0{}, std::false_type{});

  // Partial sums of the query halves: waves 4-7 hand theirs to waves 0-3
  // through LDS (the ring and the K/V rows are no longer read: every wave has
  // passed the last barrier), 512 bytes per lane, 16-byte pieces lane-major.
  f32x4* red = reinterpret_cast<f32x4*>(smem) + (kb * 2 * DB * 4) * 64 + lane;
  if (qh == 1) {
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        red[((0 * DB + db) * 4 + j) * 64] = f32x4{dkacc[db][4 * j], dkacc[db][4 * j + 1], dkacc[db][4 * j + 2], dkacc[db][4 * j + 3]};
        red[((1 * DB + db) * 4 + j) * 64] = f32x4{dvacc[db][4 * j], dvacc[db][4 * j + 1], dvacc[db][4 * j + 2], dvacc[db][4 * j + 3]};
      }
    }
  }
  __syncthreads();
  if (qh == 1 || !wave_active || my_key >= N) return;
  const int64_t off = ((int64_t)b * N + my_key) * kv_rs + (int64_t)hk * D;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 pk = red[((0 * DB + db) * 4 + j) * 64];
      const f32x4 pv = red[((1 * DB + db) * 4 + j) * 64];
      const int d = db * 32 + 8 * j + 4 * hh;
      u32x2 wk, wv;
      wk[0] = pack_bf16x2((dkacc[db][4 * j + 0] + pk[0]) * scale, (dkacc[db][4 * j + 1] + pk[1]) * scale);
      wk[1] = pack_bf16x2((dkacc[db][4 * j + 2] + pk[2]) * scale, (dkacc[db][4 * j + 3] + pk[3]) * scale);
      wv[0] = pack_bf16x2(dvacc[db][4 * j + 0] + pv[0], dvacc[db][4 * j + 1] + pv[1]);
      wv[1] = pack_bf16x2(dvacc[db][4 * j + 2] + pv[2], dvacc[db][4 * j + 3] + pv[3]);
      *reinterpret_cast<u32x2*>(dk + off + d) = wk;
      *reinterpret_cast<u32x2*>(dv + off + d) = wv;
    }
  }
}

// dQ (d = 128 or 64): one workgroup per (b, query head, 128 query rows),
// shaped like the forward: S^T = K Q^T, dP^T = V dO^T, dQ^T += K^T dS^T.
template <bool CAUSAL, bool WINDOW, int D = 128>
__global__ __launch_bounds__(kBwdThreads, 2) void bwd_dq_d128_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const __bf16* __restrict__ dout, const float* __restrict__ lse2, const float* __restrict__ delta,
    __bf16* __restrict__ dq, int B, int Hq, int Hkv, int N, float scale, float scale_log2, int num_q_tiles,
    int win_left, int win_right) {
  constexpr int DS = D / 16, DB = D / 32, BM = 128, BN = 64;
  constexpr int ROWB = 2 * D;                  // bytes of one tile row
  constexpr int KBLK = 32 * ROWB;              // 32 rows of a tile
  constexpr int TILE = 64 * ROWB;
  static_assert(D == 64 || D == 128, "d = 64 or 128");
  constexpr int STAGE = 2 * TILE;  // K tile then V tile
  extern __shared__ __align__(1024) unsigned char smem[];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, hh = lane >> 5;

  const int BH = B * Hq;
  int bh, rank;
  if (BH % 8 == 0) {
    // Every query tile of head h on XCD h % 8 (workgroups are dealt
    // round-robin to the XCDs), so the K/V tiles they stream share its L2.
    xcd_order(blockIdx.x, BH, num_q_tiles, kDqHeadGroup, bh, rank);
  } else {
    bh = blockIdx.x % BH;
    rank = blockIdx.x / BH;
  }
  const int qt = CAUSAL ? (num_q_tiles - 1 - rank) : rank;
  const int b = uniform(bh / Hq);
  const int hq = uniform(bh - b * Hq);
  const int hk = uniform(hq / (Hq / Hkv));

  const int64_t q_rs = (int64_t)Hq * D;
  const int64_t kv_rs = (int64_t)Hkv * D;
  const int q0 = qt * BM;
  const int qw0 = q0 + wave * 32;
  const int my_q = qw0 + l32;
  const bool wave_active = qw0 < N;

  bf16x8 qf[DS], dof[DS];
  float my_lse2, my_dlt;
  {
    const int row = min(my_q, N - 1);
    const int64_t off = ((int64_t)b * N + row) * q_rs + (int64_t)hq * D + 8 * hh;
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      qf[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(q + off + 16 * s));
      dof[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(dout + off + 16 * s));
    }
    my_lse2 = lse2[((int64_t)b * Hq + hq) * N + row];
    my_dlt = delta[((int64_t)b * Hq + hq) * N + row];
  }

  // Keys any query of the workgroup can see: [kv_begin, kv_end); key j is
  // visible to query i iff j <= i (causal) and i - wl <= j <= i + wr (window,
  // a negative side unbounded).
  const int wl = WINDOW ? win_left : -1;
  const int wr = WINDOW ? win_right : -1;
  const int q_last = min(q0 + BM, N) - 1;
  int t_begin = 0, t_end;
  if constexpr (!WINDOW) {
    int kv_end = N;
    if (CAUSAL) kv_end = min(N, q0 + BM);
    t_end = (kv_end + BN - 1) / BN;
  } else {
    int kv_begin = 0, kv_end = N;
    if (CAUSAL) kv_end = min(kv_end, q_last + 1);
    if (wr >= 0) kv_end = min(kv_end, q_last + wr + 1);
    if (wl >= 0) kv_begin = max(0, q0 - wl);
    t_begin = kv_begin / BN;
    t_end = kv_end > kv_begin ? (kv_end + BN - 1) / BN : t_begin;
  }
  const unsigned char* kbase = reinterpret_cast<const unsigned char*>(k + (int64_t)b * N * kv_rs + (int64_t)hk * D);
  const unsigned char* vbase = reinterpret_cast<const unsigned char*>(v + (int64_t)b * N * kv_rs + (int64_t)hk * D);
  const uint32_t kv_rs_bytes = (uint32_t)(kv_rs * 2);
  const uint32_t dma_off = dma_lane_offset_d<D>(lane, wave, kv_rs_bytes);
  constexpr int CPW = TILE / 1024 / 4;  // 1 KB chunks per wave of a tile

  const int roff = row_offset<D>(lane);
  int toff[2];
  tr_offsets<D>(lane, toff);

  f32x16 dqacc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) dqacc[i] = f32x16{};

  auto issue = [&](int t, int stage) __attribute__((always_inline)) {
    unsigned char* st = smem + stage * STAGE;
    const int64_t off = (int64_t)t * BN * kv_rs * 2;
    dma_rows64_d<D>(kbase + off, kv_rs_bytes, N - t * BN, st, wave, 4, CPW, dma_off);
    dma_rows64_d<D>(vbase + off, kv_rs_bytes, N - t * BN, st + TILE, wave, 4, CPW, dma_off);
  };

  // Same skew as the dK/dV kernel: scores of key block 1 beside the algebra
  // of block 0, the dQ product of block 0 beside the algebra of block 1.
  struct Scores { f32x16 s, dp; };
  auto scores = [&](const unsigned char* st, int kbk) __attribute__((always_inline)) {
    const unsigned char* ks = st;
    const unsigned char* vs = st + TILE;
    Scores r{f32x16{}, f32x16{}};
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      r.s = mfma32(*reinterpret_cast<const bf16x8*>(ks + kbk * KBLK + (roff ^ (32 * s))), qf[s], r.s);
      r.dp = mfma32(*reinterpret_cast<const bf16x8*>(vs + kbk * KBLK + (roff ^ (32 * s))), dof[s], r.dp);
    }
    return r;
  };
  // Element e is key k0 + 32*kbk + 4*hh + c(e), c(e) = 8*(e/4) + e%4; masked
  // keys (past the causal bound or past N) get score -inf.
  auto apply_mask = [&](Scores& sc, int k0, int kbk) __attribute__((always_inline)) {
    const int base_key = k0 + kbk * 32 + 4 * hh;
    int lim = N - 1 - base_key;
    if (CAUSAL) lim = min(lim, my_q - base_key);
    if (WINDOW && wr >= 0) lim = min(lim, my_q + wr - base_key);
    if constexpr (WINDOW) {
      const int lo = wl >= 0 ? my_q - wl - base_key : -1;  // masked iff c(e) < lo
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int c = 8 * (e >> 2) + (e & 3);
        sc.s[e] = (c > lim || c < lo) ? kNegInf : sc.s[e];
      }
      return;
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) sc.s[e] = (8 * (e >> 2) + (e & 3) > lim) ? kNegInf : sc.s[e];
  };
  struct DsB { bf16x8 v[2]; };
  auto algebra = [&](const Scores& sc) __attribute__((always_inline)) {
    DsB r;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float p = fast_exp2(fmaf(sc.s[e], scale_log2, -my_lse2));
      r.v[e >> 3][e & 7] = (__bf16)(p * (sc.dp[e] - my_dlt));
    }
    return r;
  };
  auto update = [&](const unsigned char* st, int kbk, const DsB& d) __attribute__((always_inline)) {
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        dqacc[db] = mfma32(tr_operand<D>(st, 2 * kbk + tt, db, toff), d.v[tt], dqacc[db]);
      }
    }
  };
  // MASK is a compile-time tag: tiles that need no masking (all but the
  // causal diagonal and the ragged end) run a body without branches, so the
  // whole tile is one scheduling region and its issue order can be pinned:
  // the scores of block 0 (with block 1's operand reads in between), the
  // scores of block 1 interleaved with block 0's algebra, the dQ product of
  // block 0 interleaved with block 1's algebra, then the dQ product of block 1.
  auto tile_body = [&](const unsigned char* st, int k0, auto mask_tag) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    Scores s0 = scores(st, 0);
    if constexpr (MASK) apply_mask(s0, k0, 0);
    Scores s1 = scores(st, 1);
    const DsB d0 = algebra(s0);
    if constexpr (MASK) apply_mask(s1, k0, 1);
    update(st, 0, d0);
    const DsB d1 = algebra(s1);
    update(st, 1, d1);
    if constexpr (!MASK && D == 128) {
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, DQ_SGB_VALU0, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, DQ_SGB_VALU1, 0);
      }
    }
  };

  // Two LDS stages: step t issues tile t + 1 into the other stage, consumes
  // tile t, waits for its own DMAs and meets the other waves at the barrier.
  auto step = [&](int t, auto stage_tag, auto mask_tag) __attribute__((always_inline)) {
    constexpr int STG = decltype(stage_tag)::value;
    if (t + 1 < t_end) issue(t + 1, STG ^ 1);
    const int k0 = t * BN;
    bool skip = !wave_active || (CAUSAL && k0 > qw0 + 31);
    if (WINDOW && wr >= 0) skip = skip || k0 > qw0 + 31 + wr;
    if (WINDOW && wl >= 0) skip = skip || k0 + BN - 1 < qw0 - wl;
    if (!skip) tile_body(smem + STG * STAGE, k0, mask_tag);
    wait_vmcnt<0>();
    barrier_keep_dma();
  };
  auto step_any = [&](int t, auto mask_tag) __attribute__((always_inline)) {
    if ((((WINDOW ? t - t_begin : t)) & 1) == 0) step(t, std::integral_constant<int, 0>{}, mask_tag);
    else step(t, std::integral_constant<int, 1>{}, mask_tag);
  };
  if constexpr (!WINDOW) {
    // Tiles [0, n_full) need no mask for any query of the workgroup.
    int n_full = N / BN;
    if (CAUSAL) n_full = min(n_full, q0 / BN);
    n_full = min(n_full, t_end);
    issue(0, 0);
    wait_vmcnt<0>();
    barrier_keep_dma();
    int t = 0;
    for (; t + 1 < n_full; t += 2) {
      step(t, std::integral_constant<int, 0>{}, std::false_type{});
      step(t + 1, std::integral_constant<int, 1>{}, std::false_type{});
    }
    for (; t < t_end; ++t) step_any(t, std::true_type{});
  } else {
    // Tiles [f_begin, f_end) are visible in full to every query of the
    // workgroup and run the unmasked body; the window's edges run the masked
    // one (which is also correct on full tiles and takes the single steps
    // that align or end the unrolled loop).
    int full_hi = N - 1;
    if (CAUSAL) full_hi = min(full_hi, q0);
    if (wr >= 0) full_hi = min(full_hi, q0 + wr);
    int f_begin = t_begin;
    if (wl >= 0) f_begin = max(t_begin, (max(q_last - wl, 0) + BN - 1) / BN);
    int f_end = full_hi >= 0 ? (full_hi + 1) / BN : 0;
    f_end = max(min(f_end, t_end), f_begin);
    f_begin = min(f_begin, t_end);
    if (t_begin < t_end) issue(t_begin, 0);
    wait_vmcnt<0>();
    barrier_keep_dma();
    int t = t_begin;
    for (; t < f_begin; ++t) step_any(t, std::true_type{});
    if (t < f_end && ((t - t_begin) & 1)) step_any(t++, std::true_type{});
    for (; t + 1 < f_end; t += 2) {
      step(t, std::integral_constant<int, 0>{}, std::false_type{});
      step(t + 1, std::integral_constant<int, 1>{}, std::false_type{});
    }
    for (; t < t_end; ++t) step_any(t, std::true_type{});
  }

  if (!wave_active || my_q >= N) return;
  __bf16* orow = dq + ((int64_t)b * N + my_q) * q_rs + (int64_t)hq * D;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u32x2 w;
      w[0] = pack_bf16x2(dqacc[db][4 * j + 0] * scale, dqacc[db][4 * j + 1] * scale);
      w[1] = pack_bf16x2(dqacc[db][4 * j + 2] * scale, dqacc[db][4 * j + 3] * scale);
      *reinterpret_cast<u32x2*>(orow + db * 32 + 8 * j + 4 * hh) = w;
    }
  }
}

template <int D, bool CAUSAL, bool WINDOW = false>
hipError_t launch_bwd_t(const BwdArgs& a, float* delta, int stage) {
  const float scale_log2 = a.scale * kLog2e;
  float* lse2 = delta + bwd_vec_stride(a.B, a.Hq, a.N);
  if (stage == 0) {
    const int64_t threads = (int64_t)a.B * a.N * a.Hq * (D / 8);
    const int64_t grid = (threads + 255) / 256;
    if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(bwd_preprocess_kernel<D>, dim3((unsigned)grid), dim3(256), 0, a.stream,
                       (const __bf16*)a.o, (const __bf16*)a.dout, a.lse, delta, lse2, a.B, a.Hq, a.N, a.dq_acc);
    return hipGetLastError();
  }
  if (stage == 1) {
    const int nkt = (a.N + 127) / 128;
    const int64_t grid = (int64_t)nkt * a.B * a.Hkv;
    if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    if constexpr (D == 128 && !WINDOW) {
      if (a.dq_acc) {
        auto kern = bwd_dkdv_d128_kernel<CAUSAL, false, 64, true>;
        constexpr size_t smem = 2 * (2 * 64 * 256 + 8 * 64) + 2 * 16384 + 2 * 16384;
        hipError_t e = set_smem_once<bwd_dkdv_d128_kernel<CAUSAL, false, 64, true>>(smem);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kBwdThreads), smem, a.stream, (const __bf16*)a.q,
                           (const __bf16*)a.k, (const __bf16*)a.v, (const __bf16*)a.dout, (const float*)lse2,
                           (const float*)delta, (__bf16*)a.dk, (__bf16*)a.dv, a.B, a.Hq, a.Hkv, a.N, a.scale,
                           scale_log2, -1, -1, a.dq_acc);
        return hipGetLastError();
      }
    }
    if constexpr (D == 128) {
      auto kern = bwd_dkdv8_kernel<CAUSAL, WINDOW>;
      constexpr size_t smem = 2 * (2 * 64 * 256 + 8 * 64) + 2 * 2 * 64 * 256;  // Q/dO ring + K, V rows
      hipError_t e = set_smem_once<bwd_dkdv8_kernel<CAUSAL, WINDOW>>(smem);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(512), smem, a.stream, (const __bf16*)a.q,
                         (const __bf16*)a.k, (const __bf16*)a.v, (const __bf16*)a.dout, (const float*)lse2,
                         (const float*)delta, (__bf16*)a.dk, (__bf16*)a.dv, a.B, a.Hq, a.Hkv, a.N, a.scale,
                         scale_log2, a.win_left, a.win_right);
      return hipGetLastError();
    } else {
      constexpr int BQ = kDkdvQueryTile;
      auto kern = bwd_dkdv_d128_kernel<CAUSAL, WINDOW, BQ, false, D>;
      constexpr size_t smem = 2 * (2 * BQ * 2 * D + 8 * BQ);
      hipError_t e = set_smem_once<bwd_dkdv_d128_kernel<CAUSAL, WINDOW, BQ, false, D>>(smem);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kBwdThreads), smem, a.stream, (const __bf16*)a.q,
                         (const __bf16*)a.k, (const __bf16*)a.v, (const __bf16*)a.dout, (const float*)lse2,
                         (const float*)delta, (__bf16*)a.dk, (__bf16*)a.dv, a.B, a.Hq, a.Hkv, a.N, a.scale,
                         scale_log2, a.win_left, a.win_right, nullptr);
      return hipGetLastError();
    }
  }
  if (a.dq_acc) {  // atomic backward: dQ = bf16(scale * dQacc)
    const int64_t n8 = (int64_t)a.B * a.N * a.Hq * D / 8;
    const int64_t grid = (n8 + 255) / 256;
    if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(bwd_dq_finalize_kernel, dim3((unsigned)grid), dim3(256), 0, a.stream, (const float*)a.dq_acc,
                       (__bf16*)a.dq, n8, a.scale);
    return hipGetLastError();
  }
  const int nqt = (a.N + 127) / 128;
  const int64_t grid = (int64_t)nqt * a.B * a.Hq;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  {
    auto kern = bwd_dq_d128_kernel<CAUSAL, WINDOW, D>;
    constexpr size_t smem = 2 * 2 * 64 * 2 * D;
    hipError_t e = set_smem_once<bwd_dq_d128_kernel<CAUSAL, WINDOW, D>>(smem);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kBwdThreads), smem, a.stream, (const __bf16*)a.q,
                       (const __bf16*)a.k, (const __bf16*)a.v, (const __bf16*)a.dout, (const float*)lse2,
                       (const float*)delta, (__bf16*)a.dq, a.B, a.Hq, a.Hkv, a.N, a.scale, scale_log2, nqt,
                       a.win_left, a.win_right);
    return hipGetLastError();
  }
}

}  // namespace

hipError_t launch_bwd_stage(const BwdArgs& a, float* delta, int stage) {
  const bool window = a.win_left >= 0 || a.win_right >= 0;
  if (a.d == 64) {
    if (window)
      return a.causal ? launch_bwd_t<64, true, true>(a, delta, stage) : launch_bwd_t<64, false, true>(a, delta, stage);
    return a.causal ? launch_bwd_t<64, true>(a, delta, stage) : launch_bwd_t<64, false>(a, delta, stage);
  }
  if (window) {
    return a.causal ? launch_bwd_t<128, true, true>(a, delta, stage) : launch_bwd_t<128, false, true>(a, delta, stage);
  }
  return a.causal ? launch_bwd_t<128, true>(a, delta, stage) : launch_bwd_t<128, false>(a, delta, stage);
}

hipError_t launch_bwd(const BwdArgs& a, float* delta) {
  for (int stage = 0; stage < 3; ++stage) {
    hipError_t e = launch_bwd_stage(a, delta, stage);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace fa
