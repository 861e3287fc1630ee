// Forward attention kernels for gfx950 (MI355X).
//
// O = softmax(Q K^T * scale [+ causal mask]) V, computed tile by tile
// (Qiita FlashAttention tutorial, sections 4.2-4.3; abeam.tech summary of the
// FlashAttention paper, "Tiling によるメモリアクセス削減" and "Softmax を
// ブロック単位で正しく計算する"): a workgroup keeps a block of query rows in
// registers, streams key/value tiles through LDS, keeps a running row
// maximum and exp-sum, rescales the output accumulator when the maximum
// grows, and writes only O and the row logsumexp.
//
// bf16 path, per wave (32 query rows):
//   S^T = K * Q^T with the 32x32x16 bf16 MFMA, so that every lane holds the
//   scores of a single query row (lane l: query l % 32, half the keys). Row
//   maximum and sum are then in-lane, plus one exchange with lane l ^ 32.
//   O^T += V^T * P^T with the same MFMA: the score accumulator, rounded to
//   bf16, is already the B operand once the keys of each 16-key step are
//   taken in the order the accumulator holds them; V^T is kept in LDS with
//   its keys stored in that same order, so the permutation cancels.
// fp32 path: a plain VALU kernel (one query row per lane), used for fp32
// inputs, where P must not be rounded.
#include <type_traits>

#include "fa_common.h"
#include "fa_internal.h"

namespace fa {

namespace {

constexpr int kBN = 64;  // keys per tile
// The running maximum used as the exponent reference is only raised when a
// row's new maximum exceeds it by more than this many powers of two.
constexpr float kRescaleSlack = 8.f;
// d = 64 launches of at most this many 128-row workgroups use the split-key kernel.
constexpr int64_t kSplitKMaxWorkgroups = 256;
// d = 128 path: a block's probabilities are accepted against a stale
// reference while each lane's sum of its 16 values stays at or below this.
constexpr float kSumLimit = 256.f;
// VALU instructions placed after each MFMA in the interleaved stretches.
#ifndef SGB_VALU
#define SGB_VALU 6
#endif

// Register-staged 64-key tile of the d = 64 split-key kernel: K rows (padded
// row stride), then V^T (D rows of kBN keys, stored transposed by
// store_transposed_4x8 in the order the score accumulator hands keys to the
// P V product).
template <int D, int NWAVES>
struct FwdSmem {
  static constexpr int KS = D + 8;                      // K row stride (elements), 16-byte pad
  static constexpr int K_ELEMS = kBN * KS;
  static constexpr int VT_ELEMS = D * kBN;              // V^T: D rows of kBN keys, no pad
  static constexpr int STAGE_ELEMS = K_ELEMS + VT_ELEMS;
  static constexpr int BYTES = 2 * STAGE_ELEMS * 2;     // two stages, bf16
};

// Small-grid path for d = 64 (bf16): the key range is split over the four
// waves of a workgroup, which all serve the same 32 query rows, so a short
// batch still fills the chip (one wave per 32 rows left each wave walking
// every key tile in series). Each step covers 128 keys laid out as two 64-key
// FwdSmem tiles (K rows, V^T); wave w stages and reads
// only their 32-key block w, so the waves never wait for each other inside
// the loop, and keeps its own running max (log2 units), sum and output. At
// the end the four partial results merge through LDS with log-sum-exp
// weights: O = sum_w 2^(m_w - m) O_w / sum_w 2^(m_w - m) l_w, m = max_w m_w.
template <bool CAUSAL>
__global__ __launch_bounds__(256, 2) void fwd_splitk_d64_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    __bf16* __restrict__ o, float* __restrict__ lse, int B, int Hq, int Hkv, int N, float scale_log2,
    int num_q_tiles) {
  constexpr int D = 64, DS = 4, DB = 2, C8 = 8;
  using SM = FwdSmem<64, 4>;
  constexpr int TILE_ELEMS = SM::STAGE_ELEMS;          // one 64-key tile: K rows, then V^T
  constexpr int STEP_ELEMS = 2 * TILE_ELEMS;           // 128 keys per step
  extern __shared__ __align__(16) unsigned char smem_raw[];
  __bf16* smem = reinterpret_cast<__bf16*>(smem_raw);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  const int BH = B * Hq;
  const int bh = blockIdx.x % BH;
  const int rank = blockIdx.x / BH;
  const int qt = CAUSAL ? (num_q_tiles - 1 - rank) : rank;
  const int b = bh / Hq;
  const int hq = bh - b * Hq;
  const int hk = hq / (Hq / Hkv);
  const int64_t q_rs = (int64_t)Hq * D;
  const int64_t kv_rs = (int64_t)Hkv * D;
  const __bf16* kb = k + ((int64_t)b * N) * kv_rs + (int64_t)hk * D;
  const __bf16* vb = v + ((int64_t)b * N) * kv_rs + (int64_t)hk * D;

  const int q0 = qt * 32;
  const int my_q = q0 + l32;
  bf16x8 qf[DS];
  {
    const __bf16* qrow = q + ((int64_t)b * N + min(my_q, N - 1)) * q_rs + (int64_t)hq * D + 8 * hh;
#pragma unroll
    for (int s = 0; s < DS; ++s) qf[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qrow + 16 * s));
  }
  const int kv_end = CAUSAL ? min(N, q0 + 32) : N;
  const int n_steps = (kv_end + 127) / 128;

  // Each wave stages only its own 32-key block of every step (keys
  // st*128 + 32*wave ..), in the step's shared tile layout, and reads only
  // that block, so no barrier is needed between steps (a wave's LDS
  // accesses complete in order). Register staging; rows past N read row
  // N - 1 (their scores are masked, so the duplicates never count). Every
  // lane issues the same loads, so the compiler can wait for one step's
  // loads while the next step's are in flight.
  const int ti_w = wave >> 1, kbk = wave & 1;  // this wave's tile and 32-key block within a step
  constexpr int KW = 4;                         // K chunks per lane: 32 rows x 8 chunks / 64 lanes
  const int v_kg = lane >> 3, v_dc = lane & 7;  // V group: keys 4*v_kg .. +3 of the block, dims 8*v_dc ..
  u32x4 kA[KW], kB[KW];
  u32x4 vA[4], vB[4];
  auto load_step = [&](int st, u32x4 (&kr)[KW], u32x4 (&vr)[4]) __attribute__((always_inline)) {
    const int k0w = st * 128 + wave * 32;
#pragma unroll
    for (int r = 0; r < KW; ++r) {
      const int c = lane + 64 * r;
      kr[r] = *reinterpret_cast<const u32x4*>(kb + (int64_t)min(k0w + c / C8, N - 1) * kv_rs + (c % C8) * 8);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      vr[i] = *reinterpret_cast<const u32x4*>(vb + (int64_t)min(k0w + 4 * v_kg + i, N - 1) * kv_rs + v_dc * 8);
  };
  auto store_step = [&](int stage, const u32x4 (&kr)[KW], const u32x4 (&vr)[4]) __attribute__((always_inline)) {
    __bf16* ks = smem + stage * STEP_ELEMS + ti_w * TILE_ELEMS;
#pragma unroll
    for (int r = 0; r < KW; ++r) {
      const int c = lane + 64 * r;
      *reinterpret_cast<u32x4*>(ks + (kbk * 32 + c / C8) * SM::KS + (c % C8) * 8) = kr[r];
    }
    store_transposed_4x8(ks + SM::K_ELEMS, 8 * kbk + v_kg, v_dc, vr);
  };

  f32x16 oacc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) oacc[i] = f32x16{};
  float m_run = kNegInf, l_run = 0.f;

  auto compute = [&](int st) __attribute__((always_inline)) {
    const int k0b = st * 128 + wave * 32;
    if (k0b >= kv_end) return;
    const __bf16* ks = smem + (st & 1) * STEP_ELEMS + ti_w * TILE_ELEMS;
    const __bf16* vt = ks + SM::K_ELEMS;
    f32x16 sacc = f32x16{};
    const __bf16* krow = ks + (kbk * 32 + l32) * SM::KS + 8 * hh;
#pragma unroll
    for (int s = 0; s < DS; ++s) sacc = mfma32(*reinterpret_cast<const bf16x8*>(krow + 16 * s), qf[s], sacc);
    float mt = kNegInf;
    const bool need_mask = (CAUSAL && k0b + 31 > q0) || k0b + 32 > N;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float x = sacc[e];
      if (need_mask) {
        const int key = k0b + 8 * (e >> 2) + 4 * hh + (e & 3);
        x = (key >= N || (CAUSAL && key > my_q)) ? kNegInf : x;
        sacc[e] = x;
      }
      mt = fmaxf(mt, x);
    }
    mt = pair_max(mt) * scale_log2;
    if (__builtin_amdgcn_ballot_w64(mt > m_run + kRescaleSlack)) {
      const float m_new = fmaxf(m_run, mt);
      const float alpha = (m_new == kNegInf) ? 1.f : fast_exp2(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;
      }
    }
    const float neg_m = (m_run == kNegInf) ? 0.f : -m_run;
    float psum = 0.f;
    bf16x8 pb[2];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float p = fast_exp2(fmaf(sacc[e], scale_log2, neg_m));
      psum += p;
      pb[e >> 3][e & 7] = (__bf16)p;
    }
    l_run += psum;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
        oacc[db] = mfma32(load_tr_operand(vt, db * 32 + l32, 2 * kbk + h, hh), pb[h], oacc[db]);
    }
  };

  // The loads run two steps ahead and are issued unconditionally (past the
  // last step they read clamped rows that are never stored): with the same
  // loads on every path, the wait before a store covers only the older step.
  load_step(0, kA, vA);
  load_step(1, kB, vB);
  store_step(0, kA, vA);
  for (int st = 0; st < n_steps; st += 2) {
    load_step(st + 2, kA, vA);
    compute(st);
    if (st + 1 < n_steps) store_step(1, kB, vB);
    if (st + 1 >= n_steps) break;
    load_step(st + 3, kB, vB);
    compute(st + 1);
    if (st + 2 < n_steps) store_step(0, kA, vA);
  }
  __syncthreads();  // every wave is done with the staging area before the merge reuses it

  // Merge through LDS (the stages are free after the last barrier): partial
  // O [4][32][64] fp32, then max and sum [4][32].
  constexpr int PO = D + 4;  // padded row stride of the partial outputs (no bank conflicts)
  float* part_o = reinterpret_cast<float*>(smem_raw);
  float* part_m = part_o + 4 * 32 * PO;
  float* part_l = part_m + 4 * 32;
  const float l_tot = pair_sum(l_run);
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f32x4 w4;
#pragma unroll
      for (int i = 0; i < 4; ++i) w4[i] = oacc[db][4 * j + i];
      *reinterpret_cast<f32x4*>(part_o + (wave * 32 + l32) * PO + db * 32 + 8 * j + 4 * hh) = w4;
    }
  }
  if (hh == 0) {
    part_m[wave * 32 + l32] = m_run;
    part_l[wave * 32 + l32] = l_tot;
  }
  __syncthreads();
  const int qi = wave * 8 + (lane >> 3);  // this lane's query row within the tile
  const int dc = (lane & 7) * 8;          // and its 8 output dimensions
  float m = kNegInf;
#pragma unroll
  for (int w = 0; w < 4; ++w) m = fmaxf(m, part_m[w * 32 + qi]);
  float wsum = 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float mw = part_m[w * 32 + qi];
    const float c = (mw == kNegInf) ? 0.f : fast_exp2(mw - m);
    wsum += c * part_l[w * 32 + qi];
    const f32x4 x0 = *reinterpret_cast<const f32x4*>(part_o + (w * 32 + qi) * PO + dc);
    const f32x4 x1 = *reinterpret_cast<const f32x4*>(part_o + (w * 32 + qi) * PO + dc + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[i] += c * x0[i];
      acc[4 + i] += c * x1[i];
    }
  }
  const int row = q0 + qi;
  if (row < N) {
    const bool empty = !(wsum > 0.f);
    const float inv = empty ? 0.f : 1.f / wsum;
    u32x4 out;
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = pack_bf16x2(acc[2 * i] * inv, acc[2 * i + 1] * inv);
    *reinterpret_cast<u32x4*>(o + ((int64_t)b * N + row) * q_rs + (int64_t)hq * D + dc) = out;
    if ((lane & 7) == 0) lse[((int64_t)b * Hq + hq) * N + row] = empty ? kNegInf : (m + __log2f(wsum)) * kLn2;
  }
}

// bf16 path for d = 128 and (dense batches) d = 64. K and V tiles go from
// global memory straight into swizzled row-major LDS tiles (no staging
// registers, no transposing stores; rows of 2 d bytes, swizzled by row_swz);
// the V^T operand of the P V product is read with ds_read_b64_tr_b16, whose
// 4-row blocks are exactly the key groups the score accumulator hands to one
// 16-key MFMA step: elements 0-3 are keys 16*st + 4*hh + {0..3}, elements
// 4-7 are keys 16*st + 8 + 4*hh + {0..3}.
//
// Each wave owns QB blocks of 32 query rows. Every K operand and V^T operand
// read from LDS feeds QB MFMAs (one per query block), so LDS read traffic per
// MFMA falls as 1/QB; with QB = 2 the O accumulators (128 registers) and the
// Q operands (64) need one wave per SIMD.
template <int NWAVES, int NSTAGE, int QB, bool CAUSAL, int MODE, int D = 128>
__global__ __launch_bounds__(NWAVES * 64, (QB == 1 ? (D == 64 ? 3 * 4 : 8) : 4) / NWAVES) void fwd_d128_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    __bf16* __restrict__ o, float* __restrict__ lse, int B, int Hq, int Hkv, int N, float scale_log2,
    int num_q_tiles, FwdSeq seq) {
  constexpr bool VARLEN = (MODE & kModeVarlen) != 0;
  constexpr bool WINDOW = (MODE & kModeWindow) != 0;
  constexpr bool BSPARSE = (MODE & kModeBlockSparse) != 0;
  static_assert(D == 128 || (D == 64 && QB == 1), "d = 64: one query block per wave");
  constexpr int ROWB = 2 * D;           // bytes of one tile row
  constexpr int WQ = 32 * QB;           // query rows per wave
  constexpr int BM = NWAVES * WQ;       // query rows per workgroup
  constexpr int DS = D / 16;
  constexpr int DB = D / 32;
  constexpr int TILE = 64 * ROWB;       // bytes of one 64 x D bf16 tile
  constexpr int STAGE = 2 * TILE;       // K tile then V tile
  constexpr int CPW = TILE / 1024 / NWAVES;  // 1 KB chunks per wave per tile
  static_assert(!BSPARSE || (BM == kBlockSparseBlock && !VARLEN && !WINDOW),
                "block-sparse mode: one 128-row query block per workgroup, dense batch");
  extern __shared__ __align__(1024) unsigned char smem[];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  const int BH = B * Hq;
  const int bid = blockIdx.x;
  int bh, rank;
  if (BH % 8 == 0) {
    // Workgroups are dealt round-robin to the 8 XCDs; give each XCD whole
    // heads (every query tile of head h on XCD h % 8) so its L2 holds them.
    xcd_order(bid, BH, num_q_tiles, kFwdHeadGroup, bh, rank);
  } else {
    bh = bid % BH;
    rank = bid / BH;
  }
  const int qt = CAUSAL ? (num_q_tiles - 1 - rank) : rank;
  const int b = uniform(bh / Hq);
  const int hq = uniform(bh - b * Hq);
  const int hk = uniform(hq / (Hq / Hkv));

  // This sequence: query rows [q_start, q_start + Nq) and key rows
  // [k_start, k_start + Nk) of the packed tensors (dense: b*N and N). Packed
  // offsets are clamped to the tensors, so malformed prefix sums cannot read
  // or write outside them.
  int q_start, Nq, k_start, Nk;
  if constexpr (VARLEN) {
    q_start = uniform(min(max(seq.cu_q[b], 0), seq.total_q));
    Nq = uniform(min(max(seq.cu_q[b + 1], q_start), seq.total_q)) - q_start;
    k_start = uniform(min(max(seq.cu_k[b], 0), seq.total_k));
    Nk = uniform(min(max(seq.cu_k[b + 1], k_start), seq.total_k)) - k_start;
  } else {
    q_start = b * N;
    Nq = N;
    k_start = b * N;
    Nk = N;
  }
  const int q0 = qt * BM;
  if (q0 >= Nq) return;  // whole workgroup past this sequence's queries
  const int off = Nk - Nq;  // bottom-right alignment of the causal mask / window
  const int wl = WINDOW ? seq.win_left : -1;
  const int wr = WINDOW ? seq.win_right : -1;

  const int64_t q_rs = (int64_t)Hq * D;
  const int64_t kv_rs = (int64_t)Hkv * D;
  const __bf16* kb = k + (int64_t)k_start * kv_rs + (int64_t)hk * D;
  const __bf16* vb = v + (int64_t)k_start * kv_rs + (int64_t)hk * D;

  const int qw0 = q0 + wave * WQ;
  const bool wave_active = qw0 < Nq;
  int my_q[QB];
#pragma unroll
  for (int j = 0; j < QB; ++j) my_q[j] = qw0 + 32 * j + l32;

  bf16x8 qf[QB][DS];
#pragma unroll
  for (int j = 0; j < QB; ++j) {
    const __bf16* qrow = q + ((int64_t)q_start + min(my_q[j], Nq - 1)) * q_rs + (int64_t)hq * D + 8 * hh;
#pragma unroll
    for (int s = 0; s < DS; ++s) qf[j][s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qrow + 16 * s));
  }

  // Keys any query of the workgroup can see: [kv_begin, kv_end).
  const int q_last = min(q0 + BM, Nq) - 1;
  int kv_begin = 0, kv_end = Nk;
  if (CAUSAL) kv_end = min(kv_end, q_last + off + 1);
  if (WINDOW && wr >= 0) kv_end = min(kv_end, q_last + off + wr + 1);
  if (WINDOW && wl >= 0) kv_begin = max(0, q0 + off - wl);
  const int t_begin = kv_begin / 64;
  const int t_end = kv_end > kv_begin ? (kv_end + 63) / 64 : t_begin;

  // Per-lane LDS byte offsets inside a tile (constant over the loop).
  // K operand (A of S^T): row 32*kbk + l32, logical unit 2*s + hh.
  //   offset = row*256 + 16*((2s + hh) ^ swz(row)) = koff ^ (32*s) + kbk*8192.
  const int koff = l32 * ROWB + 16 * (hh ^ row_swz<D>(l32));
  // V^T operand (A of O^T): tr reads at rows 16*st + 4*hh + j/4 (+8), column
  // block 32*db + 16*(g&1) + 4*(j&3), j = lane & 15, g = lane >> 4.
  int voff[2];
  {
    const int j = lane & 15, g = lane >> 4;
#pragma unroll
    for (int rd = 0; rd < 2; ++rd) {
      const int r = 4 * hh + (j >> 2) + 8 * rd;
      const int unit = 2 * (g & 1) + ((j & 3) >> 1);  // db = 0
      voff[rd] = r * ROWB + 16 * (unit ^ row_swz<D>(r)) + 8 * (j & 1);
    }
  }

  f32x16 oacc[QB][DB];
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int j = 0; j < QB; ++j) {
#pragma unroll
    for (int i = 0; i < DB; ++i) oacc[j][i] = f32x16{};
    m_run[j] = kNegInf;
    l_run[j] = 0.f;
  }

  const uint32_t kv_rs_bytes = (uint32_t)(kv_rs * 2);
  const uint32_t dma_off = dma_lane_offset_d<D>(lane, wave, kv_rs_bytes);
  auto issue = [&](int t, int stage) __attribute__((always_inline)) {
    unsigned char* st = smem + stage * STAGE;
    const int64_t off = (int64_t)t * 64 * kv_rs * 2;
    const int nrows = Nk - t * 64;
    dma_rows64_d<D>(reinterpret_cast<const unsigned char*>(kb) + off, kv_rs_bytes, nrows, st, wave, NWAVES, CPW,
                    dma_off);
    dma_rows64_d<D>(reinterpret_cast<const unsigned char*>(vb) + off, kv_rs_bytes, nrows, st + TILE, wave, NWAVES,
                    CPW, dma_off);
  };

  // A 64-key tile is two 32-key blocks, skewed so that independent work sits
  // side by side for the scheduler: the S^T MFMAs of block 1 beside the
  // exponentials of block 0, and the P V MFMAs of block 0 beside the
  // exponentials of block 1.
  struct Sc { f32x16 s[QB]; };
  auto scores = [&](const unsigned char* ks, int kbk) __attribute__((always_inline)) {
    Sc r;
#pragma unroll
    for (int j = 0; j < QB; ++j) r.s[j] = f32x16{};
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(ks + kbk * 32 * ROWB + (koff ^ (32 * s)));
#pragma unroll
      for (int j = 0; j < QB; ++j) r.s[j] = mfma32(a, qf[j][s], r.s[j]);
    }
    return r;
  };
  // Element e of query block j holds key k0 + 32*kbk + 4*hh + c(e),
  // c(e) = 8*(e/4) + e%4; it is masked (-inf) past the causal bound or past N.
  auto apply_mask = [&](Sc& sc, int k0, int kbk) __attribute__((always_inline)) {
    const int base_key = k0 + kbk * 32 + 4 * hh;
#pragma unroll
    for (int j = 0; j < QB; ++j) {
      int lim = Nk - 1 - base_key;                     // masked iff c(e) > lim
      if (CAUSAL) lim = min(lim, my_q[j] + off - base_key);
      if (WINDOW && wr >= 0) lim = min(lim, my_q[j] + off + wr - base_key);
      if constexpr (WINDOW) {
        const int lo = wl >= 0 ? my_q[j] + off - wl - base_key : -1;  // masked iff c(e) < lo
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int c = 8 * (e >> 2) + (e & 3);
          sc.s[j][e] = (c > lim || c < lo) ? kNegInf : sc.s[j][e];
        }
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) sc.s[j][e] = (8 * (e >> 2) + (e & 3) > lim) ? kNegInf : sc.s[j][e];
      }
    }
  };
  // Row maximum of a block in log2 units (max3 tree, then the partner lane).
  auto rowmax = [&](const f32x16& sc) __attribute__((always_inline)) {
    float m = fmaxf(sc[0], sc[1]);
#pragma unroll
    for (int e = 2; e < 16; e += 2) m = fmaxf(fmaxf(m, sc[e]), sc[e + 1]);
    return pair_max(m) * scale_log2;
  };
  // P = exp2(S*c - m) as bf16 MFMA operands; this lane's share of the row sum
  // is accumulated from the same rounded values with v_dot2_f32_bf16 against
  // (1, 1), so numerator and denominator see identical probabilities.
  struct Probs { bf16x8 pb[2]; float sum; };
  auto probs = [&](const f32x16& sc, float neg_m) __attribute__((always_inline)) {
    Probs r;
#pragma unroll
    for (int e = 0; e < 16; ++e) r.pb[e >> 3][e & 7] = (__bf16)fast_exp2(fmaf(sc[e], scale_log2, neg_m));
    const bf16x2 ones = as_bf16x2(0x3f803f80u);
    float acc = 0.f;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const u32x4 w = __builtin_bit_cast(u32x4, r.pb[h]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t wi = w[i];
        acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(wi), ones, acc, false);
      }
    }
    r.sum = acc;
    return r;
  };
  auto pv = [&](const unsigned char* vs, int kbk, const Probs* pr) __attribute__((always_inline)) {
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int st = 2 * kbk + tt;
        const i16x4 lo = tr_read(vs + st * 16 * ROWB + (voff[0] ^ (64 * db)));
        const i16x4 hi = tr_read(vs + st * 16 * ROWB + (voff[1] ^ (64 * db)));
        const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int j = 0; j < QB; ++j) oacc[j][db] = mfma32(a, pr[j].pb[tt], oacc[j][db]);
      }
    }
  };
  // O *= alpha for query block j. With one query block the accumulators sit
  // in VGPRs and are scaled in place. With two they live in AGPRs, where the
  // MFMAs read and write them; scaling them in place would make the register
  // allocator keep them in VGPRs instead (and spill), so the rare rescale goes
  // through a 4 KB per-wave LDS slot: store, scale in VGPRs, store, load
  // back, with compiler barriers so the round trip stays.
  float* resc_slot = reinterpret_cast<float*>(smem + NSTAGE * STAGE + wave * 4096) + lane * 16;  // QB > 1 only
  auto rescale_o = [&](int j, float alpha) __attribute__((always_inline)) {
    if constexpr (QB == 1) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[j][db][e] *= alpha;
      }
      return;
    }
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      *reinterpret_cast<f32x16*>(resc_slot) = oacc[j][db];
      asm volatile("" ::: "memory");
      f32x16 t = *reinterpret_cast<const f32x16*>(resc_slot);
#pragma unroll
      for (int e = 0; e < 16; ++e) t[e] *= alpha;
      *reinterpret_cast<f32x16*>(resc_slot) = t;
      asm volatile("" ::: "memory");
      oacc[j][db] = *reinterpret_cast<const f32x16*>(resc_slot);
    }
  };

  // Lazy rescale. P is first formed against the current reference m_run
  // (no row maximum in the common path). Each lane sums its 16 new
  // probabilities anyway; if no lane's sum exceeds kSumLimit, every p is at
  // most kSumLimit and the block is accepted as is. Otherwise (the reference
  // is stale by more than log2(kSumLimit), or it is still -inf, which makes
  // the sum inf or NaN) the rare path takes the block's row maximum, moves
  // the reference there, rescales O and l, and recomputes P. O and l always
  // share one reference.
  auto resync = [&](int j, const f32x16& sc) __attribute__((always_inline)) {
    const float m_new = fmaxf(m_run[j], rowmax(sc));
    const float alpha = (m_new == kNegInf) ? 1.f : fast_exp2(m_run[j] - m_new);
    l_run[j] *= alpha;
    rescale_o(j, alpha);
    m_run[j] = m_new;
    return probs(sc, (m_new == kNegInf) ? 0.f : -m_new);
  };
  auto tile = [&](const unsigned char* ks, const unsigned char* vs, int k0, auto mask_tag)
                  __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    Sc s0 = scores(ks, 0);
    if constexpr (MASK) apply_mask(s0, k0, 0);
    Sc s1 = scores(ks, 1);
    if constexpr (MASK) apply_mask(s1, k0, 1);
    Probs p0[QB], p1[QB];
#pragma unroll
    for (int j = 0; j < QB; ++j) p0[j] = probs(s0.s[j], -m_run[j]);
    if constexpr (QB == 1) {
      // Issue order for this stretch: the 8 K operand reads of block 0, its
      // 8 MFMAs each followed by one K read of block 1, then the 8 MFMAs of
      // block 1 each followed by a share of block 0's softmax VALU work.
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, SGB_VALU, 0);
      }
    }
#pragma unroll
    for (int j = 0; j < QB; ++j) {
      if (__builtin_amdgcn_ballot_w64(!(p0[j].sum <= kSumLimit))) p0[j] = resync(j, s0.s[j]);
      l_run[j] += p0[j].sum;
    }
    // Issue priority while this wave feeds its P V MFMAs: when both waves of
    // a SIMD are ready, the one holding the matrix pipe keeps it (measured
    // 0.5-5 % faster, bitwise equal).
    __builtin_amdgcn_s_setprio(1);
    pv(vs, 0, p0);
#pragma unroll
    for (int j = 0; j < QB; ++j) p1[j] = probs(s1.s[j], -m_run[j]);
    if constexpr (QB == 1) {
      // The P V MFMAs of block 0, each with its two V^T reads and a share of
      // block 1's softmax VALU work.
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, SGB_VALU, 0);
      }
    }
#pragma unroll
    for (int j = 0; j < QB; ++j) {
      if (__builtin_amdgcn_ballot_w64(!(p1[j].sum <= kSumLimit))) p1[j] = resync(j, s1.s[j]);
      l_run[j] += p1[j].sum;
    }
    pv(vs, 1, p1);
    __builtin_amdgcn_s_setprio(0);
  };

  // Tiles are prefetched NSTAGE - 1 ahead into a ring of LDS stages. Step t
  // (on stage (t - t_begin) % NSTAGE, a compile-time constant so LDS offsets
  // are immediates) issues tile t + NSTAGE - 1 into the stage freed by step
  // t - 1, consumes tile t, then waits until tile t + 1 has landed (the
  // DMAs of later tiles may stay in flight) before the workgroup barrier.
  // Tiles [f_begin, f_end) need no masking for any query of the workgroup
  // and run the unmasked body; the rest (causal diagonal, window edges,
  // ragged end) run the masked body.
  static_assert(NSTAGE == 2 || NSTAGE == 3, "two or three LDS stages");
  constexpr int DMA_PER_STEP = 2 * CPW;  // K and V chunks issued by each wave
  auto step = [&](int t, auto stage_tag, auto mask_tag) __attribute__((always_inline)) {
    constexpr int STG = decltype(stage_tag)::value;
    const bool more = t + NSTAGE - 1 < t_end;
    if (more) issue(t + NSTAGE - 1, (STG + NSTAGE - 1) % NSTAGE);
    const int k0 = t * 64;
    bool skip = !wave_active || (CAUSAL && k0 > qw0 + WQ - 1 + off);
    if (WINDOW && wr >= 0) skip = skip || k0 > qw0 + WQ - 1 + off + wr;
    if (WINDOW && wl >= 0) skip = skip || k0 + 63 < qw0 + off - wl;
    if (!skip) {
      const unsigned char* ks = smem + STG * STAGE;
      tile(ks, ks + TILE, k0, mask_tag);
    }
    if (more) wait_vmcnt<(NSTAGE - 2) * DMA_PER_STEP>();
    else wait_vmcnt<0>();
    barrier_keep_dma();
  };
  auto step_any = [&](int t, auto mask_tag) __attribute__((always_inline)) {
    const int stg = (t - t_begin) % NSTAGE;
    if (stg == 0) step(t, std::integral_constant<int, 0>{}, mask_tag);
    else if (NSTAGE > 1 && stg == 1) step(t, std::integral_constant<int, 1 % NSTAGE>{}, mask_tag);
    else step(t, std::integral_constant<int, 2 % NSTAGE>{}, mask_tag);
  };
  // Full tiles: every key of the tile visible to every query of the workgroup.
  int full_hi = Nk - 1;                                 // last key that may be in a full tile
  if (CAUSAL) full_hi = min(full_hi, q0 + off);
  if (WINDOW && wr >= 0) full_hi = min(full_hi, q0 + off + wr);
  int f_begin = t_begin;
  if (WINDOW && wl >= 0) f_begin = max(t_begin, (max(q_last + off - wl, 0) + 63) / 64);
  int f_end = full_hi >= 0 ? (full_hi + 1) / 64 : 0;
  f_end = max(min(f_end, t_end), f_begin);
  f_begin = min(f_begin, t_end);

  if constexpr (BSPARSE) {
    // Active key tiles of this query block, in order: wave 0 scans the mask
    // row 64 blocks at a time (ballot + prefix count) and writes the two
    // 64-key tiles of every active block to an LDS list; tiles at or past
    // t_end (beyond the causal diagonal or N) are dropped.
    constexpr int LIST_OFF = NSTAGE * STAGE;
    unsigned short* list = reinterpret_cast<unsigned short*>(smem + LIST_OFF);
    int* count_slot = reinterpret_cast<int*>(smem + LIST_OFF + 2 * 2 * kBlockSparseMaxBlocks);
    if (wave == 0) {
      const uint8_t* mrow = seq.block_mask + ((int64_t)b * Hq + hq) * seq.mask_stride + (int64_t)qt * seq.nbk;
      const int blk_hi = min(seq.nbk, (t_end + 1) / 2);
      int cnt = 0;
      for (int c0 = 0; c0 < blk_hi; c0 += 64) {
        const int blk = c0 + lane;
        const bool act = blk < blk_hi && mrow[blk] != 0;
        const uint64_t bal = __builtin_amdgcn_ballot_w64(act);
        const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
        if (act) {
          list[cnt + 2 * below] = (unsigned short)(2 * blk);
          list[cnt + 2 * below + 1] = (unsigned short)(2 * blk + 1);
        }
        cnt += 2 * __builtin_popcountll(bal);
      }
      // Only the last block's second tile can lie past the end (its first
      // tile 2*blk <= t_end - 1 since blk < (t_end + 1) / 2). The list was
      // written by this wave, so its LDS writes are visible to this read.
      if (cnt > 0 && (int)list[cnt - 1] >= t_end) --cnt;
      if (lane == 0) *count_slot = cnt;
    }
    __syncthreads();
    const int n_act = uniform(*count_slot);
    auto tile_at = [&](int i) __attribute__((always_inline)) { return uniform((int)list[i]); };
    auto bs_step = [&](int i, auto stage_tag, auto mask_tag) __attribute__((always_inline)) {
      constexpr int STG = decltype(stage_tag)::value;
      const bool more = i + NSTAGE - 1 < n_act;
      if (more) issue(tile_at(i + NSTAGE - 1), (STG + NSTAGE - 1) % NSTAGE);
      const int tt = tile_at(i);
      const int k0 = tt * 64;
      const bool skip = !wave_active || (CAUSAL && k0 > qw0 + WQ - 1 + off);
      if (!skip) {
        const unsigned char* ks = smem + STG * STAGE;
        tile(ks, ks + TILE, k0, mask_tag);
      }
      if (more) wait_vmcnt<(NSTAGE - 2) * DMA_PER_STEP>();
      else wait_vmcnt<0>();
      barrier_keep_dma();
    };
    auto bs_any = [&](int i) __attribute__((always_inline)) {
      const int tt = tile_at(i);
      const bool full = tt < f_end;
      const int stg = i % NSTAGE;
      if (stg == 0) {
        if (full) bs_step(i, std::integral_constant<int, 0>{}, std::false_type{});
        else bs_step(i, std::integral_constant<int, 0>{}, std::true_type{});
      } else {
        if (full) bs_step(i, std::integral_constant<int, 1 % NSTAGE>{}, std::false_type{});
        else bs_step(i, std::integral_constant<int, 1 % NSTAGE>{}, std::true_type{});
      }
    };
    static_assert(NSTAGE == 2, "block-sparse list walk uses two stages");
#pragma unroll
    for (int i = 0; i < NSTAGE - 1; ++i) {
      if (i < n_act) issue(tile_at(i), i);
    }
    wait_vmcnt<0>();
    barrier_keep_dma();
    for (int i = 0; i < n_act; ++i) bs_any(i);
  } else {
#pragma unroll
  for (int i = 0; i < NSTAGE - 1; ++i) {
    if (t_begin + i < t_end) issue(t_begin + i, i);
  }
  wait_vmcnt<0>();
  barrier_keep_dma();
  int t = t_begin;
  for (; t < f_begin; ++t) step_any(t, std::true_type{});
  for (; t < f_end && (t - t_begin) % NSTAGE != 0; ++t) step_any(t, std::false_type{});
  for (; t + NSTAGE <= f_end; t += NSTAGE) {
    step(t, std::integral_constant<int, 0>{}, std::false_type{});
    step(t + 1, std::integral_constant<int, 1 % NSTAGE>{}, std::false_type{});
    if constexpr (NSTAGE == 3) step(t + 2, std::integral_constant<int, 2>{}, std::false_type{});
  }
  for (; t < f_end; ++t) step_any(t, std::false_type{});
  for (; t < t_end; ++t) step_any(t, std::true_type{});
  }

  if (!wave_active) return;
  const int64_t lse_base = VARLEN ? (int64_t)hq * seq.total_q + q_start : ((int64_t)b * Hq + hq) * N;
  if constexpr (QB == 1) {
    // The wave's 32 x 128 output tile goes out through LDS (the tile ring is
    // free: every wave has passed the last barrier), so the global stores
    // are 16 bytes per lane over whole 256-byte rows instead of 8-byte
    // pieces of 32 rows. Lane (l32, hh) holds row l32, dims 32 db + 8 i +
    // 4 hh .. + 3; unit u = 4 db + i of the row lands at u ^ tile_swz(row).
    const float l_tot = pair_sum(l_run[0]);
    const bool empty = !(l_tot > 0.f);
    const float inv = empty ? 0.f : 1.f / l_tot;
    unsigned char* ot = smem + wave * 32 * ROWB;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        u32x2 w;
        w[0] = pack_bf16x2(oacc[0][db][4 * i + 0] * inv, oacc[0][db][4 * i + 1] * inv);
        w[1] = pack_bf16x2(oacc[0][db][4 * i + 2] * inv, oacc[0][db][4 * i + 3] * inv);
        *reinterpret_cast<u32x2*>(ot + l32 * ROWB + 16 * ((4 * db + i) ^ row_swz<D>(l32)) + 8 * hh) = w;
      }
    }
    constexpr int UNITS = D / 8;              // 16-byte units per row
    constexpr int RPI = 64 / UNITS;           // rows per wave instruction
    const int unit = lane % UNITS;
#pragma unroll
    for (int c = 0; c < 32 / RPI; ++c) {
      const int row = RPI * c + lane / UNITS;
      const u32x4 val = *reinterpret_cast<const u32x4*>(ot + row * ROWB + 16 * (unit ^ row_swz<D>(row)));
      if (qw0 + row < Nq)
        *reinterpret_cast<u32x4*>(o + ((int64_t)q_start + qw0 + row) * q_rs + (int64_t)hq * D + 8 * unit) = val;
    }
    if (hh == 0 && my_q[0] < Nq) lse[lse_base + my_q[0]] = empty ? kNegInf : (m_run[0] + __log2f(l_tot)) * kLn2;
    return;
  }
#pragma unroll
  for (int j = 0; j < QB; ++j) {
    const float l_tot = pair_sum(l_run[j]);
    if (my_q[j] < Nq) {
      const bool empty = !(l_tot > 0.f);
      const float inv = empty ? 0.f : 1.f / l_tot;
      __bf16* orow = o + ((int64_t)q_start + my_q[j]) * q_rs + (int64_t)hq * D;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          u32x2 w;
          w[0] = pack_bf16x2(oacc[j][db][4 * i + 0] * inv, oacc[j][db][4 * i + 1] * inv);
          w[1] = pack_bf16x2(oacc[j][db][4 * i + 2] * inv, oacc[j][db][4 * i + 3] * inv);
          *reinterpret_cast<u32x2*>(orow + db * 32 + 8 * i + 4 * hh) = w;
        }
      }
      if (hh == 0) lse[lse_base + my_q[j]] = empty ? kNegInf : (m_run[j] + __log2f(l_tot)) * kLn2;
    }
  }
}

// fp32 path: eight query rows per wave, eight lanes per row. Each lane keeps
// D / 8 consecutive dimensions of its row's query and output accumulator; a
// score is the sum of the eight lanes' partial dot products (xor shuffles
// inside the lane group), so every lane of the group holds the same score and
// softmax state. 32-key tiles of K and V are staged in LDS.
template <int D>
__global__ __launch_bounds__(256) void fwd_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    float* __restrict__ o, float* __restrict__ lse, int B, int Hq, int Hkv, int N, float scale_log2,
    int causal, int num_q_tiles) {
  constexpr int LP = 8, DL = D / LP;  // lanes per row, dimensions per lane
  constexpr int BMQ = 32;             // query rows per workgroup (4 waves x 8)
  constexpr int TK = 32;
  __shared__ __align__(16) float ks[TK][D];
  __shared__ __align__(16) float vs[TK][D];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int part = lane % LP;
  const int bh = blockIdx.x % (B * Hq);
  const int qt = blockIdx.x / (B * Hq);
  const int b = bh / Hq, hq = bh % Hq, hk = hq / (Hq / Hkv);
  const int my_q = qt * BMQ + wave * (64 / LP) + lane / LP;
  const int64_t qs = (int64_t)Hq * D, kvs = (int64_t)Hkv * D;
  const float* qrow = q + ((int64_t)b * N + min(my_q, N - 1)) * qs + (int64_t)hq * D + part * DL;
  float qr[DL], acc[DL];
#pragma unroll
  for (int c = 0; c < DL; ++c) { qr[c] = qrow[c]; acc[c] = 0.f; }
  float m_run = kNegInf, l_run = 0.f;
  int kv_end = N;
  if (causal) kv_end = min(N, qt * BMQ + BMQ);
  for (int k0 = 0; k0 < kv_end; k0 += TK) {
    __syncthreads();
    for (int i = tid; i < TK * D / 4; i += 256) {
      const int r = i / (D / 4), c4 = i % (D / 4);
      const int key = k0 + r;
      const int64_t off = ((int64_t)b * N + min(key, N - 1)) * kvs + (int64_t)hk * D + 4 * c4;
      const float4 kv4 = *reinterpret_cast<const float4*>(k + off);
      const float4 vv4 = *reinterpret_cast<const float4*>(v + off);
      *reinterpret_cast<float4*>(&ks[r][4 * c4]) = key < N ? kv4 : float4{0.f, 0.f, 0.f, 0.f};
      *reinterpret_cast<float4*>(&vs[r][4 * c4]) = key < N ? vv4 : float4{0.f, 0.f, 0.f, 0.f};
    }
    __syncthreads();
    float s[TK];
    float mt = kNegInf;
#pragma unroll
    for (int j = 0; j < TK; ++j) {
      float dot = 0.f;
#pragma unroll
      for (int c = 0; c < DL; ++c) dot = fmaf(qr[c], ks[j][part * DL + c], dot);
#pragma unroll
      for (int w = 1; w < LP; w <<= 1) dot += __shfl_xor(dot, w, 64);
      const int key = k0 + j;
      const bool masked = key >= N || (causal && key > my_q);
      s[j] = masked ? kNegInf : dot * scale_log2;
      mt = fmaxf(mt, s[j]);
    }
    const float m_new = fmaxf(m_run, mt);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int c = 0; c < DL; ++c) acc[c] *= alpha;
#pragma unroll
    for (int j = 0; j < TK; ++j) {
      const float p = exp2f(s[j] - m_use);
      l_run += p;
#pragma unroll
      for (int c = 0; c < DL; ++c) acc[c] = fmaf(p, vs[j][part * DL + c], acc[c]);
    }
  }
  if (my_q < N) {
    const bool empty = !(l_run > 0.f);
    const float inv = empty ? 0.f : 1.f / l_run;
    float* orow = o + ((int64_t)b * N + my_q) * qs + (int64_t)hq * D + part * DL;
#pragma unroll
    for (int c = 0; c < DL; ++c) orow[c] = acc[c] * inv;
    if (part == 0) lse[((int64_t)b * Hq + hq) * N + my_q] = empty ? kNegInf : (m_run + log2f(l_run)) * kLn2;
  }
}

template <int NWAVES, int NSTAGE, int QB, bool CAUSAL, int MODE = 0, int D = 128>
hipError_t launch_d128(const FwdArgs& a, const FwdSeq& seq = FwdSeq{}) {
  constexpr int BM = NWAVES * 32 * QB;
  const int rows = (MODE & kModeVarlen) ? seq.max_q : a.N;
  const int num_q_tiles = (rows + BM - 1) / BM;
  const int64_t grid = (int64_t)num_q_tiles * a.B * a.Hq;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  // Tile ring, then (QB > 1) one 4 KB rescale slot per wave or (block-sparse)
  // the active-tile list and its count.
  constexpr size_t smem = (size_t)NSTAGE * 2 * 64 * 2 * D + (QB > 1 ? NWAVES * 4096 : 0) +
                          ((MODE & kModeBlockSparse) ? 2 * 2 * kBlockSparseMaxBlocks + 16 : 0);
  auto kern = fwd_d128_kernel<NWAVES, NSTAGE, QB, CAUSAL, MODE, D>;
  hipError_t e = set_smem_once<fwd_d128_kernel<NWAVES, NSTAGE, QB, CAUSAL, MODE, D>>(smem);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(NWAVES * 64), smem, a.stream,
                     (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v, (__bf16*)a.o, a.lse,
                     a.B, a.Hq, a.Hkv, a.N, a.scale * kLog2e, num_q_tiles, seq);
  return hipGetLastError();
}

template <bool CAUSAL>
hipError_t launch_splitk64(const FwdArgs& a) {
  const int num_q_tiles = (a.N + 31) / 32;
  const int64_t grid = (int64_t)num_q_tiles * a.B * a.Hq;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  constexpr size_t smem = 2 * 2 * FwdSmem<64, 4>::STAGE_ELEMS * 2;
  auto kern = fwd_splitk_d64_kernel<CAUSAL>;
  hipError_t e = set_smem_once<fwd_splitk_d64_kernel<CAUSAL>>(smem);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), smem, a.stream, (const __bf16*)a.q, (const __bf16*)a.k,
                     (const __bf16*)a.v, (__bf16*)a.o, a.lse, a.B, a.Hq, a.Hkv, a.N, a.scale * kLog2e, num_q_tiles);
  return hipGetLastError();
}

template <int D>
hipError_t launch_f32(const FwdArgs& a) {
  const int num_q_tiles = (a.N + 31) / 32;
  const int64_t grid = (int64_t)num_q_tiles * a.B * a.Hq;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(fwd_f32_kernel<D>, dim3((unsigned)grid), dim3(256), 0, a.stream,
                     (const float*)a.q, (const float*)a.k, (const float*)a.v, (float*)a.o, a.lse,
                     a.B, a.Hq, a.Hkv, a.N, a.scale * kLog2e, a.causal, num_q_tiles);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd(const FwdArgs& a) {
  if (a.dtype == kDtypeF32) {
    return a.d == 64 ? launch_f32<64>(a) : launch_f32<128>(a);
  }
  if (a.d == 64) {
    // Fewer 128-row workgroups than a launch needs to cover the CUs: split the
    // key range over the waves of 32-row workgroups instead (measured 1.2-1.7x
    // faster at B=2, H=8, N=1024; 2x slower than the 128-row kernel once the
    // grid is large, where the split quadruples the K/V reads per query).
    // Otherwise the DMA kernel of d = 128 with 128-byte rows (161 registers,
    // so three workgroups share a CU).
    if ((int64_t)a.B * a.Hq * ((a.N + 127) / 128) <= kSplitKMaxWorkgroups)
      return a.causal ? launch_splitk64<true>(a) : launch_splitk64<false>(a);
    return a.causal ? launch_d128<4, 2, 1, true, 0, 64>(a) : launch_d128<4, 2, 1, false, 0, 64>(a);
  }
  return a.causal ? launch_d128<4, 2, 1, true>(a) : launch_d128<4, 2, 1, false>(a);
}

// The masked modes (block-sparse, varlen, window) run the DMA kernel at
// either head dim (at d = 64 with 128-byte rows, as dense batches of many
// workgroups do).
template <int MODE>
hipError_t launch_mode(const FwdArgs& a, const FwdSeq& seq) {
  if (a.d == 64) return a.causal ? launch_d128<4, 2, 1, true, MODE, 64>(a, seq) : launch_d128<4, 2, 1, false, MODE, 64>(a, seq);
  return a.causal ? launch_d128<4, 2, 1, true, MODE>(a, seq) : launch_d128<4, 2, 1, false, MODE>(a, seq);
}

hipError_t launch_fwd_blocksparse(const FwdArgs& a, const FwdSeq& seq) { return launch_mode<kModeBlockSparse>(a, seq); }

hipError_t launch_fwd_seq(const FwdArgs& a, const FwdSeq& seq) {
  const bool varlen = seq.cu_q != nullptr;
  const bool window = seq.win_left >= 0 || seq.win_right >= 0;
  if (varlen && window) return launch_mode<kModeVarlen | kModeWindow>(a, seq);
  if (varlen) return launch_mode<kModeVarlen>(a, seq);
  if (window) return launch_mode<kModeWindow>(a, seq);
  return launch_fwd(a);
}

}  // namespace fa
