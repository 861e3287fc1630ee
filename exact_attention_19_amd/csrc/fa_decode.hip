// KV-cache decode kernels for gfx950 (MI355X): split-KV partials, then an
// LSE-weighted merge.
//
// One new query token per sequence attends the first L_b rows of that
// sequence's cache (flash_attn_with_kvcache in the hysenlabs digest of the
// flash-attention README, "出力と運用記録"; the v2.2 changelog entry there
// optimises inference with short queries). The work is memory bound: every
// K/V byte is read once and serves all query heads of its group.
//
// Split kernel: workgroup = (sequence b, kv head, group of GP query heads,
// chunk s of `chunk` cache rows). Lanes are grouped by LPT = D/8 lanes per
// cache row (16 bytes each), so a wave reads 64/LPT whole rows per load.
// Each row group keeps its own online-softmax state (running max, sum and
// an output slice), the states of all row groups of the workgroup are merged
// through LDS, and the chunk's (O_s, LSE_s) partial goes to the workspace.
// The merge kernel combines the partials of a (b, query head):
//   LSE = log sum_s exp(LSE_s),  O = sum_s exp(LSE_s - LSE) O_s,
// which is the same running-max/sum recurrence as the online softmax of
// the Qiita FlashAttention tutorial (section 4.3), applied once across chunks.
#include <algorithm>
#include <atomic>

#include "fa_common.h"
#include "fa_internal.h"

namespace fa {

namespace {

constexpr int kDecThreads = 256;
constexpr int kDecWaves = kDecThreads / 64;
constexpr int kDecUnroll = 8;  // cache rows per row group per iteration
constexpr int kWideUnroll = 8;  // rows per wave per iteration (wide-row kernels)

template <int D, int GP>
struct DecSmem {
  static constexpr int LPT = D / 8;
  static constexpr int RPW = 64 / LPT;                  // row groups per wave
  static constexpr int NSTATE = kDecWaves * RPW;        // partial states per workgroup
  static constexpr int BYTES = NSTATE * GP * (D + 2) * 4;
};

// Paged-cache geometry for the split kernel (unused for a contiguous cache).
struct PageMap {
  const int32_t* table;  // [B, max_pages]
  int shift;             // log2(page_size)
  int max_pages;
  int num_pages;
};

// In-place append (flash_attn_with_kvcache updates k_cache / v_cache in
// place: hysenlabs digest, outputs section): row seqlens[b] of sequence b
// receives k_new[b], v_new[b]; positions outside [0, N) are skipped. One
// thread copies 16 bytes of one (b, kv head) row of K and of V.
template <int D, bool PAGED>
__global__ __launch_bounds__(256) void decode_append_kernel(
    __bf16* __restrict__ kc, __bf16* __restrict__ vc, const __bf16* __restrict__ k_new,
    const __bf16* __restrict__ v_new, const int32_t* __restrict__ seqlens, PageMap pm, int B, int Hkv, int N) {
  constexpr int PER_ROW = D / 8;
  const int64_t gt = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gt >= (int64_t)B * Hkv * PER_ROW) return;
  const int c = (int)(gt % PER_ROW);
  const int bh = (int)(gt / PER_ROW);
  const int b = bh / Hkv, hk = bh % Hkv;
  const int pos = seqlens[b];
  if (pos < 0 || pos >= N) return;
  int64_t row;
  if constexpr (PAGED) {
    const int page = min(max(pm.table[(int64_t)b * pm.max_pages + (pos >> pm.shift)], 0), pm.num_pages - 1);
    row = ((int64_t)page << pm.shift) + (pos & ((1 << pm.shift) - 1));
  } else {
    row = (int64_t)b * N + pos;
  }
  const int64_t dst = (row * Hkv + hk) * D + c * 8;
  const int64_t src = ((int64_t)b * Hkv + hk) * D + c * 8;
  *reinterpret_cast<u32x4*>(kc + dst) = *reinterpret_cast<const u32x4*>(k_new + src);
  *reinterpret_cast<u32x4*>(vc + dst) = *reinterpret_cast<const u32x4*>(v_new + src);
}

// Chunk rows are at most this many pages long in the paged split kernel
// (chunks of <= kDecodeDefaultChunk = 1024 rows, pages of >= 16 rows, plus
// one partial page).
constexpr int kDecMaxChunkPages = 128;
static_assert(kDecodeDefaultChunk / 16 + 1 <= kDecMaxChunkPages, "page list too small");

template <int D, int GP, bool PAGED>
__global__ __launch_bounds__(kDecThreads) void decode_split_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ kc, const __bf16* __restrict__ vc,
    const int32_t* __restrict__ seqlens, float* __restrict__ part_o, float* __restrict__ part_lse,
    int B, int Hq, int Hkv, int Lmax, int chunk, int nsplit, float scale_log2, int append, PageMap pm) {
  constexpr int LPT = D / 8;
  constexpr int RPW = 64 / LPT;
  constexpr int NSTATE = DecSmem<D, GP>::NSTATE;
  __shared__ float sm_m[NSTATE][GP];
  __shared__ float sm_l[NSTATE][GP];
  __shared__ float sm_o[NSTATE][GP][D];
  __shared__ int sm_page[PAGED ? kDecMaxChunkPages : 1];

  const int HG = Hq / GP;
  const int bid = blockIdx.x;
  const int hg = bid % HG;
  const int s = (bid / HG) % nsplit;
  const int b = bid / (HG * nsplit);
  const int L = seqlens[b] + append;
  if (L < 1 || L > Lmax) return;
  const int start = s * chunk;
  if (start >= L) return;
  const int end = min(L, start + chunk);
  const int first_page = PAGED ? (start >> pm.shift) : 0;
  if constexpr (PAGED) {
    const int n_pages = ((end - 1) >> pm.shift) - first_page + 1;
    for (int i = threadIdx.x; i < n_pages; i += kDecThreads)
      sm_page[i] = min(max(pm.table[(int64_t)b * pm.max_pages + first_page + i], 0), pm.num_pages - 1);
    __syncthreads();
  }
  const int h0 = hg * GP;                // first query head of this workgroup
  const int hk = h0 / (Hq / Hkv);        // its kv head (GP divides the group size)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int rg = lane / LPT;             // row group within the wave
  const int dl = lane % LPT;             // 16-byte slice of the row
  const int state = wave * RPW + rg;

  u32x4 qv[GP];
#pragma unroll
  for (int g = 0; g < GP; ++g) {
    qv[g] = *reinterpret_cast<const u32x4*>(q + ((int64_t)b * Hq + h0 + g) * D + dl * 8);
  }

  const int64_t row_stride = (int64_t)Hkv * D;
  const int64_t seq_rows = PAGED ? 0 : (int64_t)b * Lmax;
  const __bf16* kbase = kc + seq_rows * row_stride + (int64_t)hk * D + dl * 8;
  const __bf16* vbase = vc + seq_rows * row_stride + (int64_t)hk * D + dl * 8;
  // Storage row of logical row `row` of this sequence.
  auto phys = [&](int row) -> int64_t {
    if constexpr (PAGED) {
      return ((int64_t)sm_page[(row >> pm.shift) - first_page] << pm.shift) + (row & ((1 << pm.shift) - 1));
    } else {
      return row;
    }
  };

  float m[GP], l[GP], acc[GP][8];
#pragma unroll
  for (int g = 0; g < GP; ++g) {
    m[g] = kNegInf;
    l[g] = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[g][c] = 0.f;
  }

  constexpr int ROWS_PER_ITER = kDecWaves * RPW * kDecUnroll;
  u32x4 kr[kDecUnroll], vr[kDecUnroll];
  // Rows past the chunk end are read as the chunk's last row (never past
  // L_b - 1); their scores are masked to -inf, so they weigh exactly 0.
  auto load = [&](int base) {
#pragma unroll
    for (int u = 0; u < kDecUnroll; ++u) {
      const int64_t row = phys(min(base + u * kDecWaves * RPW + state, end - 1));
      kr[u] = *reinterpret_cast<const u32x4*>(kbase + row * row_stride);
      vr[u] = *reinterpret_cast<const u32x4*>(vbase + row * row_stride);
    }
  };

  load(start);
  for (int base = start; base < end; base += ROWS_PER_ITER) {
    u32x4 kcur[kDecUnroll], vcur[kDecUnroll];
#pragma unroll
    for (int u = 0; u < kDecUnroll; ++u) { kcur[u] = kr[u]; vcur[u] = vr[u]; }
    if (base + ROWS_PER_ITER < end) load(base + ROWS_PER_ITER);

    float sc[kDecUnroll][GP];
#pragma unroll
    for (int u = 0; u < kDecUnroll; ++u) {
      const int row = base + u * kDecWaves * RPW + state;
      const bool ok = row < end;
#pragma unroll
      for (int g = 0; g < GP; ++g) {
        const float part = dot8_bf16(qv[g], kcur[u], 0.f);
        const float tot = row_group_sum<LPT>(part);
        sc[u][g] = ok ? tot * scale_log2 : kNegInf;
      }
    }
#pragma unroll
    for (int g = 0; g < GP; ++g) {
      float mb = sc[0][g];
#pragma unroll
      for (int u = 1; u < kDecUnroll; ++u) mb = fmaxf(mb, sc[u][g]);
      const float m_new = fmaxf(m[g], mb);
      const float m_use = (m_new == kNegInf) ? 0.f : m_new;
      const float alpha = fast_exp2(m[g] - m_use);
      m[g] = m_new;
      l[g] *= alpha;
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[g][c] *= alpha;
#pragma unroll
      for (int u = 0; u < kDecUnroll; ++u) {
        const float p = fast_exp2(sc[u][g] - m_use);
        l[g] += p;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          acc[g][2 * w] = fmaf(p, bf16_lo(vcur[u][w]), acc[g][2 * w]);
          acc[g][2 * w + 1] = fmaf(p, bf16_hi(vcur[u][w]), acc[g][2 * w + 1]);
        }
      }
    }
  }

  // Merge the NSTATE row-group states through LDS.
#pragma unroll
  for (int g = 0; g < GP; ++g) {
    if (dl == 0) {
      sm_m[state][g] = m[g];
      sm_l[state][g] = l[g];
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) sm_o[state][g][dl * 8 + c] = acc[g][c];
  }
  __syncthreads();
  for (int idx = tid; idx < GP * D; idx += kDecThreads) {
    const int g = idx / D, d = idx % D;
    float mm = kNegInf;
    for (int st = 0; st < NSTATE; ++st) mm = fmaxf(mm, sm_m[st][g]);
    float wsum = 0.f, osum = 0.f;
    for (int st = 0; st < NSTATE; ++st) {
      const float w = fast_exp2(sm_m[st][g] - mm);  // states without rows have m = -inf: weight 0
      wsum = fmaf(w, sm_l[st][g], wsum);
      osum = fmaf(w, sm_o[st][g][d], osum);
    }
    const int64_t ps = ((int64_t)b * Hq + h0 + g) * nsplit + s;
    part_o[ps * D + d] = osum / wsum;
    if (d == 0) part_lse[ps] = mm + __log2f(wsum);  // log2 units
  }
}

// Wide-row layout: one wave instruction reads the 16-byte slices of
// HPW = 64 / LPT consecutive kv heads of one cache row (1 KB contiguous for
// d = 128). A streaming read in this layout runs at full HBM speed, while
// one head's 256-byte slice per instruction (rows 2 KB apart) measured ~7 %
// slower. Lane group j (LPT lanes) serves kv head HPW * blk + j and GP of
// its query heads; wave w takes rows start + w, start + w + 4, ...
template <int GP>
struct DecState {
  float m[GP], l[GP], acc[GP][8];  // running max (log2 units), exp-sum, 8 output dims
};

template <int GP>
__device__ __forceinline__ void dec_state_init(DecState<GP>& st) {
#pragma unroll
  for (int g = 0; g < GP; ++g) {
    st.m[g] = kNegInf;
    st.l[g] = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) st.acc[g][c] = 0.f;
  }
}

// Rows [start, end) of one sequence into the lane's state. kbase/vbase point
// at this lane's 16 bytes of storage row 0; phys maps a logical row to its
// storage row. Rows past `end` are read as row end - 1 and weigh exactly 0.
template <int D, int GP, typename Phys>
__device__ __forceinline__ void wide_rows(DecState<GP>& st, const u32x4 (&qv)[GP], const __bf16* kbase,
                                          const __bf16* vbase, int64_t row_stride, int start, int end, int wave,
                                          float scale_log2, const Phys& phys) {
  constexpr int LPT = D / 8;
  constexpr int ROWS_PER_ITER = kDecWaves * kWideUnroll;
  u32x4 kr[kWideUnroll], vr[kWideUnroll];
  auto load = [&](int base) {
#pragma unroll
    for (int u = 0; u < kWideUnroll; ++u) {
      const int64_t row = phys(min(base + u * kDecWaves + wave, end - 1));
      kr[u] = *reinterpret_cast<const u32x4*>(kbase + row * row_stride);
      vr[u] = *reinterpret_cast<const u32x4*>(vbase + row * row_stride);
    }
  };
  load(start);
  for (int base = start; base < end; base += ROWS_PER_ITER) {
    u32x4 kcur[kWideUnroll], vcur[kWideUnroll];
#pragma unroll
    for (int u = 0; u < kWideUnroll; ++u) { kcur[u] = kr[u]; vcur[u] = vr[u]; }
    if (base + ROWS_PER_ITER < end) load(base + ROWS_PER_ITER);

    float sc[kWideUnroll][GP];
#pragma unroll
    for (int u = 0; u < kWideUnroll; ++u) {
      const bool ok = base + u * kDecWaves + wave < end;
#pragma unroll
      for (int g = 0; g < GP; ++g) {
        const float tot = row_group_sum<LPT>(dot8_bf16(qv[g], kcur[u], 0.f));
        sc[u][g] = ok ? tot * scale_log2 : kNegInf;
      }
    }
#pragma unroll
    for (int g = 0; g < GP; ++g) {
      float mb = sc[0][g];
#pragma unroll
      for (int u = 1; u < kWideUnroll; ++u) mb = fmaxf(mb, sc[u][g]);
      const float m_new = fmaxf(st.m[g], mb);
      const float m_use = (m_new == kNegInf) ? 0.f : m_new;
      const float alpha = fast_exp2(st.m[g] - m_use);
      st.m[g] = m_new;
      st.l[g] *= alpha;
#pragma unroll
      for (int c = 0; c < 8; ++c) st.acc[g][c] *= alpha;
#pragma unroll
      for (int u = 0; u < kWideUnroll; ++u) {
        const float p = fast_exp2(sc[u][g] - m_use);
        st.l[g] += p;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          st.acc[g][2 * w] = fmaf(p, bf16_lo(vcur[u][w]), st.acc[g][2 * w]);
          st.acc[g][2 * w + 1] = fmaf(p, bf16_hi(vcur[u][w]), st.acc[g][2 * w + 1]);
        }
      }
    }
  }
}

// LDS for merging the four waves' states of each query head of a block.
template <int D, int GP>
struct WideMergeSmem {
  static constexpr int HPW = 512 / D;
  float m[kDecWaves][HPW][GP];
  float l[kDecWaves][HPW][GP];
  float o[kDecWaves][HPW][GP][D];
};

// Merges the four waves' states (LDS) and hands (j, g, d, O, LSE in log2
// units) to store for every output of the block; callers sync before reuse.
template <int D, int GP, typename Store>
__device__ __forceinline__ void wide_merge(WideMergeSmem<D, GP>& sm, const DecState<GP>& st, int wave, int j,
                                           int dl, const Store& store) {
  constexpr int HPW = 512 / D;
#pragma unroll
  for (int g = 0; g < GP; ++g) {
    if (dl == 0) {
      sm.m[wave][j][g] = st.m[g];
      sm.l[wave][j][g] = st.l[g];
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) sm.o[wave][j][g][dl * 8 + c] = st.acc[g][c];
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < HPW * GP * D; idx += kDecThreads) {
    const int jj = idx / (GP * D), g = (idx / D) % GP, d = idx % D;
    float mm = kNegInf;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) mm = fmaxf(mm, sm.m[w][jj][g]);
    float wsum = 0.f, osum = 0.f;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) {
      const float wt = fast_exp2(sm.m[w][jj][g] - mm);  // waves without rows have m = -inf: weight 0
      wsum = fmaf(wt, sm.l[w][jj][g], wsum);
      osum = fmaf(wt, sm.o[w][jj][g][d], osum);
    }
    store(jj, g, d, osum / wsum, mm + __log2f(wsum));
  }
}

// Split kernel in the wide-row layout with fixed chunks: workgroup =
// (sequence b, block of HPW kv heads, group of GP query heads per kv head,
// chunk s of cache rows). Used with an explicit split count when HPW
// divides Hkv.
template <int D, int GP, bool PAGED>
__global__ __launch_bounds__(kDecThreads) void decode_split_wide_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ kc, const __bf16* __restrict__ vc,
    const int32_t* __restrict__ seqlens, float* __restrict__ part_o, float* __restrict__ part_lse,
    int B, int Hq, int Hkv, int Lmax, int chunk, int nsplit, float scale_log2, int append, PageMap pm) {
  constexpr int LPT = D / 8;
  constexpr int HPW = 64 / LPT;
  __shared__ WideMergeSmem<D, GP> sm;
  __shared__ int sm_page[PAGED ? kDecMaxChunkPages : 1];

  const int G = Hq / Hkv;
  const int QG = G / GP;
  const int NB = Hkv / HPW;
  const int bid = blockIdx.x;
  const int qg = bid % QG;
  const int blk = (bid / QG) % NB;
  const int s = (bid / (QG * NB)) % nsplit;
  const int b = bid / (QG * NB * nsplit);
  const int L = seqlens[b] + append;
  if (L < 1 || L > Lmax) return;
  const int start = s * chunk;
  if (start >= L) return;
  const int end = min(L, start + chunk);
  const int first_page = PAGED ? (start >> pm.shift) : 0;
  if constexpr (PAGED) {
    const int n_pages = ((end - 1) >> pm.shift) - first_page + 1;
    for (int i = threadIdx.x; i < n_pages; i += kDecThreads)
      sm_page[i] = min(max(pm.table[(int64_t)b * pm.max_pages + first_page + i], 0), pm.num_pages - 1);
    __syncthreads();
  }

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int j = lane / LPT, dl = lane % LPT;
  const int hq0 = (blk * HPW + j) * G + qg * GP;  // first query head of this lane group
  u32x4 qv[GP];
#pragma unroll
  for (int g = 0; g < GP; ++g) qv[g] = *reinterpret_cast<const u32x4*>(q + ((int64_t)b * Hq + hq0 + g) * D + dl * 8);

  const int64_t row_stride = (int64_t)Hkv * D;
  const int64_t seq_rows = PAGED ? 0 : (int64_t)b * Lmax;
  const __bf16* kbase = kc + seq_rows * row_stride + (int64_t)blk * HPW * D + lane * 8;
  const __bf16* vbase = vc + seq_rows * row_stride + (int64_t)blk * HPW * D + lane * 8;
  auto phys = [&](int row) -> int64_t {
    if constexpr (PAGED) {
      return ((int64_t)sm_page[(row >> pm.shift) - first_page] << pm.shift) + (row & ((1 << pm.shift) - 1));
    } else {
      return row;
    }
  };
  DecState<GP> st;
  dec_state_init(st);
  wide_rows<D, GP>(st, qv, kbase, vbase, row_stride, start, end, wave, scale_log2, phys);
  wide_merge<D, GP>(sm, st, wave, j, dl, [&](int jj, int g, int d, float ov, float lv) {
    const int64_t ps = ((int64_t)b * Hq + (blk * HPW + jj) * G + qg * GP + g) * nsplit + s;
    part_o[ps * D + d] = ov;
    if (d == 0) part_lse[ps] = lv;
  });
}

// Balanced split kernel (wide-row layout). The valid rows of all sequences,
// concatenated (R rows in total), are cut into P equal ranges, range p =
// [floor(p R / P), floor((p + 1) R / P)), and workgroup (p, block of HPW kv
// heads, group of GP query heads) takes range p: every workgroup reads the
// same number of bytes, whatever the mix of cache lengths. It writes one
// partial per sequence b its range overlaps, at slot p + b: along the
// concatenated rows the (range, sequence) overlaps form a monotone
// staircase, so the slots are distinct and those of sequence b are
// consecutive. Sequence prefix sums are built in LDS (B <= kDecBalMaxB);
// workgroup 0 also stores them for the merge kernel.
template <int D, int GP, bool PAGED>
__global__ __launch_bounds__(kDecThreads) void decode_split_bal_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ kc, const __bf16* __restrict__ vc,
    const int32_t* __restrict__ seqlens, float* __restrict__ part_o, float* __restrict__ part_lse,
    long long* __restrict__ cum_out, int B, int Hq, int Hkv, int Lmax, int P, float scale_log2, int append,
    PageMap pm) {
  constexpr int LPT = D / 8;
  constexpr int HPW = 64 / LPT;
  __shared__ WideMergeSmem<D, GP> sm;
  __shared__ long long sm_cum[kDecBalMaxB + 1];
  __shared__ long long sm_wsum[kDecWaves];
  __shared__ int sm_page[PAGED ? kDecMaxChunkPages : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  // Exclusive prefix sums of the valid lengths (invalid ones count 0).
  {
    int lv[4];
    long long loc = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = 4 * tid + i;
      int L = idx < B ? seqlens[idx] + append : 0;
      if (L < 1 || L > Lmax) L = 0;
      lv[i] = L;
      loc += L;
    }
    long long x = loc;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const long long y = __shfl_up(x, off, 64);
      if (lane >= off) x += y;
    }
    if (lane == 63) sm_wsum[wave] = x;
    __syncthreads();
    long long excl = x - loc;
    for (int w = 0; w < wave; ++w) excl += sm_wsum[w];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = 4 * tid + i;
      if (idx < B) sm_cum[idx] = excl;
      excl += lv[i];
    }
    if (tid == 0) {
      long long tot = 0;
      for (int w = 0; w < kDecWaves; ++w) tot += sm_wsum[w];
      sm_cum[B] = tot;
    }
    __syncthreads();
  }
  const int G = Hq / Hkv;
  const int QG = G / GP;
  const int NB = Hkv / HPW;
  const int NBQ = QG * NB;
  if (blockIdx.x == 0) {
    for (int i = tid; i <= B; i += kDecThreads) cum_out[i] = sm_cum[i];
  }
  const int bq = blockIdx.x % NBQ;
  const int p = blockIdx.x / NBQ;
  const int qg = bq % QG;
  const int blk = bq / QG;
  const long long R = sm_cum[B];
  const long long r0 = (long long)p * R / P;
  const long long r1 = (long long)(p + 1) * R / P;
  if (r0 >= r1) return;
  // Sequence holding row r0: the last b with cum[b] <= r0.
  int b = 0;
  {
    int lo = 0, hi = B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (sm_cum[mid] <= r0) lo = mid;
      else hi = mid - 1;
    }
    b = lo;
  }

  const int j = lane / LPT, dl = lane % LPT;
  const int hq0 = (blk * HPW + j) * G + qg * GP;
  const int64_t row_stride = (int64_t)Hkv * D;
  for (; b < B && sm_cum[b] < r1; ++b) {
    const long long c0 = sm_cum[b], c1 = sm_cum[b + 1];
    if (c1 == c0) continue;
    const int start = (int)(max(r0, c0) - c0);
    const int end = (int)(min(r1, c1) - c0);
    u32x4 qv[GP];
#pragma unroll
    for (int g = 0; g < GP; ++g) qv[g] = *reinterpret_cast<const u32x4*>(q + ((int64_t)b * Hq + hq0 + g) * D + dl * 8);
    const int64_t seq_rows = PAGED ? 0 : (int64_t)b * Lmax;
    const __bf16* kbase = kc + seq_rows * row_stride + (int64_t)blk * HPW * D + lane * 8;
    const __bf16* vbase = vc + seq_rows * row_stride + (int64_t)blk * HPW * D + lane * 8;
    DecState<GP> st;
    dec_state_init(st);
    if constexpr (PAGED) {
      // Page ids of at most kDecodeDefaultChunk rows at a time go to LDS.
      for (int c = start; c < end; c += kDecodeDefaultChunk) {
        const int ce = min(end, c + kDecodeDefaultChunk);
        const int first_page = c >> pm.shift;
        const int n_pages = ((ce - 1) >> pm.shift) - first_page + 1;
        __syncthreads();
        for (int i = tid; i < n_pages; i += kDecThreads)
          sm_page[i] = min(max(pm.table[(int64_t)b * pm.max_pages + first_page + i], 0), pm.num_pages - 1);
        __syncthreads();
        auto phys = [&](int row) -> int64_t {
          return ((int64_t)sm_page[(row >> pm.shift) - first_page] << pm.shift) + (row & ((1 << pm.shift) - 1));
        };
        wide_rows<D, GP>(st, qv, kbase, vbase, row_stride, c, ce, wave, scale_log2, phys);
      }
    } else {
      auto phys = [](int row) -> int64_t { return row; };
      wide_rows<D, GP>(st, qv, kbase, vbase, row_stride, start, end, wave, scale_log2, phys);
    }
    __syncthreads();  // the previous segment's merge has read the LDS states
    const int64_t slot = (int64_t)p + b;
    wide_merge<D, GP>(sm, st, wave, j, dl, [&](int jj, int g, int d, float ov, float lv) {
      const int64_t ps = slot * Hq + (blk * HPW + jj) * G + qg * GP + g;
      part_o[ps * D + d] = ov;
      if (d == 0) part_lse[ps] = lv;
    });
  }
}

// Merge for the balanced split: output (b, hq) combines the partials at
// slots p + b of the ranges p that overlap sequence b (empty ranges skipped).
// One wave: 64 slots at a time, lane i holding slot p_first + i; the LSE max
// and the weights come from wave reductions, and each lane then sums its
// D / 64 output dims over the slots with independent loads.
template <int D>
__global__ __launch_bounds__(64) void decode_merge_bal_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_lse, const long long* __restrict__ cum,
    __bf16* __restrict__ o, float* __restrict__ lse, int B, int Hq, int P) {
  constexpr int PER = D / 64;
  __shared__ float sm_w[64];
  const int bh = blockIdx.x;
  const int b = bh / Hq, hq = bh - b * Hq;
  const int tid = threadIdx.x;
  __bf16* orow = o + (int64_t)bh * D;
  const long long c0 = cum[b], c1 = cum[b + 1], R = cum[B];
  if (c1 <= c0) {
#pragma unroll
    for (int i = 0; i < PER; ++i) orow[tid * PER + i] = (__bf16)0.f;
    if (tid == 0 && lse) lse[bh] = kNegInf;
    return;
  }
  // Range p starts at floor(p R / P); the last p starting at or before c0
  // and the last p starting before c1.
  const int p_first = (int)min((long long)P - 1, ((c0 + 1) * P - 1) / R);
  const int p_last = (int)min((long long)P - 1, (c1 * P - 1) / R);
  auto r_of = [&](int p) { return (long long)p * R / P; };
  auto slot_lse = [&](int p) {  // -inf for ranges past p_last or empty
    if (p > p_last || r_of(p) == r_of(p + 1)) return kNegInf;
    return part_lse[((int64_t)p + b) * Hq + hq];
  };
  float mm = kNegInf;
  for (int p0 = p_first; p0 <= p_last; p0 += 64) mm = fmaxf(mm, slot_lse(p0 + tid));
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mm = fmaxf(mm, __shfl_xor(mm, off, 64));
  float wsum = 0.f;
  float os[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) os[i] = 0.f;
  for (int p0 = p_first; p0 <= p_last; p0 += 64) {
    const float w = fast_exp2(slot_lse(p0 + tid) - mm);  // 0 for empty or absent slots
    float ws = w;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) ws += __shfl_xor(ws, off, 64);
    wsum += ws;
    __syncthreads();
    sm_w[tid] = w;
    __syncthreads();
    const int n = min(64, p_last - p0 + 1);
    // Eight slots per batch, all loads issued before any is used. Indices
    // past n re-read slot n - 1 (in bounds) and get weight 0; a slot of
    // weight 0 (empty range, never written) is excluded by a select, so
    // whatever its memory holds cannot reach the sum.
    for (int i0 = 0; i0 < n; i0 += 8) {
      float v[8][PER];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = min(i0 + u, n - 1);
        const float* po = part_o + (((int64_t)p0 + i + b) * Hq + hq) * D + tid * PER;
#pragma unroll
        for (int e = 0; e < PER; ++e) v[u][e] = po[e];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float wi = i0 + u < n ? sm_w[i0 + u] : 0.f;
#pragma unroll
        for (int e = 0; e < PER; ++e) os[e] = wi != 0.f ? fmaf(wi, v[u][e], os[e]) : os[e];
      }
    }
  }
  const float inv = 1.f / wsum;
#pragma unroll
  for (int i = 0; i < PER; ++i) orow[tid * PER + i] = (__bf16)(os[i] * inv);
  if (tid == 0 && lse) lse[bh] = (mm + __log2f(wsum)) * kLn2;
}

template <int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_lse, const int32_t* __restrict__ seqlens,
    __bf16* __restrict__ o, float* __restrict__ lse, int B, int Hq, int Lmax, int chunk, int nsplit, int append) {
  constexpr int PER = D / 64;
  const int bh = blockIdx.x;
  const int b = bh / Hq;
  const int tid = threadIdx.x;
  const int L = seqlens[b] + append;
  __bf16* orow = o + (int64_t)bh * D;
  if (L < 1 || L > Lmax) {
#pragma unroll
    for (int i = 0; i < PER; ++i) orow[tid * PER + i] = (__bf16)0.f;
    if (tid == 0 && lse) lse[bh] = kNegInf;
    return;
  }
  const int n = (L + chunk - 1) / chunk;
  const float* pl = part_lse + (int64_t)bh * nsplit;
  const float* po = part_o + (int64_t)bh * nsplit * D;
  float mm = kNegInf;
  for (int s = tid; s < n; s += 64) mm = fmaxf(mm, pl[s]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mm = fmaxf(mm, __shfl_xor(mm, off, 64));
  float wsum = 0.f;
  float os[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) os[i] = 0.f;
  for (int s = 0; s < n; ++s) {
    const float w = fast_exp2(pl[s] - mm);
    wsum += w;
#pragma unroll
    for (int i = 0; i < PER; ++i) os[i] = fmaf(w, po[(int64_t)s * D + tid * PER + i], os[i]);
  }
  const float inv = 1.f / wsum;
#pragma unroll
  for (int i = 0; i < PER; ++i) orow[tid * PER + i] = (__bf16)(os[i] * inv);
  if (tid == 0 && lse) lse[bh] = (mm + __log2f(wsum)) * kLn2;
}

PageMap page_map(const DecodeArgs& a) {
  return PageMap{a.block_table, a.page_shift, a.max_pages, a.num_pages};
}

template <int D, int GP, bool PAGED>
hipError_t launch_split(const DecodeArgs& a, int chunk, int nsplit, float* part_o, float* part_lse) {
  const int64_t grid = (int64_t)a.B * nsplit * (a.Hq / GP);
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  constexpr int HPW = 512 / D;  // kv heads per wave instruction in the wide-row kernel
  if (a.Hkv % HPW == 0) {
    hipLaunchKernelGGL((decode_split_wide_kernel<D, GP, PAGED>), dim3((unsigned)(grid / HPW)), dim3(kDecThreads), 0,
                       a.stream, (const __bf16*)a.q, (const __bf16*)a.k_cache, (const __bf16*)a.v_cache, a.seqlens,
                       part_o, part_lse, a.B, a.Hq, a.Hkv, a.N, chunk, nsplit, a.scale * kLog2e,
                       a.k_new ? 1 : 0, page_map(a));
    return hipGetLastError();
  }
  hipLaunchKernelGGL((decode_split_kernel<D, GP, PAGED>), dim3((unsigned)grid), dim3(kDecThreads), 0, a.stream,
                     (const __bf16*)a.q, (const __bf16*)a.k_cache, (const __bf16*)a.v_cache, a.seqlens,
                     part_o, part_lse, a.B, a.Hq, a.Hkv, a.N, chunk, nsplit, a.scale * kLog2e,
                     a.k_new ? 1 : 0, page_map(a));
  return hipGetLastError();
}

template <int D, bool PAGED>
hipError_t launch_split_gp(const DecodeArgs& a, int gp, int chunk, int nsplit, float* po, float* pl) {
  switch (gp) {
    case 1: return launch_split<D, 1, PAGED>(a, chunk, nsplit, po, pl);
    case 2: return launch_split<D, 2, PAGED>(a, chunk, nsplit, po, pl);
    default: return launch_split<D, 4, PAGED>(a, chunk, nsplit, po, pl);
  }
}

template <int D, bool PAGED>
hipError_t launch_append(const DecodeArgs& a) {
  const int64_t threads = (int64_t)a.B * a.Hkv * (D / 8);
  const int64_t grid = (threads + 255) / 256;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((decode_append_kernel<D, PAGED>), dim3((unsigned)grid), dim3(256), 0, a.stream,
                     (__bf16*)a.k_cache, (__bf16*)a.v_cache, (const __bf16*)a.k_new, (const __bf16*)a.v_new,
                     a.seqlens, page_map(a), a.B, a.Hkv, a.N);
  return hipGetLastError();
}

}  // namespace

int decode_heads_per_group(int Hq, int Hkv) {
  const int g = Hq / Hkv;
  int gp = 1;
  while (gp * 2 <= kDecodeMaxHeadsPerGroup && g % (gp * 2) == 0) gp *= 2;
  return gp;
}

void decode_split_plan(int N, int num_splits, int* chunk, int* nsplit) {
  int ns = num_splits;
  if (ns <= 0) ns = (N + kDecodeDefaultChunk - 1) / kDecodeDefaultChunk;
  if (ns > N) ns = N;
  if (ns < 1) ns = 1;
  int c = (N + ns - 1) / ns;
  *chunk = c;
  *nsplit = (N + c - 1) / c;
}

namespace {

size_t round_up256(size_t x) { return (x + 255) / 256 * 256; }

// Partials of fa_decode_kvcache_noalloc: every call on a device shares this
// array, so calls that overlap on one device race. Host code never passes
// the array's name to a kernel (in host code it names a host-side stand-in);
// it uses the address looked up per device below.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];
std::atomic<void*> g_scratch_addr[kMaxDevices];

template <int D, int GP>
const void* bal_kernel_ptr() {
  return reinterpret_cast<const void*>(decode_split_bal_kernel<D, GP, false>);
}

// Resident workgroups of the balanced split kernel per CU, cached per device.
int bal_slots_per_cu(int dev, int d, int gp) {
  static std::atomic<int> cache[kMaxDevices][2][3];
  const int di = d == 64 ? 0 : 1, gi = gp == 1 ? 0 : (gp == 2 ? 1 : 2);
  if (dev < 0 || dev >= kMaxDevices) return 0;
  int v = cache[dev][di][gi].load(std::memory_order_relaxed);
  if (v > 0) return v;
  const void* k = d == 64 ? (gp == 1 ? bal_kernel_ptr<64, 1>() : gp == 2 ? bal_kernel_ptr<64, 2>() : bal_kernel_ptr<64, 4>())
                          : (gp == 1 ? bal_kernel_ptr<128, 1>() : gp == 2 ? bal_kernel_ptr<128, 2>() : bal_kernel_ptr<128, 4>());
  int occ = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, k, kDecThreads, 0) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  v = occ * cus;
  if (v > 0) cache[dev][di][gi].store(v, std::memory_order_relaxed);
  return v;
}

template <int D, int GP, bool PAGED>
hipError_t launch_bal(const DecodeArgs& a, void* ws, int P) {
  constexpr int HPW = 512 / D;
  const int nbq = (a.Hkv / HPW) * (a.Hq / a.Hkv / GP);
  const int64_t grid = (int64_t)P * nbq;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  const DecodeBalLayout l = decode_bal_layout(a.B, a.Hq, D, P);
  char* base = static_cast<char*>(ws);
  long long* cum = reinterpret_cast<long long*>(base);
  float* part_lse = reinterpret_cast<float*>(base + l.cum_bytes);
  float* part_o = reinterpret_cast<float*>(base + l.cum_bytes + l.lse_bytes);
  const int append = a.k_new ? 1 : 0;
  hipLaunchKernelGGL((decode_split_bal_kernel<D, GP, PAGED>), dim3((unsigned)grid), dim3(kDecThreads), 0, a.stream,
                     (const __bf16*)a.q, (const __bf16*)a.k_cache, (const __bf16*)a.v_cache, a.seqlens, part_o,
                     part_lse, cum, a.B, a.Hq, a.Hkv, a.N, P, a.scale * kLog2e, append, page_map(a));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_merge_bal_kernel<D>, dim3((unsigned)(a.B * a.Hq)), dim3(64), 0, a.stream, part_o, part_lse,
                     cum, (__bf16*)a.o, a.lse, a.B, a.Hq, P);
  return hipGetLastError();
}

template <int D, bool PAGED>
hipError_t launch_bal_gp(const DecodeArgs& a, int gp, void* ws, int P) {
  switch (gp) {
    case 1: return launch_bal<D, 1, PAGED>(a, ws, P);
    case 2: return launch_bal<D, 2, PAGED>(a, ws, P);
    default: return launch_bal<D, 4, PAGED>(a, ws, P);
  }
}

}  // namespace

void* decode_noalloc_scratch(hipError_t* err) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess && (dev < 0 || dev >= kMaxDevices)) e = hipErrorInvalidDevice;
  if (e != hipSuccess) {
    *err = e;
    return nullptr;
  }
  void* ptr = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (ptr) return ptr;
  e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !ptr) {
    *err = e != hipSuccess ? e : hipErrorInvalidSymbol;
    return nullptr;
  }
  g_scratch_addr[dev].store(ptr, std::memory_order_release);
  return ptr;
}

int decode_balanced_ranges(int B, int Hq, int Hkv, int d, int num_splits) {
  if (num_splits != 0 || B > kDecBalMaxB || B <= 0 || (d != 64 && d != 128) || Hkv <= 0 || Hq % Hkv != 0) return 0;
  if (Hkv % (512 / d) != 0) return 0;
  const int gp = decode_heads_per_group(Hq, Hkv);
  const int nbq = (Hkv / (512 / d)) * (Hq / Hkv / gp);
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  const int slots = bal_slots_per_cu(dev, d, gp);
  if (slots <= 0) return 0;
  return std::max(1, slots * kDecBalRounds / nbq);
}

DecodeBalLayout decode_bal_layout(int B, int Hq, int d, int P) {
  const size_t slots = (size_t)P + B - 1;
  return DecodeBalLayout{round_up256((size_t)(B + 1) * sizeof(long long)),
                         round_up256(slots * Hq * sizeof(float)),
                         round_up256(slots * Hq * (size_t)d * sizeof(float))};
}

hipError_t launch_decode_balanced(const DecodeArgs& a, void* workspace, int P) {
  const bool paged = a.block_table != nullptr;
  hipError_t e = hipSuccess;
  if (a.k_new) {
    if (a.d == 64) e = paged ? launch_append<64, true>(a) : launch_append<64, false>(a);
    else e = paged ? launch_append<128, true>(a) : launch_append<128, false>(a);
    if (e != hipSuccess) return e;
  }
  const int gp = decode_heads_per_group(a.Hq, a.Hkv);
  if (a.d == 64) return paged ? launch_bal_gp<64, true>(a, gp, workspace, P) : launch_bal_gp<64, false>(a, gp, workspace, P);
  return paged ? launch_bal_gp<128, true>(a, gp, workspace, P) : launch_bal_gp<128, false>(a, gp, workspace, P);
}

hipError_t launch_decode(const DecodeArgs& a, float* part_o, float* part_lse, int chunk, int nsplit) {
  const bool paged = a.block_table != nullptr;
  hipError_t e = hipSuccess;
  if (a.k_new) {
    if (a.d == 64) e = paged ? launch_append<64, true>(a) : launch_append<64, false>(a);
    else e = paged ? launch_append<128, true>(a) : launch_append<128, false>(a);
    if (e != hipSuccess) return e;
  }
  const int gp = decode_heads_per_group(a.Hq, a.Hkv);
  if (a.d == 64) {
    e = paged ? launch_split_gp<64, true>(a, gp, chunk, nsplit, part_o, part_lse)
              : launch_split_gp<64, false>(a, gp, chunk, nsplit, part_o, part_lse);
  } else {
    e = paged ? launch_split_gp<128, true>(a, gp, chunk, nsplit, part_o, part_lse)
              : launch_split_gp<128, false>(a, gp, chunk, nsplit, part_o, part_lse);
  }
  if (e != hipSuccess) return e;
  const int64_t grid = (int64_t)a.B * a.Hq;
  const int append = a.k_new ? 1 : 0;
  if (a.d == 64) {
    hipLaunchKernelGGL(decode_merge_kernel<64>, dim3((unsigned)grid), dim3(64), 0, a.stream, part_o, part_lse,
                       a.seqlens, (__bf16*)a.o, a.lse, a.B, a.Hq, a.N, chunk, nsplit, append);
  } else {
    hipLaunchKernelGGL(decode_merge_kernel<128>, dim3((unsigned)grid), dim3(64), 0, a.stream, part_o, part_lse,
                       a.seqlens, (__bf16*)a.o, a.lse, a.B, a.Hq, a.N, chunk, nsplit, append);
  }
  return hipGetLastError();
}

}  // namespace fa
