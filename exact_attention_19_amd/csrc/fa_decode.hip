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
#include "fa_common.h"
#include "fa_internal.h"

namespace fa {

namespace {

constexpr int kDecThreads = 256;
constexpr int kDecWaves = kDecThreads / 64;
constexpr int kDecUnroll = 8;  // cache rows per row group per iteration

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
