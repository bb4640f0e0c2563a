// Exact top-k selection over fp32 score rows (step a3).
//
// "MiniMax-M3: share the sparse index top-k across layers ..." (description)
// and the "XM-Sparse" blog (2,048 selected entries per layer and step) need
// an exact top-k of each request's scores; ties go to the lower index and
// the k indices come out ascending.
//
// Design (radix select on order-preserving 32-bit keys, few long rows):
//   hist    rows x chunks workgroups: each counts the top 12 key bits of
//           its chunk's valid units in a 4096-bin LDS histogram and stores it
//           as one 16-bit part of the row's histogram, followed by 64 coarse
//           counts.  The fused score kernels store the same parts while they
//           write scores.
//   When a row has at most 64 parts, each one contiguous span of units:
//   filter_fused  rows x parts workgroups: each finds b* (the bin holding the
//           k-th largest key) from the coarse counts and the 64 bins of one
//           coarse bin, derives every part's candidate count from the same
//           counts, and compacts its part's units with bin >= b* in index
//           order straight into the row's single candidate list.
//   Otherwise:
//   bin     one workgroup per row: sums the row's parts, finds b* and the
//           count of units above it.
//   filter  rows x chunks workgroups: compacts, in index order, every unit
//           whose bin is >= b* into its chunk's slice of a candidate buffer
//           (keys and indices) and stores the chunk count (one block scan).
//   Rows of at most kTopkDirectMax units take the select alone: it stages
//   the row's own keys as the candidates and counts their top 12 bits to
//   find b* first.
//   select  one workgroup per row: stages the candidates in LDS while
//           counting bits [19:8] of those in bin b*, resolves
//           the last 8 bits in a second LDS histogram, which gives the exact
//           k-th key T and how many units equal to T are needed, then
//           writes the selection in index order with block prefix sums
//           (ties to the lowest indices).
#include "select.hpp"

namespace sd {

// --------------------------------------------------------------------- hist
// Part c of row r's histogram: the valid units of chunk c (p.parts must be
// p.n_chunks).
__global__ __launch_bounds__(256) void topk_hist_kernel(TopkPlan p) {
  __shared__ uint32_t h[kHistBins];
  const int r = blockIdx.y;
  const int c = blockIdx.x;
  for (int i = threadIdx.x; i < kHistBins; i += 256) h[i] = 0u;
  __syncthreads();
  const int v = row_valid_units(p, r);
  const float* row = p.scores + (int64_t)r * p.row_stride;
  const int lo = c * kTopkChunk;
  const int hi = min(lo + kTopkChunk, v);
  for (int u = lo + threadIdx.x; u < hi; u += 256)
    atomicAdd(&h[score_key(row[u]) >> 20], 1u);
  __syncthreads();
  store_hist_part(h, p.hist + ((int64_t)r * p.parts + c) * kHistPartWords, 256);
}

hipError_t launch_topk_hist(const TopkPlan& p, hipStream_t s) {
  dim3 grid(p.n_chunks, p.rows);
  topk_hist_kernel<<<grid, 256, 0, s>>>(p);
  return hipGetLastError();
}

// --------------------------------------------------------------------- bin
// One workgroup per row: sums the row's histogram parts, then the bin b*
// holding the k_eff-th largest key and the number of units in higher bins.
constexpr int kBinThreads = 1024;
constexpr int kBinGroups = kBinThreads / (kHistWords / 4);  // 2 part groups
constexpr int kBinUnroll = 8;

__global__ __launch_bounds__(kBinThreads) void topk_bin_kernel(TopkPlan p) {
  __shared__ uint32_t hs[kBinGroups][kHistBins];
  __shared__ int scan_lds[kBinThreads / 64 + 1];
  __shared__ int res[2];
  const int r = blockIdx.x;
  const int t = threadIdx.x;
  const int k_eff = min(p.k, row_valid_units(p, r));
  // thread t: words 4 (t % 512) .. +3 (bins 8 (t % 512) .. +7) of parts
  // t / 512, t / 512 + 2, ...; kBinUnroll loads in flight
  const int grp = t / (kHistWords / 4);
  const int wq = t % (kHistWords / 4);
  const uint32_t* base = p.hist + (int64_t)r * p.parts * kHistPartWords + 4 * wq;
  uint32_t cnt[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int q0 = grp; q0 < p.parts; q0 += kBinGroups * kBinUnroll) {
    u32x4 w[kBinUnroll];
#pragma unroll
    for (int u = 0; u < kBinUnroll; ++u) {
      const int q = q0 + u * kBinGroups;
      w[u] = q < p.parts ? *(const u32x4*)(base + (int64_t)q * kHistPartWords) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kBinUnroll; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        cnt[2 * e] += w[u][e] & 0xFFFFu;
        cnt[2 * e + 1] += w[u][e] >> 16;
      }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) hs[grp][8 * wq + e] = cnt[e];
  if (t == 0) { res[0] = 0; res[1] = 0; }
  __syncthreads();
  for (int i = t; i < kHistBins; i += kBinThreads) {
    uint32_t x = hs[0][i];
#pragma unroll
    for (int gq = 1; gq < kBinGroups; ++gq) x += hs[gq][i];
    hs[0][i] = x;
  }
  __syncthreads();
  if (k_eff > 0) find_bin_from_top<kBinThreads>(hs[0], kHistBins, k_eff, scan_lds, res);
  if (t == 0) {
    p.bstar[2 * r] = (uint32_t)res[0];
    p.bstar[2 * r + 1] = (uint32_t)res[1];
  }
}

hipError_t launch_topk_bin(const TopkPlan& p, hipStream_t s) {
  topk_bin_kernel<<<p.rows, kBinThreads, 0, s>>>(p);
  return hipGetLastError();
}

// ------------------------------------------------------------------- filter
// One workgroup per (chunk, row); thread t owns the 16 consecutive units
// lo + 16t .. lo + 16t + 15 of the chunk, so one block scan orders them all.
constexpr int kFiltThreads = 256;
constexpr int kFiltPer = kTopkChunk / kFiltThreads;  // 16
static_assert(kFiltPer == 16, "four float4 loads per thread");

__global__ __launch_bounds__(kFiltThreads) void topk_filter_kernel(TopkPlan p) {
  __shared__ int scan_lds[kFiltThreads / 64 + 1];
  const int r = blockIdx.y;
  const int c = blockIdx.x;
  const int v = row_valid_units(p, r);
  const int k_eff = min(p.k, v);
  uint32_t* cnt = p.chunk_cnt + (int64_t)r * p.n_chunks + c;
  if (k_eff <= 0) {
    if (threadIdx.x == 0) *cnt = 0u;
    return;
  }
  const uint32_t bstar = p.bstar[2 * r];
  const float* row = p.scores + (int64_t)r * p.row_stride;
  uint32_t* ck = p.cand_key + (int64_t)r * p.n_units + (int64_t)c * kTopkChunk;
  int32_t* ci = p.cand_idx + (int64_t)r * p.n_units + (int64_t)c * kTopkChunk;
  const int lo = c * kTopkChunk;
  const int hi = min(lo + kTopkChunk, v);
  const int u0 = lo + kFiltPer * threadIdx.x;
  uint32_t keys[kFiltPer];
  uint32_t flags = 0;
  int n_t = 0;
  if (u0 + kFiltPer <= hi && ((uintptr_t)(row + u0) & 15u) == 0) {
#pragma unroll
    for (int i = 0; i < kFiltPer; i += 4) {
      const f32x4 x = *(const f32x4*)(row + u0 + i);
#pragma unroll
      for (int e = 0; e < 4; ++e) keys[i + e] = score_key(x[e]);
    }
#pragma unroll
    for (int i = 0; i < kFiltPer; ++i)
      if ((keys[i] >> 20) >= bstar) { flags |= 1u << i; ++n_t; }
  } else {
#pragma unroll
    for (int i = 0; i < kFiltPer; ++i) {
      keys[i] = 0u;
      if (u0 + i < hi) {
        keys[i] = score_key(row[u0 + i]);
        if ((keys[i] >> 20) >= bstar) { flags |= 1u << i; ++n_t; }
      }
    }
  }
  int total;
  const int incl = block_inclusive_scan<kFiltThreads>(n_t, scan_lds, &total);
  int pos = incl - n_t;
#pragma unroll
  for (int i = 0; i < kFiltPer; ++i) {
    if (flags & (1u << i)) {
      ck[pos] = keys[i];
      ci[pos] = u0 + i;
      ++pos;
    }
  }
  if (threadIdx.x == 0) *cnt = (uint32_t)total;
}

hipError_t launch_topk_filter(const TopkPlan& p, hipStream_t s) {
  dim3 grid(p.n_chunks, p.rows);
  topk_filter_kernel<<<grid, kFiltThreads, 0, s>>>(p);
  return hipGetLastError();
}

// ------------------------------------------------------------- fused filter
// One workgroup per (part, row) when a row's histogram parts are at most
// kFuseMaxParts contiguous spans of part_span units.  Each workgroup finds
// the boundary bin b* itself: the coarse counts of all parts give the coarse
// bin holding the k-th largest key, and the 64 bins of that coarse bin in
// all parts give b*.  The same counts give every part's number of
// candidates (units with bin >= b*), hence this part's offset in the row's
// contiguous candidate list, so the candidates are written in index order
// straight to their final place.  Part 0 stores b*, the units above it and
// the row's candidate count for the select.
// NT threads, PER units per thread and pass: 1024 x 16 for parts of more
// than 8192 units, 512 x 16 down to 4097, 256 x 16 or 256 x 8 for parts of
// at most 4096 or 2048 units.

// (counts stay below 2^31)
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t x, int) {
  return (uint32_t)wave_incl_scan((int)x);
}
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t x) { return (uint32_t)wave_sum((int)x); }

template <int NT, int PER>
__global__ __launch_bounds__(NT) void topk_filter_fused_kernel(TopkPlan p) {
  constexpr int kFfThreads = NT, kFfPer = PER, kFfPass = NT * PER;
  constexpr int NW = kFfThreads / kWave;
  constexpr int PPW = kFuseMaxParts / NW;  // parts per wave: q = wave + NW i
  __shared__ uint32_t ptot[NW][64];
  __shared__ uint32_t cnt_s[kFuseMaxParts];
  __shared__ int res[5];
  __shared__ int scan_lds[NW + 1];
  const int r = blockIdx.y;
  const int q0 = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int P = p.parts;
  const int v = row_valid_units(p, r);
  const int k_eff = min(p.k, v);
  const int lo = q0 * p.part_span;
  if (k_eff <= 0 || (lo >= v && q0 != 0)) return;  // (uniform)
  const int hi = min(lo + p.part_span, v);
  const float* row = p.scores + (int64_t)r * p.row_stride;
  const uint32_t* hrow = p.hist + (int64_t)r * P * kHistPartWords;
  if (tid == 0) { res[0] = 0; res[1] = 0; res[2] = 0; res[3] = 0; }

  // coarse counts of this wave's parts; lane j holds coarse bin 63 - j
  uint32_t xc[PPW];
#pragma unroll
  for (int i = 0; i < PPW; ++i) {
    const int q = wid + NW * i;
    xc[i] = q < P ? hrow[(int64_t)q * kHistPartWords + kHistWords + 63 - lane] : 0u;
  }
  // the first pass of this part's scores is in flight during the search
  float raw[kFfPer];
  auto load_raw = [&](int base) __attribute__((always_inline)) {
    const int u0 = base + kFfPer * tid;
    if (u0 + kFfPer <= hi && ((uintptr_t)(row + u0) & 15u) == 0) {
#pragma unroll
      for (int i = 0; i < kFfPer; i += 4) {
        // scores are read once here: non-temporal
        const f32x4 x = __builtin_nontemporal_load((const f32x4*)(row + u0 + i));
#pragma unroll
        for (int e = 0; e < 4; ++e) raw[i + e] = x[e];
      }
    } else {
#pragma unroll
      for (int i = 0; i < kFfPer; ++i) raw[i] = u0 + i < hi ? row[u0 + i] : 0.f;
    }
  };
  load_raw(lo);

  // coarse bin cb holding the k_eff-th largest key (totals from the top)
  {
    uint32_t x = 0;
#pragma unroll
    for (int i = 0; i < PPW; ++i) x += xc[i];
    ptot[wid][lane] = x;
  }
  __syncthreads();
  if (wid == 0) {
    uint32_t t = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) t += ptot[w][lane];
    const uint32_t incl = wave_incl_scan_u32(t, lane);
    if (incl - t < (uint32_t)k_eff && incl >= (uint32_t)k_eff) {
      res[0] = 63 - lane;
      res[1] = (int)(incl - t);
    }
  }
  __syncthreads();
  const int cb = res[0];
  const int above_c = res[1];
  // the 64 bins of coarse bin cb in this wave's parts; lane j holds bin
  // 64 cb + 63 - j
  uint32_t xf[PPW];
  {
    const int fb = 63 - lane;
    uint32_t x = 0;
#pragma unroll
    for (int i = 0; i < PPW; ++i) {
      const int q = wid + NW * i;
      uint32_t f = 0;
      if (q < P) {
        const uint32_t word = hrow[(int64_t)q * kHistPartWords + 32 * cb + (fb >> 1)];
        f = (fb & 1) ? word >> 16 : word & 0xFFFFu;
      }
      xf[i] = f;
      x += f;
    }
    ptot[wid][lane] = x;
  }
  __syncthreads();
  if (wid == 0) {
    const uint32_t need = (uint32_t)(k_eff - above_c);
    uint32_t t = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) t += ptot[w][lane];
    const uint32_t incl = wave_incl_scan_u32(t, lane);
    if (incl - t < need && incl >= need) {
      res[2] = 64 * cb + 63 - lane;
      res[3] = above_c + (int)(incl - t);
    }
  }
  __syncthreads();
  const uint32_t bstar = (uint32_t)res[2];
  const int fine = res[2] - 64 * cb;
  // candidates of this wave's parts: coarse bins above cb (lanes < 63 - cb)
  // and bins >= b* inside cb (lanes <= 63 - fine)
#pragma unroll
  for (int i = 0; i < PPW; ++i) {
    const int q = wid + NW * i;
    if (q < P) {
      const uint32_t c = (lane < 63 - cb ? xc[i] : 0u) + (lane <= 63 - fine ? xf[i] : 0u);
      const uint32_t sum = wave_sum_u32(c);
      if (lane == 0) cnt_s[q] = sum;
    }
  }
  __syncthreads();
  if (wid == 0) {
    const uint32_t x = lane < P ? cnt_s[lane] : 0u;
    const uint32_t incl = wave_incl_scan_u32(x, lane);
    if (lane < P) cnt_s[lane] = incl - x;
    if (lane == 63) res[4] = (int)incl;
  }
  __syncthreads();
  if (q0 == 0 && tid == 0) {
    p.bstar[2 * r] = bstar;
    p.bstar[2 * r + 1] = (uint32_t)res[3];
    p.cand_total[r] = (uint32_t)res[4];
  }

  uint32_t* ck = p.cand_key + (int64_t)r * p.n_units;
  int32_t* ci = p.cand_idx + (int64_t)r * p.n_units;
  int carry = (int)cnt_s[q0];
  for (int base = lo; base < hi; base += kFfPass) {
    const int u0 = base + kFfPer * tid;
    uint32_t keys[kFfPer];
#pragma unroll
    for (int i = 0; i < kFfPer; ++i) keys[i] = score_key(raw[i]);
    // the next pass's scores are in flight while this one is compacted
    if (base + kFfPass < hi) load_raw(base + kFfPass);
    uint32_t flags = 0;
    int n_t = 0;
#pragma unroll
    for (int i = 0; i < kFfPer; ++i) {
      if (u0 + i < hi && (keys[i] >> 20) >= bstar) {
        flags |= 1u << i;
        ++n_t;
      }
    }
    int total;
    const int incl = block_inclusive_scan<kFfThreads>(n_t, scan_lds, &total);
    int pos = carry + incl - n_t;
#pragma unroll
    for (int i = 0; i < kFfPer; ++i) {
      if ((flags & (1u << i)) && pos < p.n_units) {  // (the counts bound pos)
        ck[pos] = keys[i];
        ci[pos] = u0 + i;
        ++pos;
      }
    }
    carry += total;
  }
}

hipError_t launch_topk_filter_fused(const TopkPlan& p, hipStream_t s) {
  dim3 grid(p.parts, p.rows);
  if (p.part_span > 8192) topk_filter_fused_kernel<1024, 16><<<grid, 1024, 0, s>>>(p);
  else if (p.part_span > 4096) topk_filter_fused_kernel<512, 16><<<grid, 512, 0, s>>>(p);
  else if (p.part_span > 2048) topk_filter_fused_kernel<256, 16><<<grid, 256, 0, s>>>(p);
  else topk_filter_fused_kernel<256, 8><<<grid, 256, 0, s>>>(p);
  return hipGetLastError();
}

// ------------------------------------------------------------------- select
constexpr int kSelThreads = 1024;
constexpr int kSelCap = 12288;  // candidates staged in LDS (96 KB)
static_assert(kTopkDirectMax <= kSelCap, "a direct row fits in LDS");

// One workgroup per row (select_row); the fused filter's first 4 x 1024
// list entries are loaded together with the count.
__global__ __launch_bounds__(kSelThreads) void topk_select_kernel(TopkPlan p) {
  __shared__ SelectLds<kSelThreads, kSelCap> L;
  const int r = blockIdx.x;
  int32_t* oi = p.idx_out + (int64_t)r * p.k;
  float* ov = p.val_out ? p.val_out + (int64_t)r * p.k : nullptr;
  select_row<kSelThreads, kSelCap, 4>(
      p, r, L,
      [&](int pos, int32_t idx, uint32_t key) {
        oi[pos] = idx;
        if (ov) ov[pos] = key_score(key);
      },
      [&](int pos) {
        oi[pos] = -1;
        if (ov) ov[pos] = -__builtin_huge_valf();
      });
}

hipError_t launch_topk_select(const TopkPlan& p, hipStream_t s) {
  topk_select_kernel<<<p.rows, kSelThreads, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace sd
