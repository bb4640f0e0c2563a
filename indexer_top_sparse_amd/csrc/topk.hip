// Exact top-k selection over fp32 score rows (step a3).
//
// "MiniMax-M3: share the sparse index top-k across layers ..." (description)
// and the "XM-Sparse" blog (2,048 selected entries per layer and step) need
// an exact top-k of each request's scores; ties go to the lower index and
// the k indices come out ascending.
//
// Design (radix select on order-preserving 32-bit keys, few long rows):
//   hist    rows x chunks workgroups: a 4096-bin histogram of the top 12 key
//           bits of every valid unit (LDS, then global atomics).  The fused
//           score kernels build the same histogram while they write scores.
//   bin     one workgroup per row: the bin b* holding the k-th largest key,
//           and the count of units above it.
//   filter  rows x chunks workgroups: compacts, in index order, every unit
//           whose bin is >= b* into its chunk's slice of a candidate buffer
//           (keys and indices) and stores the chunk count.
//   select  one workgroup per row: stages the candidates in LDS and resolves
//           the remaining 20 key bits over those of bin b* (two histogram
//           passes), which
//           gives the exact k-th key T and how many units equal to T are
//           needed, then writes the selection in index order with block
//           prefix sums (ties to the lowest indices).
#include "common.hpp"

namespace sd {

__global__ void zero_u32_kernel(uint32_t* __restrict__ p, int64_t count) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (; i < count; i += stride) p[i] = 0u;
}

hipError_t launch_zero_u32(uint32_t* p, int64_t count, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  int64_t blocks = (count + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  zero_u32_kernel<<<(unsigned)blocks, 256, 0, s>>>(p, count);
  return hipGetLastError();
}

__device__ __forceinline__ int row_valid_units(const TopkPlan& p, int r) {
  int v = p.n_units;
  if (p.valid) {
    int t = p.valid[r / p.rows_per_valid];
    if (p.unit_div > 1) t = (t + p.unit_div - 1) / p.unit_div;
    v = t < 0 ? 0 : (t > p.n_units ? p.n_units : t);
  }
  return v;
}

// --------------------------------------------------------------------- hist
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
  uint32_t* g = p.hist + (int64_t)r * kHistStride;
  for (int i = threadIdx.x; i < kHistBins; i += 256)
    if (h[i]) atomicAdd(&g[i], h[i]);
}

hipError_t launch_topk_hist(const TopkPlan& p, hipStream_t s) {
  dim3 grid(p.n_chunks, p.rows);
  topk_hist_kernel<<<grid, 256, 0, s>>>(p);
  return hipGetLastError();
}

// Find, over `nbins` LDS bins counted from the top, the bin holding the
// need-th largest key: out[0] = bin, out[1] = units in higher bins.
template <int NT>
__device__ void find_bin_from_top(const uint32_t* hist, int nbins, int need,
                                  int* scan_lds, int* out) {
  const int per = nbins / NT > 0 ? nbins / NT : 1;
  const int t = threadIdx.x;
  const bool owns = per * t < nbins;
  const int top = nbins - 1 - per * t;
  int local = 0;
  if (owns)
    for (int i = 0; i < per; ++i) local += (int)hist[top - i];
  int total;
  int incl = block_inclusive_scan<NT>(local, scan_lds, &total);
  int excl = incl - local;
  if (owns && excl < need && incl >= need) {
    int cum = excl;
    for (int i = 0; i < per; ++i) {
      int b = top - i;
      int c = (int)hist[b];
      if (cum + c >= need) {
        out[0] = b;
        out[1] = cum;
        break;
      }
      cum += c;
    }
  }
  __syncthreads();
}

// --------------------------------------------------------------------- bin
// One workgroup per row: the bin b* holding the k_eff-th largest key of the
// complete histogram, and the number of units in higher bins, stored in the
// row's tail for the filter and select kernels.
constexpr int kBinThreads = 512;

__global__ __launch_bounds__(kBinThreads) void topk_bin_kernel(TopkPlan p) {
  __shared__ uint32_t hs[kHistBins];
  __shared__ int scan_lds[kBinThreads / 64 + 1];
  __shared__ int res[2];
  const int r = blockIdx.x;
  const int k_eff = min(p.k, row_valid_units(p, r));
  uint32_t* g = p.hist + (int64_t)r * kHistStride;
  for (int i = threadIdx.x; i < kHistBins; i += kBinThreads) hs[i] = g[i];
  if (threadIdx.x == 0) { res[0] = 0; res[1] = 0; }
  __syncthreads();
  if (k_eff > 0) find_bin_from_top<kBinThreads>(hs, kHistBins, k_eff, scan_lds, res);
  if (threadIdx.x == 0) {
    g[kHistBstar] = (uint32_t)res[0];
    g[kHistAbove] = (uint32_t)res[1];
  }
}

hipError_t launch_topk_bin(const TopkPlan& p, hipStream_t s) {
  topk_bin_kernel<<<p.rows, kBinThreads, 0, s>>>(p);
  return hipGetLastError();
}

// ------------------------------------------------------------------- filter
__global__ __launch_bounds__(256) void topk_filter_kernel(TopkPlan p) {
  __shared__ int scan_lds[8];
  const int r = blockIdx.y;
  const int c = blockIdx.x;
  const int v = row_valid_units(p, r);
  const int k_eff = min(p.k, v);
  uint32_t* cnt = p.chunk_cnt + (int64_t)r * p.n_chunks + c;
  if (k_eff <= 0) {
    if (threadIdx.x == 0) *cnt = 0u;
    return;
  }
  const uint32_t bstar = p.hist[(int64_t)r * kHistStride + kHistBstar];
  const float* row = p.scores + (int64_t)r * p.row_stride;
  uint32_t* ck = p.cand_key + (int64_t)r * p.n_units + (int64_t)c * kTopkChunk;
  int32_t* ci = p.cand_idx + (int64_t)r * p.n_units + (int64_t)c * kTopkChunk;
  const int lo = c * kTopkChunk;
  const int hi = min(lo + kTopkChunk, v);
  int base = 0;
  for (int it = lo; it < hi; it += 256 * 4) {
    const int u0 = it + threadIdx.x * 4;
    uint32_t keys[4];
    int flags = 0, cnt_t = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int u = u0 + i;
      keys[i] = 0u;
      if (u < hi) {
        keys[i] = score_key(row[u]);
        if ((keys[i] >> 20) >= bstar) { flags |= 1 << i; ++cnt_t; }
      }
    }
    int total;
    int incl = block_inclusive_scan<256>(cnt_t, scan_lds, &total);
    int pos = base + incl - cnt_t;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (flags & (1 << i)) {
        ck[pos] = keys[i];
        ci[pos] = u0 + i;
        ++pos;
      }
    }
    base += total;
  }
  if (threadIdx.x == 0) *cnt = (uint32_t)base;
}

hipError_t launch_topk_filter(const TopkPlan& p, hipStream_t s) {
  dim3 grid(p.n_chunks, p.rows);
  topk_filter_kernel<<<grid, 256, 0, s>>>(p);
  return hipGetLastError();
}

// ------------------------------------------------------------------- select
constexpr int kSelThreads = 1024;
constexpr int kSelCap = 12288;  // candidates staged in LDS (96 KB)

__device__ __forceinline__ int find_chunk(const int* excl, int nchunks, int p) {
  // largest c with excl[c] <= p
  int lo = 0, hi = nchunks - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (excl[mid] <= p) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__global__ __launch_bounds__(kSelThreads) void topk_select_kernel(TopkPlan p) {
  __shared__ uint32_t ckey_s[kSelCap];
  __shared__ int32_t cidx_s[kSelCap];
  __shared__ uint32_t hs[kHistBins];
  __shared__ int excl[1025];
  __shared__ int scan_lds[kSelThreads / 64 + 1];
  __shared__ int res[2];
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const int v = row_valid_units(p, r);
  const int k_eff = min(p.k, v);
  int32_t* oi = p.idx_out + (int64_t)r * p.k;
  float* ov = p.val_out ? p.val_out + (int64_t)r * p.k : nullptr;
  for (int j = k_eff + tid; j < p.k; j += kSelThreads) {
    oi[j] = -1;
    if (ov) ov[j] = -__builtin_huge_valf();
  }
  if (k_eff <= 0) return;

  const uint32_t* g = p.hist + (int64_t)r * kHistStride;
  const uint32_t b1 = g[kHistBstar];
  int above = (int)g[kHistAbove];

  // chunk offsets
  const uint32_t* cc = p.chunk_cnt + (int64_t)r * p.n_chunks;
  int M = 0;
  for (int base = 0; base < p.n_chunks; base += kSelThreads) {
    int c = base + tid;
    int x = c < p.n_chunks ? (int)cc[c] : 0;
    int total;
    int incl = block_inclusive_scan<kSelThreads>(x, scan_lds, &total);
    if (c < p.n_chunks) excl[c] = M + incl - x;
    M += total;
    __syncthreads();
  }
  const uint32_t* ck = p.cand_key + (int64_t)r * p.n_units;
  const int32_t* ci = p.cand_idx + (int64_t)r * p.n_units;
  const int nch = p.n_chunks;
  auto cand_off = [&](int q) -> int64_t {
    int c = find_chunk(excl, nch, q);
    return (int64_t)c * kTopkChunk + (q - excl[c]);
  };
  // stage the candidates (in index order) in LDS when they fit
  const bool inlds = M <= kSelCap;
  if (inlds) {
    for (int q = tid; q < M; q += kSelThreads) {
      const int64_t o = cand_off(q);
      ckey_s[q] = ck[o];
      cidx_s[q] = ci[o];
    }
  }
  auto key_at = [&](int q) -> uint32_t { return inlds ? ckey_s[q] : ck[cand_off(q)]; };
  auto idx_at = [&](int q) -> int32_t { return inlds ? cidx_s[q] : ci[cand_off(q)]; };

  // level 2: bits [19:8] of the keys in bin b1
  for (int i = tid; i < kHistBins; i += kSelThreads) hs[i] = 0u;
  __syncthreads();
  for (int q = tid; q < M; q += kSelThreads) {
    uint32_t key = key_at(q);
    if ((key >> 20) == b1) atomicAdd(&hs[(key >> 8) & 0xFFFu], 1u);
  }
  if (tid == 0) { res[0] = 0; res[1] = 0; }
  __syncthreads();
  find_bin_from_top<kSelThreads>(hs, kHistBins, k_eff - above, scan_lds, res);
  const uint32_t b2 = (uint32_t)res[0];
  above += res[1];
  __syncthreads();

  // level 3: bits [7:0] of the keys with prefix (b1, b2)
  const uint32_t pre = (b1 << 12) | b2;
  for (int i = tid; i < 256; i += kSelThreads) hs[i] = 0u;
  __syncthreads();
  for (int q = tid; q < M; q += kSelThreads) {
    uint32_t key = key_at(q);
    if ((key >> 8) == pre) atomicAdd(&hs[key & 0xFFu], 1u);
  }
  if (tid == 0) { res[0] = 0; res[1] = 0; }
  __syncthreads();
  find_bin_from_top<kSelThreads>(hs, 256, k_eff - above, scan_lds, res);
  const uint32_t d3 = (uint32_t)res[0];
  const uint32_t T = (pre << 8) | d3;
  const int count_gt = above + res[1];
  const int eq_need = k_eff - count_gt;
  const int eq_total = (int)hs[d3];
  __syncthreads();

  // final ordered pass, 4 consecutive candidates per thread per round
  int eq_carry = 0, take_carry = 0;
  const bool all_ties = (eq_total == eq_need);
  for (int base = 0; base < M; base += 4 * kSelThreads) {
    const int q0 = base + 4 * tid;
    uint32_t key[4];
    int gt[4], eq[4];
    int n_eq = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = q0 + i;
      key[i] = q < M ? key_at(q) : 0u;
      gt[i] = (q < M) && key[i] > T;
      eq[i] = (q < M) && key[i] == T;
      n_eq += eq[i];
    }
    int take[4];
    if (all_ties) {
#pragma unroll
      for (int i = 0; i < 4; ++i) take[i] = gt[i] | eq[i];
    } else {
      int total;
      int incl = block_inclusive_scan<kSelThreads>(n_eq, scan_lds, &total);
      int rank = eq_carry + incl - n_eq;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        take[i] = gt[i] || (eq[i] && rank < eq_need);
        rank += eq[i];
      }
      eq_carry += total;
    }
    const int n_take = take[0] + take[1] + take[2] + take[3];
    int total;
    int incl = block_inclusive_scan<kSelThreads>(n_take, scan_lds, &total);
    int pos = take_carry + incl - n_take;
    take_carry += total;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (take[i] && pos < k_eff) {
        oi[pos] = idx_at(q0 + i);
        if (ov) ov[pos] = key_score(key[i]);
        ++pos;
      }
    }
  }
}

hipError_t launch_topk_select(const TopkPlan& p, hipStream_t s) {
  topk_select_kernel<<<p.rows, kSelThreads, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace sd
