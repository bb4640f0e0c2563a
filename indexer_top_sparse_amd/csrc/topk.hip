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
//   filter  rows x chunks workgroups: each finds the bin b* holding the k-th
//           largest key from the histogram, then compacts, in index order,
//           every unit whose bin is >= b* into its chunk's slice of a
//           candidate buffer (keys and indices) and stores the chunk count.
//   select  one workgroup per row: resolves the remaining 20 key bits over
//           the few candidates of bin b* (two LDS histogram passes), which
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
  uint32_t* g = p.hist + (int64_t)r * kHistBins;
  for (int i = threadIdx.x; i < kHistBins; i += 256)
    if (h[i]) atomicAdd(&g[i], h[i]);
}

hipError_t launch_topk_hist(const TopkPlan& p, hipStream_t s) {
  dim3 grid(p.n_chunks, p.rows);
  topk_hist_kernel<<<grid, 256, 0, s>>>(p);
  return hipGetLastError();
}

// Find the bin holding the k-th largest key.  NT threads; each thread owns
// kHistBins/NT consecutive bins counted from the top.  Writes b* and the
// number of units in higher bins to out[0], out[1].  k_eff >= 1.
template <int NT>
__device__ void find_bin_from_top(const uint32_t* hist, int nbins, int need,
                                  int* scan_lds, int* out) {
  constexpr int PER = kHistBins / NT;
  const int per = nbins / NT;  // nbins is 4096 or 256 (and NT divides it)
  (void)PER;
  const int t = threadIdx.x;
  // thread t covers bins [top - per*(t+1) + 1, top - per*t] (descending)
  const int top = nbins - 1 - per * t;
  int local = 0;
  for (int i = 0; i < per; ++i) local += (int)hist[top - i];
  int total;
  int incl = block_inclusive_scan<NT>(local, scan_lds, &total);
  int excl = incl - local;
  if (excl < need && incl >= need) {
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

// ------------------------------------------------------------------- filter
__global__ __launch_bounds__(256) void topk_filter_kernel(TopkPlan p) {
  __shared__ uint32_t hs[kHistBins];
  __shared__ int scan_lds[8];
  __shared__ int res[2];
  const int r = blockIdx.y;
  const int c = blockIdx.x;
  const int v = row_valid_units(p, r);
  const int k_eff = min(p.k, v);
  uint32_t* cnt = p.chunk_cnt + (int64_t)r * p.n_chunks + c;
  if (k_eff <= 0) {
    if (threadIdx.x == 0) *cnt = 0u;
    return;
  }
  const uint32_t* g = p.hist + (int64_t)r * kHistBins;
  for (int i = threadIdx.x; i < kHistBins; i += 256) hs[i] = g[i];
  if (threadIdx.x == 0) { res[0] = 0; res[1] = 0; }
  __syncthreads();
  find_bin_from_top<256>(hs, kHistBins, k_eff, scan_lds, res);
  const uint32_t bstar = (uint32_t)res[0];

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

  // level 1 (from the 12-bit histogram)
  const uint32_t* g = p.hist + (int64_t)r * kHistBins;
  for (int i = tid; i < kHistBins; i += kSelThreads) hs[i] = g[i];
  if (tid == 0) { res[0] = 0; res[1] = 0; }
  __syncthreads();
  find_bin_from_top<kSelThreads>(hs, kHistBins, k_eff, scan_lds, res);
  const uint32_t b1 = (uint32_t)res[0];
  int above = res[1];
  __syncthreads();

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

  // level 2: bits [19:8] of the keys in bin b1
  for (int i = tid; i < kHistBins; i += kSelThreads) hs[i] = 0u;
  __syncthreads();
  for (int q = tid; q < M; q += kSelThreads) {
    uint32_t key = ck[cand_off(q)];
    if ((key >> 20) == b1) atomicAdd(&hs[(key >> 8) & 0xFFFu], 1u);
  }
  __syncthreads();
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
    uint32_t key = ck[cand_off(q)];
    if ((key >> 8) == pre) atomicAdd(&hs[key & 0xFFu], 1u);
  }
  __syncthreads();
  if (tid == 0) { res[0] = 0; res[1] = 0; }
  __syncthreads();
  // 256 bins over 1024 threads: only the first 256 threads own bins
  {
    int local = tid < 256 ? (int)hs[255 - tid] : 0;
    int total;
    int incl = block_inclusive_scan<kSelThreads>(local, scan_lds, &total);
    int ex = incl - local;
    int need = k_eff - above;
    if (tid < 256 && ex < need && incl >= need) {
      res[0] = 255 - tid;
      res[1] = ex;
    }
    __syncthreads();
  }
  const uint32_t T = (pre << 8) | (uint32_t)res[0];
  const int count_gt = above + res[1];
  const int eq_need = k_eff - count_gt;
  __syncthreads();

  // final ordered pass
  int eq_carry = 0, take_carry = 0;
  for (int base = 0; base < M; base += kSelThreads) {
    int q = base + tid;
    uint32_t key = 0;
    int32_t idx = -1;
    if (q < M) {
      int64_t o = cand_off(q);
      key = ck[o];
      idx = ci[o];
    }
    int gt = (q < M) && key > T;
    int eq = (q < M) && key == T;
    int total;
    int eq_incl = block_inclusive_scan<kSelThreads>(eq, scan_lds, &total);
    int eq_rank = eq_carry + eq_incl - eq;
    eq_carry += total;
    int take = gt || (eq && eq_rank < eq_need);
    int t_incl = block_inclusive_scan<kSelThreads>(take, scan_lds, &total);
    int pos = take_carry + t_incl - take;
    take_carry += total;
    if (take && pos < k_eff) {
      oi[pos] = idx;
      if (ov) ov[pos] = key_score(key);
    }
  }
}

hipError_t launch_topk_select(const TopkPlan& p, hipStream_t s) {
  topk_select_kernel<<<p.rows, kSelThreads, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace sd
