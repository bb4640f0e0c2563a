// The last step of the exact top-k (step a3): one workgroup selects one score
// row from its candidates, the units whose top 12 key bits are at or above
// the boundary bin b*.  "MiniMax-M3: share the sparse index top-k across
// layers ..." (description) and the "XM-Sparse" blog (2,048 entries per layer
// and step) need the exact top-k of each request's scores, ties to the lower
// index, indices ascending.
//
// The select kernel (topk.hip) runs it with one workgroup per row; the
// latent attention (attn.hip) runs it in its prologue when the fused step
// hands it the candidate list instead of a finished selection, so that the
// selection never makes a round trip through a kernel of its own.
#pragma once

#include "common.hpp"

namespace sd {

__device__ __forceinline__ int row_valid_units(const TopkPlan& p, int r) {
  int v = p.n_units;
  if (p.valid) {
    int t = p.valid[r / p.rows_per_valid];
    if (p.unit_div > 1) t = (t + p.unit_div - 1) / p.unit_div;
    v = t < 0 ? 0 : (t > p.n_units ? p.n_units : t);
  }
  return v;
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

__device__ __forceinline__ int find_chunk(const int* excl, int nchunks, int p) {
  // largest c with excl[c] <= p
  int lo = 0, hi = nchunks - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (excl[mid] <= p) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// LDS of one row's select by NT threads: up to CAP candidates staged (more
// are read from global memory on every pass), the level-2 / level-3
// histogram, chunk offsets of per-chunk candidate slices, scan scratch.
template <int NT, int CAP>
struct SelectLds {
  uint32_t ckey[CAP];
  int32_t cidx[CAP];
  uint32_t hs[kHistBins];
  int excl[1025];
  int scan[NT / 64 + 1];
  int res[2];
};

// Select row r of p with the NT threads of the workgroup (every thread must
// call it: it holds block barriers; the row is uniform).  The row's
// candidates are (p.direct) its own valid units, (p.fused) the fused filter's
// single list with b* in p.bstar, or per-chunk slices.  It stages them in LDS
// while counting bits [19:8] of those in bin b*, resolves the last 8 bits
// when the boundary 24-bit prefix is not taken whole, which gives the exact
// k-th key T and how many units equal to T are needed, and then walks the
// candidates in index order with block prefix sums (ties to the lowest
// indices): emit(pos, unit, key) for pos = 0 .. k_eff - 1, each once, and
// pad(pos) for k_eff <= pos < k.  SPEC * NT list entries of the fused filter
// are loaded together with the count.  No barrier follows the last emit.
template <int NT, int CAP, int SPEC, typename Emit, typename Pad>
__device__ void select_row(const TopkPlan& p, int r, SelectLds<NT, CAP>& L, Emit&& emit,
                           Pad&& pad) {
  const int tid = threadIdx.x;
  const int v = row_valid_units(p, r);
  const int k_eff = min(p.k, v);
  for (int j = k_eff + tid; j < p.k; j += NT) pad(j);
  if (k_eff <= 0) return;

  uint32_t b1;
  int above;
  const int wid = tid >> 6;
  const int lane = tid & 63;

  // level-2 histogram (bits [19:8] of the keys in bin b1), counted while
  // the candidates are staged
  for (int i = tid; i < kHistBins; i += NT) L.hs[i] = 0u;
  uint32_t skey[SPEC];
  int32_t sidx[SPEC];
  int M = 0;
  if (p.direct) {
    // the row is the candidate list: every valid unit, in index order; its
    // top 12 key bits give b* and the count above it
    M = v;
    const float* sr = p.scores + (int64_t)r * p.row_stride;
    __syncthreads();  // hs cleared
    for (int q = tid; q < M; q += NT) {
      const uint32_t key = score_key(sr[q]);
      L.ckey[q] = key;
      L.cidx[q] = q;
      atomicAdd(&L.hs[key >> 20], 1u);
    }
    if (tid == 0) { L.res[0] = 0; L.res[1] = 0; }
    __syncthreads();
    find_bin_from_top<NT>(L.hs, kHistBins, k_eff, L.scan, L.res);
    b1 = (uint32_t)L.res[0];
    above = L.res[1];
    for (int i = tid; i < kHistBins; i += NT) L.hs[i] = 0u;
    __syncthreads();
    for (int q = tid; q < M; q += NT) {
      const uint32_t key = L.ckey[q];
      if ((key >> 20) == b1) atomicAdd(&L.hs[(key >> 8) & 0xFFFu], 1u);
    }
  } else if (p.fused) {
    b1 = p.bstar[2 * r];
    above = (int)p.bstar[2 * r + 1];
    const uint32_t* ck0 = p.cand_key + (int64_t)r * p.n_units;
    const int32_t* ci0 = p.cand_idx + (int64_t)r * p.n_units;
#pragma unroll
    for (int j = 0; j < SPEC; ++j) {
      const int q = tid + j * NT;
      skey[j] = q < p.n_units ? __builtin_nontemporal_load(ck0 + q) : 0u;
      sidx[j] = q < p.n_units ? __builtin_nontemporal_load(ci0 + q) : 0;
    }
    M = min((int)p.cand_total[r], p.n_units);
    __syncthreads();
  } else {
    b1 = p.bstar[2 * r];
    above = (int)p.bstar[2 * r + 1];
    const uint32_t* cc = p.chunk_cnt + (int64_t)r * p.n_chunks;
    for (int base = 0; base < p.n_chunks; base += NT) {
      int c = base + tid;
      int x = c < p.n_chunks ? (int)cc[c] : 0;
      int total;
      int incl = block_inclusive_scan<NT>(x, L.scan, &total);
      if (c < p.n_chunks) L.excl[c] = M + incl - x;
      M += total;
      __syncthreads();
    }
  }
  const uint32_t* ck = p.cand_key + (int64_t)r * p.n_units;
  const int32_t* ci = p.cand_idx + (int64_t)r * p.n_units;
  const int nch = p.n_chunks;
  auto cand_off = [&](int q) -> int64_t {
    if (p.fused) return q;
    int c = find_chunk(L.excl, nch, q);
    return (int64_t)c * kTopkChunk + (q - L.excl[c]);
  };
  // stage the candidates (in index order) in LDS when they fit: the fused
  // filter's single list by all threads, per-chunk slices by wave w copying
  // chunks w, w + NT / 64, ...
  const bool inlds = p.direct || M <= CAP;
  if (p.direct) {
    // staged and counted above
  } else if (inlds && p.fused) {
#pragma unroll
    for (int j = 0; j < SPEC; ++j) {
      const int q = tid + j * NT;
      if (q < M) {
        L.ckey[q] = skey[j];
        L.cidx[q] = sidx[j];
        if ((skey[j] >> 20) == b1) atomicAdd(&L.hs[(skey[j] >> 8) & 0xFFFu], 1u);
      }
    }
    for (int q = tid + SPEC * NT; q < M; q += NT) {
      const uint32_t key = ck[q];
      L.ckey[q] = key;
      L.cidx[q] = ci[q];
      if ((key >> 20) == b1) atomicAdd(&L.hs[(key >> 8) & 0xFFFu], 1u);
    }
  } else if (inlds) {
    for (int c = wid; c < nch; c += NT / 64) {
      const int cnt = (c + 1 < nch ? L.excl[c + 1] : M) - L.excl[c];
      const int dst = L.excl[c];
      for (int i = lane; i < cnt; i += 64) {
        const uint32_t key = ck[(int64_t)c * kTopkChunk + i];
        L.ckey[dst + i] = key;
        L.cidx[dst + i] = ci[(int64_t)c * kTopkChunk + i];
        if ((key >> 20) == b1) atomicAdd(&L.hs[(key >> 8) & 0xFFFu], 1u);
      }
    }
  } else {
    for (int q = tid; q < M; q += NT) {
      const uint32_t key = ck[cand_off(q)];
      if ((key >> 20) == b1) atomicAdd(&L.hs[(key >> 8) & 0xFFFu], 1u);
    }
  }
  auto key_at = [&](int q) -> uint32_t { return inlds ? L.ckey[q] : ck[cand_off(q)]; };
  auto idx_at = [&](int q) -> int32_t { return inlds ? L.cidx[q] : ci[cand_off(q)]; };
  if (tid == 0) { L.res[0] = 0; L.res[1] = 0; }
  __syncthreads();
  find_bin_from_top<NT>(L.hs, kHistBins, k_eff - above, L.scan, L.res);
  const uint32_t b2 = (uint32_t)L.res[0];
  above += L.res[1];
  const uint32_t pre = (b1 << 12) | b2;
  // When every key of the boundary 24-bit prefix is needed (the usual case),
  // the prefix itself is the threshold and the last level is skipped.
  const bool whole_prefix = (int)L.hs[b2] == k_eff - above;
  __syncthreads();

  uint32_t T;      // threshold on key >> shift
  int shift;
  int eq_need, eq_total;
  if (whole_prefix) {
    T = pre;
    shift = 8;
    eq_need = eq_total = k_eff - above;
  } else {
    // level 3: bits [7:0] of the keys with prefix (b1, b2)
    for (int i = tid; i < 256; i += NT) L.hs[i] = 0u;
    __syncthreads();
    for (int q = tid; q < M; q += NT) {
      uint32_t key = key_at(q);
      if ((key >> 8) == pre) atomicAdd(&L.hs[key & 0xFFu], 1u);
    }
    if (tid == 0) { L.res[0] = 0; L.res[1] = 0; }
    __syncthreads();
    find_bin_from_top<NT>(L.hs, 256, k_eff - above, L.scan, L.res);
    const uint32_t d3 = (uint32_t)L.res[0];
    T = (pre << 8) | d3;
    shift = 0;
    eq_need = k_eff - (above + L.res[1]);
    eq_total = (int)L.hs[d3];
    __syncthreads();
  }

  // final ordered pass, 4 consecutive candidates per thread per round
  int eq_carry = 0, take_carry = 0;
  const bool all_ties = (eq_total == eq_need);
  for (int base = 0; base < M; base += 4 * NT) {
    const int q0 = base + 4 * tid;
    uint32_t key[4];
    int gt[4], eq[4];
    int n_eq = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = q0 + i;
      key[i] = q < M ? key_at(q) : 0u;
      gt[i] = (q < M) && (key[i] >> shift) > T;
      eq[i] = (q < M) && (key[i] >> shift) == T;
      n_eq += eq[i];
    }
    int take[4];
    if (all_ties) {
#pragma unroll
      for (int i = 0; i < 4; ++i) take[i] = gt[i] | eq[i];
    } else {
      int total;
      int incl = block_inclusive_scan<NT>(n_eq, L.scan, &total);
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
    int incl = block_inclusive_scan<NT>(n_take, L.scan, &total);
    int pos = take_carry + incl - n_take;
    take_carry += total;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (take[i] && pos < k_eff) {
        emit(pos, idx_at(q0 + i), key[i]);
        ++pos;
      }
    }
  }
}

}  // namespace sd
