// Hot-buffer replacement after a decode step.
//
// "XM-Sparse: Pushing the Throughput Frontier of Sparse Attention with Netpreme
// X-Mem", Figure 1 and the decode-path list: each request keeps a hot KV buffer
// in HBM and a step fetches only its missing selected rows.  The page keeps
// HiSparse's cache management without stating its rule; the rule here is
// least recently used:
//   * a selected token held in a slot (a hit) stamps the slot with `step`;
//   * the missed tokens, in selection order, take the slots not stamped
//     `step` with the smallest (stamp, slot) -- an empty slot has stamp -1 --
//     in ascending slot order; the slot's old token loses its slot and the
//     miss's row, staged in the workspace by the step, is copied in;
//   * misses beyond the slots available stay out.
//
// One workgroup per request:
//   1. keys of the request's slots into LDS (stamp + 1; the two largest
//      values mark slots that are not eligible); hits take the top mark and
//      the misses are compacted in selection order (block scans);
//   2. the need-th smallest key by radix select (four 8-bit digits, LDS
//      histograms, the digit found by one wave), then the victims in slot
//      order: keys below it, and the lowest slots among the keys equal to it;
//   3. the maps are updated, the staged rows copied and the stamps written.
//
// The same kernel runs the prefetch (staging NULL), which preloads rows the
// next steps are likely to select.  The pages keep HiSparse's prefetch
// mechanism without stating it, and CXL-SpecKV's abstract names speculative
// preloading of the entries future tokens will use; here the caller names
// the candidates (e.g. the tokens ranked just below the top-k), and:
//   * a resident candidate is left as it is (neither replaced nor stamped);
//   * the other candidates, in list order, take the slots neither stamped
//     `step` nor holding a resident candidate, smallest (stamp, slot) first,
//     in ascending slot order; rows come from the pinned host KV and the
//     filled slots are stamped `step`;
//   * candidates beyond the slots available stay out.
#include "common.hpp"

namespace sd {

constexpr int kHotThreads = 1024;
constexpr uint32_t kKeyUsed = 0xFFFFFFFFu;  // hit or filled by this update
constexpr uint32_t kKeyLater = 0xFFFFFFFEu; // stamp at or past `step`: kept

__global__ __launch_bounds__(kHotThreads) void hot_update_kernel(HotPlan p) {
  __shared__ uint32_t key_s[kHotMaxSlots];
  __shared__ int32_t mtok_s[kHotMaxSel];  // missed tokens, selection order
  __shared__ int32_t mpos_s[kHotMaxSel];  // their selection positions
  __shared__ int32_t vic_s[kHotMaxSel];   // victim slots, ascending
  __shared__ uint32_t hist_s[256];
  __shared__ int scan_s[kHotThreads / 64 + 1];
  __shared__ int res_s[2];

  const sparse_attn_args& A = p.a;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int S = p.n_slots;
  const int K = p.k_tokens;
  int32_t* hs = (int32_t*)A.hot_slot + (int64_t)b * A.hs_stride_b;
  int32_t* st = p.slot_token + (int64_t)b * S;
  int32_t* ss = p.slot_stamp + (int64_t)b * S;
  const int32_t* selrow = p.sel + (int64_t)b * p.k;
  const int valid = valid_tokens(A, b);
  const bool prefetch = p.staging == nullptr;
  // a hit is stamped by the update; a resident prefetch candidate is only
  // kept out of the eligible set
  const uint32_t hit_key = prefetch ? kKeyLater : kKeyUsed;

  for (int s = tid; s < S; s += kHotThreads) {
    const int32_t stamp = ss[s];
    key_s[s] = stamp < p.step ? (uint32_t)(stamp + 1) : kKeyLater;
  }
  __syncthreads();

  // hits and misses; a hit's slot leaves the eligible set
  int M = 0;
  for (int base = 0; base < K; base += kHotThreads) {
    const int j = base + tid;
    int t = -1;
    bool miss = false;
    if (j < K) {
      t = sel_token(selrow, j, p.sel_unit, valid);
      if (t >= 0) {
        const int s = hs[t];
        if (s < 0) miss = true;
        else if (s < S) key_s[s] = hit_key;  // (a slot past S is not ours to touch)
      }
    }
    int total;
    const int incl = block_inclusive_scan<kHotThreads>(miss ? 1 : 0, scan_s, &total);
    if (miss) {
      mtok_s[M + incl - 1] = t;
      mpos_s[M + incl - 1] = j;
    }
    M += total;
  }
  __syncthreads();

  // eligible slots and the number of victims
  int E = 0;
  for (int base = 0; base < S; base += kHotThreads) {
    const int s = base + tid;
    int total;
    block_inclusive_scan<kHotThreads>((s < S && key_s[s] < kKeyLater) ? 1 : 0, scan_s, &total);
    E += total;
  }
  const int need = min(M, E);

  if (need > 0) {
    // radix select of the need-th smallest key (every eligible key is below
    // the two marks, so it is an eligible one)
    uint32_t prefix = 0;
    int rem = need;
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int i = tid; i < 256; i += kHotThreads) hist_s[i] = 0u;
      __syncthreads();
      const uint32_t hi_mask = shift == 24 ? 0u : (0xFFFFFFFFu << (shift + 8));
      for (int s = tid; s < S; s += kHotThreads) {
        const uint32_t key = key_s[s];
        if ((key & hi_mask) == prefix) atomicAdd(&hist_s[(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (tid < 64) {
        // lane l holds digits 4l .. 4l + 3
        const int c0 = (int)hist_s[4 * tid], c1 = (int)hist_s[4 * tid + 1];
        const int c2 = (int)hist_s[4 * tid + 2], c3 = (int)hist_s[4 * tid + 3];
        const int sum = c0 + c1 + c2 + c3;
        const int incl = wave_incl_scan(sum);
        const int excl = incl - sum;
        if (excl < rem && incl >= rem) {
          int below = excl, d = 4 * tid;
          const int cs[4] = {c0, c1, c2, c3};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (below + cs[i] >= rem) {
              d = 4 * tid + i;
              break;
            }
            below += cs[i];
          }
          res_s[0] = d;
          res_s[1] = below;
        }
      }
      __syncthreads();
      prefix |= (uint32_t)res_s[0] << shift;
      rem -= res_s[1];
      __syncthreads();
    }
    // victims in slot order: keys below the threshold, then the first `rem`
    // slots holding it
    const uint32_t T = prefix;
    int eq_carry = 0, vic_carry = 0;
    for (int base = 0; base < S; base += kHotThreads) {
      const int s = base + tid;
      const uint32_t key = s < S ? key_s[s] : kKeyUsed;
      const bool eq = key == T;
      int total;
      const int eq_incl = block_inclusive_scan<kHotThreads>(eq ? 1 : 0, scan_s, &total);
      const bool vic = key < T || (eq && eq_carry + eq_incl - 1 < rem);
      eq_carry += total;
      const int v_incl = block_inclusive_scan<kHotThreads>(vic ? 1 : 0, scan_s, &total);
      if (vic && vic_carry + v_incl - 1 < need) vic_s[vic_carry + v_incl - 1] = s;
      vic_carry += total;
    }
    __syncthreads();

    // pair victim i with miss i: maps first, then the rows
    for (int i = tid; i < need; i += kHotThreads) {
      const int v = vic_s[i];
      const int t = mtok_s[i];
      const int u = st[v];
      if (u >= 0 && u < A.n) hs[u] = -1;
      hs[t] = v;
      st[v] = t;
      key_s[v] = kKeyUsed;
    }
    const int cpr = A.d_qk * 2 / 16;  // 16-byte chunks per row
    char* hot = (char*)A.hot_kv + (int64_t)b * A.hot_stride_b * 2;
    if (prefetch) {
      // rows straight from the pinned host KV (device alias, over PCIe)
      const char* host = (const char*)A.host_kv + (int64_t)b * A.host_stride_b * 2;
      for (int q = tid; q < need * cpr; q += kHotThreads) {
        const int i = q / cpr, c = q % cpr;
        const uint4 x = *(const uint4*)(host + ((int64_t)mtok_s[i] * A.host_stride_t * 2 + 16 * c));
        *(uint4*)(hot + (int64_t)vic_s[i] * A.hot_stride_s * 2 + 16 * c) = x;
      }
    } else {
      const char* stage = (const char*)(p.staging + (int64_t)b * K * A.d_qk);
      for (int q = tid; q < need * cpr; q += kHotThreads) {
        const int i = q / cpr, c = q % cpr;
        const uint4 x = *(const uint4*)(stage + ((int64_t)mpos_s[i] * A.d_qk * 2 + 16 * c));
        *(uint4*)(hot + (int64_t)vic_s[i] * A.hot_stride_s * 2 + 16 * c) = x;
      }
    }
  }
  __syncthreads();
  for (int s = tid; s < S; s += kHotThreads)
    if (key_s[s] == kKeyUsed) ss[s] = p.step;
}

hipError_t launch_hot_update(const HotPlan& p, hipStream_t s) {
  hot_update_kernel<<<p.a.batch, kHotThreads, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace sd
