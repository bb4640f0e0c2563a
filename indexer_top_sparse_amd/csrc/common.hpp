// Shared device/host helpers of the sparse decode library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sparse_decode.h"

namespace sd {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

constexpr int kTopkChunk = 4096;
constexpr int kHistBins = 4096;
// Histograms of the first radix digit (the top 12 key bits) are written in
// parts: every producing workgroup stores its own 4096 16-bit counts (two
// per 32-bit word), so no global atomics and no clearing are needed, and
// the bin kernel sums the parts of a row.  A part never counts more than
// kHistPartMax units.
constexpr int kHistWords = kHistBins / 2;
constexpr int kHistPartMax = 65535;
// Each part is followed by kCoarseBins 32-bit coarse counts (sums of 64
// consecutive bins), so that a consumer finds the boundary bin from the
// coarse counts and the 64 bins of one coarse bin instead of all 4096.
constexpr int kCoarseBins = 64;
constexpr int kHistPartWords = kHistWords + kCoarseBins;
// Rows whose parts are at most this many contiguous unit spans take the
// fused filter (no separate bin kernel).
constexpr int kFuseMaxParts = 64;
// Rows of at most this many units skip the histogram and filter kernels:
// the select kernel stages the whole row in LDS and finds b* itself.
constexpr int kTopkDirectMax = 12288;

// Pointer into the global address space: loads through it compile to
// global_load (vector memory counter only) rather than flat_load.
template <typename T>
using gptr = __attribute__((address_space(1))) T*;

// ---------------------------------------------------------------- numbers
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// Order-preserving map of an fp32 score to an unsigned key: a larger float
// gives a larger key; -0 is folded onto +0 so that equal values tie.
__device__ __forceinline__ uint32_t score_key(float x) {
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_score(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

// Store an LDS histogram h[kHistBins] as one part: the 16-bit counts in
// pairs, then the coarse counts.  Needs at least 256 threads (whole waves).
__device__ __forceinline__ void store_hist_part(const uint32_t* h, uint32_t* part, int nt) {
  for (int i = threadIdx.x; i < kHistWords; i += nt) part[i] = h[2 * i] | (h[2 * i + 1] << 16);
  if (threadIdx.x < 4 * kCoarseBins) {
    const int c = threadIdx.x >> 2, q = threadIdx.x & 3;
    uint32_t s = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) s += h[64 * c + 16 * q + i];
    s += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)s, 0xB1, 0xF, 0xF, false);  // quad [1,0,3,2]
    s += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)s, 0x4E, 0xF, 0xF, false);  // quad [2,3,0,1]
    if (q == 0) part[kHistWords + c] = s;
  }
}

// Cross-half exchange: value of lane l ^ 32.
__device__ __forceinline__ float swap_halves(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v),
                                            __float_as_uint(v), false, false);
  uint32_t o = (threadIdx.x & 32) ? r[0] : r[1];
  return __uint_as_float(o);
}

// Inclusive prefix sum over the 64 lanes of a wave, entirely in DPP: shifts
// by 1, 2, 4 and 8 within each row of 16 lanes (lanes shifted past the row
// start add 0), then the row totals carried by the row broadcasts of lane 15
// (into rows 1 and 3) and lane 31 (into rows 2 and 3).
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return x;
}
// Sum over the wave, in every lane.
__device__ __forceinline__ int wave_sum(int x) {
  return __builtin_amdgcn_readlane(wave_incl_scan(x), 63);
}

// Value of lane l ^ m (m a power of two below 64, known at compile time
// once the caller's loop is unrolled): quad permutes for 1 and 2, a
// half-row mirror then a quad reverse for 4, a row mirror then a half-row
// mirror for 8, and the 16- and 32-lane swaps.
__device__ __forceinline__ uint32_t lane_xor_u32(uint32_t v, int m) {
  const int x = (int)v;
  switch (m) {
    case 1: return (uint32_t)__builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false);
    case 2: return (uint32_t)__builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false);
    case 4: {
      const int y = __builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, false);
      return (uint32_t)__builtin_amdgcn_update_dpp(0, y, 0x1B, 0xF, 0xF, false);
    }
    case 8: {
      const int y = __builtin_amdgcn_update_dpp(0, x, 0x140, 0xF, 0xF, false);
      return (uint32_t)__builtin_amdgcn_update_dpp(0, y, 0x141, 0xF, 0xF, false);
    }
    case 16: {
      auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
      return (threadIdx.x & 16) ? r[0] : r[1];
    }
    default: {
      auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
      return (threadIdx.x & 32) ? r[0] : r[1];
    }
  }
}

// ------------------------------------------------------ selection helpers
// Valid tokens of request b of the attention arguments.
__device__ __forceinline__ int valid_tokens(const sparse_attn_args& a, int b) {
  if (!a.seq_lens) return a.n;
  int v = a.seq_lens[b];
  return v < 0 ? 0 : (v > a.n ? a.n : v);
}

// Token of selection list position j (-1 if padding or past seq_len).
__device__ __forceinline__ int sel_token(const int32_t* selrow, int j, int unit,
                                         int valid) {
  int u = selrow[j / unit];
  if (u < 0) return -1;
  int t = u * unit + (j % unit);
  return t < valid ? t : -1;
}

// ---------------------------------------------------------------- block scan
// Inclusive prefix sum over a block of NT threads (NT multiple of 64).
// `lds` must hold NT/64 + 1 ints.  Returns the inclusive sum for the thread
// and writes the block total to *total.
template <int NT>
__device__ __forceinline__ int block_inclusive_scan(int v, int* lds,
                                                    int* total) {
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int x = wave_incl_scan(v);
  if (lane == 63) lds[wid] = x;
  __syncthreads();
  if (wid == 0) {
    const int w = wave_incl_scan(lane < NW ? lds[lane] : 0);
    if (lane < NW) lds[lane] = w;
  }
  __syncthreads();
  int prefix = wid > 0 ? lds[wid - 1] : 0;
  *total = lds[NW - 1];
  __syncthreads();
  return x + prefix;
}

}  // namespace sd

// ---------------------------------------------------------------- launchers
// Internal launch helpers implemented in the kernel translation units.  All
// return hipError_t of the launch.
namespace sd {

struct TopkPlan {
  int rows, n_units, k, n_chunks, rows_per_valid;
  int64_t row_stride;
  const float* scores;
  const int32_t* valid;
  int32_t unit_div;  // valid units = ceil(valid / unit_div)
  uint32_t* hist;    // [rows][parts][kHistPartWords]: 16-bit counts in pairs, coarse counts
  int parts;         // histogram parts per row
  int part_span;     // units per part (part q: units [q span, (q + 1) span))
  int fused;         // candidates in one contiguous list per row (fused filter)
  int direct;        // rows of <= kTopkDirectMax units: the select alone, on the scores
  uint32_t* bstar;   // [rows][2]: boundary bin b*, units in higher bins
  uint32_t* cand_total;  // [rows]: candidates of the row (fused filter)
  uint32_t* cand_key;  // [rows][n_units]
  int32_t* cand_idx;   // [rows][n_units]
  uint32_t* chunk_cnt; // [rows][n_chunks]
  int32_t* idx_out;
  float* val_out;
};


hipError_t launch_topk_hist(const TopkPlan& p, hipStream_t s);
hipError_t launch_topk_bin(const TopkPlan& p, hipStream_t s);
hipError_t launch_topk_filter(const TopkPlan& p, hipStream_t s);
hipError_t launch_topk_filter_fused(const TopkPlan& p, hipStream_t s);
hipError_t launch_topk_select(const TopkPlan& p, hipStream_t s);

struct ScorePlan {
  const sparse_index_args* a;
  float* scores;     // [B][R][n_units]
  uint32_t* hist;    // [B*R][score_hist_parts][kHistWords] (nullable)
  int n_units;
};
// Histogram parts per row that the score kernel of `a` writes, and the
// units each covers (0 when a part is not one contiguous span).
int score_hist_parts(const sparse_index_args& a);
int score_part_span(const sparse_index_args& a);
hipError_t launch_score_dot(const ScorePlan& p, hipStream_t s);
hipError_t launch_score_lightning(const ScorePlan& p, hipStream_t s);
hipError_t launch_read_depth(const sparse_index_args* a, int8_t* depth, hipStream_t s);
hipError_t launch_score_bitplane(const ScorePlan& p, hipStream_t s);

struct AttnPlan {
  sparse_attn_args a;   // by value: kernels read it from their arguments
  const int32_t* sel;
  int sel_heads, k, sel_unit;
  float* out;
  float* lse;
  int splits;         // token splits per (request, head group)
  float* part;        // [B][Hq][splits][d_v + 4] partials when splits > 1:
                      // d_v unnormalised sums, then max, sum, 2 pad
  // hot buffer: staging of fetched rows [B][k_tokens][d_qk] bf16
  uint16_t* staging;
  int k_tokens;       // selected tokens per (request, sel row)
  // fused step, latent rows (attn_selects): the attention selects each
  // request's top-k itself from the fused filter's candidates (tk) and
  // writes the selection to sel_out [B][k]; sel is then unused
  int fsel;
  int32_t* sel_out;
  TopkPlan tk;
};
// Whether the attention over these arguments can take the selection from the
// fused filter's candidates itself (latent rows, no hot buffer).
bool attn_selects(const sparse_attn_args& a);
hipError_t launch_attn_f32(const AttnPlan& p, hipStream_t s);
hipError_t launch_attn_bf16(const AttnPlan& p, hipStream_t s);
hipError_t launch_attn_combine(const AttnPlan& p, hipStream_t s);
hipError_t launch_miss_fetch(const AttnPlan& p, hipStream_t s);
// Hot-buffer replacement after a step (hot.hip).
constexpr int kHotMaxSlots = 8192;  // slots per request
constexpr int kHotMaxSel = 4096;    // selected tokens per request
struct HotPlan {
  sparse_attn_args a;          // hot_slot and hot_kv are written
  const int32_t* sel;          // [B][k] the step's selection
  int k, sel_unit, k_tokens;
  int n_slots, step;
  int32_t* slot_token;         // [B][n_slots] token held, or -1
  int32_t* slot_stamp;         // [B][n_slots] step of the last use
  const uint16_t* staging;     // [B][k_tokens][d_qk] the step's fetched rows;
                               // NULL: a prefetch, rows from host_kv
};
hipError_t launch_hot_update(const HotPlan& p, hipStream_t s);
hipError_t launch_append(const sparse_index_args* ia, const sparse_attn_args* aa,
                         const int32_t* pos, const float* key_new, const void* k_new,
                         const void* v_new, int batch, hipStream_t s);

}  // namespace sd
