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

// Cross-half exchange: value of lane l ^ 32.
__device__ __forceinline__ float swap_halves(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v),
                                            __float_as_uint(v), false, false);
  uint32_t o = (threadIdx.x & 32) ? r[0] : r[1];
  return __uint_as_float(o);
}

// Reductions over each row of 16 lanes (DPP row rotates and quad perms; no
// LDS round trip).  Every lane of the row receives the result.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp_f<0x128>(x));  // row_ror:8
  x = fmaxf(x, dpp_f<0x124>(x));  // row_ror:4
  x = fmaxf(x, dpp_f<0x4E>(x));   // quad_perm [2,3,0,1]
  x = fmaxf(x, dpp_f<0xB1>(x));   // quad_perm [1,0,3,2]
  return x;
}
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_f<0x128>(x);
  x += dpp_f<0x124>(x);
  x += dpp_f<0x4E>(x);
  x += dpp_f<0xB1>(x);
  return x;
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
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) lds[wid] = x;
  __syncthreads();
  if (wid == 0) {
    int w = lane < NW ? lds[lane] : 0;
#pragma unroll
    for (int off = 1; off < NW; off <<= 1) {
      int y = __shfl_up(w, off, 64);
      if (lane >= off) w += y;
    }
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
  uint32_t* hist;    // [rows][parts][kHistWords] 16-bit counts in pairs
  int parts;         // histogram parts per row
  uint32_t* bstar;   // [rows][2]: boundary bin b*, units in higher bins
  uint32_t* cand_key;  // [rows][n_units]
  int32_t* cand_idx;   // [rows][n_units]
  uint32_t* chunk_cnt; // [rows][n_chunks]
  int32_t* idx_out;
  float* val_out;
};


hipError_t launch_topk_hist(const TopkPlan& p, hipStream_t s);
hipError_t launch_topk_bin(const TopkPlan& p, hipStream_t s);
hipError_t launch_topk_filter(const TopkPlan& p, hipStream_t s);
hipError_t launch_topk_select(const TopkPlan& p, hipStream_t s);

struct ScorePlan {
  const sparse_index_args* a;
  float* scores;     // [B][R][n_units]
  uint32_t* hist;    // [B*R][score_hist_parts][kHistWords] (nullable)
  int n_units;
  int8_t* depth;     // BITPLANE: [B][Hkv][D]
  int32_t* plist;    // BITPLANE: [B][Hkv][4D] read planes (index 4c + j), then
  float* pwl;        //   their weights q_bar_c * cell_c * 2^(3-j)
  int32_t* npl;      //   [B][Hkv] number of read planes
  float* score_c;    // BITPLANE: [B][Hkv] constant term
};
// Histogram parts per row that the score kernel of `a` writes.
int score_hist_parts(const sparse_index_args& a);
hipError_t launch_score_dot(const ScorePlan& p, hipStream_t s);
hipError_t launch_score_lightning(const ScorePlan& p, hipStream_t s);
hipError_t launch_read_depth(const sparse_index_args* a, int8_t* depth, int32_t* plist,
                             float* pwl, int32_t* npl, float* score_c, hipStream_t s);
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
};
hipError_t launch_attn_f32(const AttnPlan& p, hipStream_t s);
hipError_t launch_attn_bf16(const AttnPlan& p, hipStream_t s);
hipError_t launch_attn_combine(const AttnPlan& p, hipStream_t s);
hipError_t launch_miss_fetch(const AttnPlan& p, hipStream_t s);
hipError_t launch_append(const sparse_index_args* ia, const sparse_attn_args* aa,
                         const int32_t* pos, const float* key_new, const void* k_new,
                         const void* v_new, int batch, hipStream_t s);

}  // namespace sd
