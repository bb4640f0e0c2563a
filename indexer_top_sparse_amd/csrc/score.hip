// Index scores (step a2) and Fathom read depth (step a1).
//
// Every kernel here streams the HBM-resident index once, keeps the query in
// registers, writes fp32 unit scores and, when asked, counts each valid
// unit's top-12-bit key in a 4096-bin LDS histogram (the first radix digit
// of the top-k select) that the workgroup stores as its own part of the
// row's histogram, so the select never re-reads the scores for it.
#include <algorithm>

#include "common.hpp"

namespace sd {

// max(0, x) as one integer max on the bit pattern: non-negative floats are
// non-negative integers, negative floats (and -0) are negative integers.
// Unlike fmaxf it needs no NaN canonicalisation of MFMA results.
__device__ __forceinline__ float relu_bits(float x) {
  return __int_as_float(max(__float_as_int(x), 0));
}

// Per-workgroup histogram in LDS, stored as one part of its row's
// histogram: 16-bit counts, two per word (a workgroup counts at most
// kHistPartMax units).  clear() ends with a barrier.
struct LdsHist {
  uint32_t* h;
  __device__ void clear(int nt) {
    for (int i = threadIdx.x; i < kHistBins; i += nt) h[i] = 0u;
    __syncthreads();
  }
  __device__ void add(float s) { atomicAdd(&h[score_key(s) >> 20], 1u); }
  __device__ void store(uint32_t* part, int nt) { store_hist_part(h, part, nt); }
};

__device__ __forceinline__ int valid_len(const int32_t* seq_lens, int b,
                                         int n) {
  if (!seq_lens) return n;
  int v = seq_lens[b];
  return v < 0 ? 0 : (v > n ? n : v);
}

// ========================================================================
// DOT: s_t = sum_h q_h . k_t  (= q_bar . k_t, q_bar = sum_h q_h formed once
// in fp64 and rounded to fp32), optional max over 64-token blocks.
//
// A wave streams 64-token tiles with fully coalesced non-temporal 16-byte
// loads: LPR lanes cover one row (16 for 256-byte bf16 rows, 32 for 512-byte
// fp32 rows), so load j of a tile holds rows RPI j .. RPI j + RPI - 1
// (RPI = 64 / LPR) and a lane always reads the same 16-byte column chunk c,
// whose q_bar values it keeps in registers.  After the LPR loads a lane
// holds LPR partial dots (one per load); a reduce-scatter over the LPR lanes
// of a row -- exchanges by DPP row rotate / mirror / quad permutes and one
// 16-lane swap, no LDS -- leaves lane l with the full dot of tile row
// RPI (l % LPR) + l / LPR.  bf16 tiles are double buffered in registers.
// ========================================================================
template <typename T>
struct DotTraits;
template <>
struct DotTraits<float> {
  static constexpr int kLPR = 32;  // 128 fp32 = 512 B = 32 x 16 B
  static constexpr int kPerLoad = 4;
  static constexpr int kStages = 1;
};
template <>
struct DotTraits<uint16_t> {
  static constexpr int kLPR = 16;  // 128 bf16 = 256 B = 16 x 16 B
  static constexpr int kPerLoad = 8;
  static constexpr int kStages = 2;
};

__device__ __forceinline__ void unpack16(const u32x4& v, float* x) {  // 4 fp32
  x[0] = __uint_as_float(v[0]); x[1] = __uint_as_float(v[1]);
  x[2] = __uint_as_float(v[2]); x[3] = __uint_as_float(v[3]);
}
__device__ __forceinline__ void unpack16_bf16(const u32x4& v, float* x) {  // 8 bf16
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(v[i] << 16);
    x[2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u);
  }
}

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float lane_xor16(float v) {  // value of lane l ^ 16
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float((threadIdx.x & 16) ? r[0] : r[1]);
}

// One halving step of the reduce-scatter over N partials: partner lanes
// (given by XCH) exchange halves; a lane with `up` keeps the upper half.
template <int N, typename F>
__device__ __forceinline__ void rs_step(float* p, bool up, F xch) {
#pragma unroll
  for (int i = 0; i < N / 2; ++i) {
    const float keep = up ? p[i + N / 2] : p[i];
    const float send = up ? p[i] : p[i + N / 2];
    p[i] = keep + xch(send);
  }
}

template <int LPR>
__device__ __forceinline__ float reduce_scatter(float (&p)[LPR], int lane) {
  float* q = p;
  if constexpr (LPR == 32) rs_step<32>(q, lane & 16, [](float v) { return lane_xor16(v); });
  rs_step<16>(q, lane & 8, [](float v) { return dpp_mov<0x128>(v); });  // row_ror:8 = lane ^ 8
  rs_step<8>(q, lane & 4, [](float v) { return dpp_mov<0x141>(v); });   // half-row mirror
  rs_step<4>(q, lane & 2, [](float v) { return dpp_mov<0x4E>(v); });    // lane ^ 2
  rs_step<2>(q, lane & 1, [](float v) { return dpp_mov<0xB1>(v); });    // lane ^ 1
  return q[0];
}

__device__ __forceinline__ float wave_max(float m) {
  m = fmaxf(m, dpp_mov<0xB1>(m));
  m = fmaxf(m, dpp_mov<0x4E>(m));
  m = fmaxf(m, dpp_mov<0x141>(m));
  m = fmaxf(m, dpp_mov<0x128>(m));
  m = fmaxf(m, lane_xor16(m));
  m = fmaxf(m, swap_halves(m));
  return m;
}

constexpr int kDotThreads = 256;
constexpr int kDotWaves = kDotThreads / kWave;
constexpr int kDotTile = 64;                       // tokens per wave tile
constexpr int kDotRound = kDotWaves * kDotTile;    // tokens per workgroup round
constexpr int kDotMaxRounds = kHistPartMax / kDotRound;

// Rounds per workgroup: about 512 workgroups in all, within one histogram
// part's capacity.
int dot_rounds(const sparse_index_args& a) {
  const int64_t rounds_total = (int64_t)a.batch * ((a.n + kDotRound - 1) / kDotRound);
  int64_t r = (rounds_total + 511) / 512;
  return (int)std::min<int64_t>(std::max<int64_t>(r, 1), kDotMaxRounds);
}
int dot_parts(const sparse_index_args& a) {
  const int span = dot_rounds(a) * kDotRound;
  return (a.n + span - 1) / span;
}

template <typename T, int BLOCK>
// (At most 168 VGPRs: three waves per SIMD.  The bf16 block-max variant
// compiled to 169, i.e. two.)
__global__ __launch_bounds__(kDotThreads, 3) void score_dot_kernel(
    sparse_index_args a, float* __restrict__ scores, uint32_t* hist, int n_units,
    int rounds) {
  constexpr int LPR = DotTraits<T>::kLPR;
  constexpr int PL = DotTraits<T>::kPerLoad;
  constexpr int RPI = kWave / LPR;  // rows per load instruction
  constexpr int NS = DotTraits<T>::kStages;
  static_assert(BLOCK == 1 || BLOCK == kDotTile, "block = 1 or one tile");
  __shared__ float qbar_s[128];
  __shared__ uint32_t hist_s[kHistBins];
  LdsHist lh{hist_s};

  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int n = a.n;
  const int valid = valid_len(a.seq_lens, b, n);

  const int c = lane % LPR;  // the 16-byte column chunk this lane reads
  const int g = lane / LPR;  // row within a load instruction
  float qv[PL];

  const char* kb = (const char*)a.keys + (int64_t)b * a.k_stride_b * (int64_t)sizeof(T);
  const int64_t rstride = a.k_stride_t * (int64_t)sizeof(T);
  const int span0 = blockIdx.x * rounds * kDotRound;
  float* srow = scores + (int64_t)b * n_units;

  struct Tile { u32x4 k[LPR]; };
  auto tile_base = [&](int r) { return span0 + (r * kDotWaves + wid) * kDotTile; };
  auto issue = [&](Tile& tl, int r) __attribute__((always_inline)) {
    const int tb = tile_base(r);
#pragma unroll
    for (int j = 0; j < LPR; ++j) {
      int t = tb + RPI * j + g;
      t = t < n ? t : n - 1;
      tl.k[j] = __builtin_nontemporal_load((gptr<const u32x4>)(kb + t * rstride + 16 * c));
    }
  };
  auto consume = [&](const Tile& tl, int r) __attribute__((always_inline)) {
    const int tb = tile_base(r);
    if (tb >= n) return;  // whole tile past the keys (uniform)
    float part[LPR];
#pragma unroll
    for (int j = 0; j < LPR; ++j) {
      float x[PL];
      if constexpr (sizeof(T) == 4) unpack16(tl.k[j], x);
      else unpack16_bf16(tl.k[j], x);
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < PL; ++e) acc = fmaf(qv[e], x[e], acc);
      part[j] = acc;
    }
    const float dot = reduce_scatter<LPR>(part, lane);
    const int t = tb + RPI * c + g;
    const float sc = t < valid ? dot : -__builtin_huge_valf();
    if constexpr (BLOCK == 1) {
      if (t < n) {
        srow[t] = sc;
        if (hist && t < valid) lh.add(sc);
      }
    } else {
      const float m = wave_max(sc);
      const int u = tb / BLOCK;
      if (lane == 0 && u < n_units) {
        srow[u] = m;
        if (hist && tb < valid) lh.add(m);
      }
    }
  };

  // the first tiles' loads go out before q_bar is formed and the histogram
  // cleared, whose latency they then cover
  Tile buf[NS];
#pragma unroll
  for (int st = 0; st < NS; ++st) issue(buf[st], st);

  if (threadIdx.x < 128) {
    double acc = 0.0;
#pragma unroll 8
    for (int h = 0; h < a.n_heads; ++h) {
      const T* qh = (const T*)a.q + (int64_t)b * a.q_stride_b + (int64_t)h * a.q_stride_h;
      float x;
      if constexpr (sizeof(T) == 4) x = qh[threadIdx.x];
      else x = bf16_bits_to_f32(qh[threadIdx.x]);
      acc += (double)x;
    }
    qbar_s[threadIdx.x] = (float)acc;
  }
  if (hist) lh.clear(kDotThreads);  // (ends with a barrier)
  else __syncthreads();
#pragma unroll
  for (int e = 0; e < PL; ++e) qv[e] = qbar_s[c * PL + e];

  for (int r = 0; r < rounds; r += NS) {
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      if (r + st < rounds) consume(buf[st], r + st);
      if (r + st + NS < rounds) issue(buf[st], r + st + NS);
    }
  }
  if (hist) {
    __syncthreads();
    lh.store(hist + ((int64_t)b * gridDim.x + blockIdx.x) * kHistPartWords, kDotThreads);
  }
}

hipError_t launch_score_dot(const ScorePlan& p, hipStream_t s) {
  const sparse_index_args& a = *p.a;
  const int rounds = dot_rounds(a);
  dim3 grid(dot_parts(a), a.batch);
  if (a.k_dtype == SPARSE_F32) {
    if (a.block_size == 1)
      score_dot_kernel<float, 1><<<grid, kDotThreads, 0, s>>>(a, p.scores, p.hist, p.n_units, rounds);
    else
      score_dot_kernel<float, 64><<<grid, kDotThreads, 0, s>>>(a, p.scores, p.hist, p.n_units, rounds);
  } else {
    if (a.block_size == 1)
      score_dot_kernel<uint16_t, 1><<<grid, kDotThreads, 0, s>>>(a, p.scores, p.hist, p.n_units, rounds);
    else
      score_dot_kernel<uint16_t, 64><<<grid, kDotThreads, 0, s>>>(a, p.scores, p.hist, p.n_units, rounds);
  }
  return hipGetLastError();
}

// ========================================================================
// LIGHTNING: s_t = scale_t * sum_h w_h * max(0, q_h . k8_t)
// (scale_t > 0 factors out of the ReLU).  The q.K tile is dense, so it runs
// on MFMA: v_mfma_f32_32x32x16_bf16 with A = q (32 heads x 16 dims), B = the
// fp8 keys converted exactly to bf16 in registers (16 dims x 32 tokens).
//
// A wave streams 32-token tiles (32 x 128 B): four non-temporal loads in
// which the 64 lanes read one contiguous KiB each, so every load instruction
// is fully coalesced.  The tile then passes through a wave-private LDS slot
// (16-byte chunks XOR-swizzled by row to spread the banks) into the MFMA
// layout: lane l owns token l % 32 and dims [64*(l/32), 64*(l/32)+64).  The
// K-dim order inside the MFMA is permuted the same way for q and k, which
// leaves the dot products unchanged.  The accumulator of lane l holds heads
// 32*mt + 8*jj + 4*(l/32) + ii for token l % 32, so the weighted ReLU sum is
// lane-local up to one exchange between the two halves of the wave.
// ========================================================================
constexpr int kLtThreads = 256;
constexpr int kLtStages = 4;        // tiles in flight per wave
constexpr int kLtStride = (kLtThreads / kWave) * 32;  // tokens between a wave's tiles

__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint32_t lo, uint32_t hi) {
  bf16x2 a0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  bf16x2 a1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  bf16x2 a2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  bf16x2 a3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  bf16x8 r;
  r[0] = a0[0]; r[1] = a0[1]; r[2] = a1[0]; r[3] = a1[1];
  r[4] = a2[0]; r[5] = a2[1]; r[6] = a3[0]; r[7] = a3[1];
  return r;
}

// One 32-token tile of a wave: 4 x 16-byte key loads and the token scale.
struct LtTile {
  u32x4 k[4];
  float sc;
};

// TPW: tiles per wave (a multiple of kLtStages); a workgroup covers
// TPW * kLtStride tokens of one request.
template <int H, int TPW>
__global__ __launch_bounds__(kLtThreads) void score_lightning_kernel(
    sparse_index_args a, float* __restrict__ scores, uint32_t* hist,
    int n_units) {
  constexpr int MT = H / 32;  // 32-head MFMA row tiles
  __shared__ uint32_t hist_s[kHistBins];
  __shared__ __attribute__((aligned(16))) u32x4 tile_s[kLtThreads / kWave][256];
  LdsHist lh{hist_s};
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int half = lane >> 5;
  const int col = lane & 31;
  const int n = a.n;
  const int valid = valid_len(a.seq_lens, b, n);

  bf16x8 qa[MT][8];
  float wv[MT][16];
  const uint8_t* kb = (const uint8_t*)a.keys + (int64_t)b * a.k_stride_b;
  const float* ksb = a.k_scale + (int64_t)b * a.ks_stride_b;
  float* srow = scores + (int64_t)b * n_units;
  constexpr int kStride = kLtStride;
  const int t0 = blockIdx.x * (TPW * kLtStride) + wid * 32;
  // tiles of this wave that hold at least one token
  const int ntiles = t0 < n ? min(TPW, (n - t0 + kStride - 1) / kStride) : 0;

  // The K-index is streamed exactly once per step: non-temporal loads keep
  // it from displacing reusable lines in L2 and the last-level cache.
  // Load j, lane l: row 8j + l/8 of the tile, 16-byte chunk l % 8.  The
  // request's keys and scales are read as buffers.  In a wave whose tiles
  // all lie below n, a tile's loads take its first token's byte offset as
  // the scalar offset and a per-lane constant as the vector offset, so no
  // load needs address arithmetic.  The ragged last wave puts the whole
  // offset in the vector operand instead: the buffer's range check then
  // turns every row past n into zeros (their scores are not stored).
  const __amdgpu_buffer_rsrc_t krsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)kb, (short)0, (int)((int64_t)n * a.k_stride_t), 0x00020000);
  const __amdgpu_buffer_rsrc_t srsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)ksb, (short)0, n * 4, 0x00020000);
  uint32_t kvo[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    kvo[j] = (uint32_t)(8 * j + (lane >> 3)) * (uint32_t)a.k_stride_t + 16u * (lane & 7);
  u32x4* slot = tile_s[wid];
  auto issue = [&](LtTile& tl, int it) {
    const uint32_t tb = (uint32_t)(t0 + it * kStride);
    const uint32_t koff = tb * (uint32_t)a.k_stride_t;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      tl.k[j] = __builtin_amdgcn_raw_buffer_load_b128(krsrc, kvo[j], koff, 2 /* nt */);
    tl.sc = __uint_as_float(
        __builtin_amdgcn_raw_buffer_load_b32(srsrc, 4u * col, 4u * tb, 2 /* nt */));
  };
  auto issue_ragged = [&](LtTile& tl, int it) {
    const uint32_t tb = (uint32_t)(t0 + it * kStride);
    const uint32_t koff = tb * (uint32_t)a.k_stride_t;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      tl.k[j] = __builtin_amdgcn_raw_buffer_load_b128(krsrc, kvo[j] + koff, 0, 2 /* nt */);
    tl.sc = __uint_as_float(
        __builtin_amdgcn_raw_buffer_load_b32(srsrc, 4u * (tb + col), 0, 2 /* nt */));
  };
  // Re-layout through LDS: chunk c of row r sits at r*8 + (c ^ (r & 7)).
  auto transpose = [&](const LtTile& tl, u32x4 (&kk)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 8 * j + (lane >> 3);
      slot[r * 8 + ((lane & 7) ^ (r & 7))] = tl.k[j];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = col;
      kk[i] = slot[r * 8 + ((4 * half + i) ^ (r & 7))];
    }
  };

  auto consume = [&](const LtTile& tl, int it) {
    f32x16 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[mt][e] = 0.f;
    u32x4 kk[4];
    transpose(tl, kk);
    const uint32_t* w = (const uint32_t*)kk;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      bf16x8 kv = fp8x8_to_bf16(w[2 * s], w[2 * s + 1]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[mt][s], kv, acc[mt], 0, 0, 0);
    }
    float sum = 0.f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int e = 0; e < 16; ++e) sum = fmaf(wv[mt][e], relu_bits(acc[mt][e]), sum);
    // lanes l and l^32 hold the two halves of the heads of the same token
    float other = swap_halves(sum);
    float total = half ? other + sum : sum + other;
    const int t = t0 + it * kStride + col;
    float s_t = tl.sc * total;
    if (t >= valid) s_t = -__builtin_huge_valf();
    if (half == 0 && t < n) {
      srow[t] = s_t;
      if (hist && t < valid) lh.add(s_t);
    }
  };

  // kLtStages tiles in flight: tile it+kLtStages is issued into the buffer
  // that tile it has just released.  A wave whose tiles are all full runs
  // the loop below, unrolled by kLtStages so every buffer index is a
  // compile-time constant and no load sits behind a branch; each tile then
  // waits for its own loads only.  The ragged last wave of a request takes
  // the guarded loop.
  static_assert(TPW % kLtStages == 0, "whole stage groups");
  LtTile buf[kLtStages];
  const bool full = ntiles == TPW && t0 + (TPW - 1) * kStride + 32 <= n;
  // the first tiles' loads go out before q, the weights and the histogram
  // clear, whose latency they then cover
  if (full) {
#pragma unroll
    for (int s = 0; s < kLtStages; ++s) issue(buf[s], s);
  }
  // A operands: q[32*mt + col][64*half + 8*s + 0..7]
  const uint16_t* qb = (const uint16_t*)a.q + (int64_t)b * a.q_stride_b;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const uint16_t* qh = qb + (int64_t)(32 * mt + col) * a.q_stride_h + 64 * half;
#pragma unroll
    for (int s = 0; s < 8; ++s) qa[mt][s] = *(const bf16x8*)(qh + 8 * s);
  }
  // weights of the heads this lane's accumulators hold
  const float* wb = a.head_w + (int64_t)b * a.w_stride_b;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii)
        wv[mt][4 * jj + ii] = wb[32 * mt + 8 * jj + 4 * half + ii];

  if (hist) lh.clear(kLtThreads);
  if (full) {
    for (int g = 0; g < TPW / kLtStages - 1; ++g) {
#pragma unroll
      for (int s = 0; s < kLtStages; ++s) {
        consume(buf[s], g * kLtStages + s);
        issue(buf[s], (g + 1) * kLtStages + s);
      }
    }
#pragma unroll
    for (int s = 0; s < kLtStages; ++s) consume(buf[s], TPW - kLtStages + s);
  } else {
    for (int it = 0; it < ntiles; ++it) {
      issue_ragged(buf[0], it);
      consume(buf[0], it);
    }
  }
  if (hist) {
    __syncthreads();
    lh.store(hist + ((int64_t)b * gridDim.x + blockIdx.x) * kHistPartWords, kLtThreads);
  }
}

// long spans per workgroup (fewer histogram clears and stores) when the
// batch still gives about two workgroups per compute unit (448: 1.75 per unit
// already beats four times as many short spans)
constexpr int kLtLong = 64, kLtShort = 16;
static_assert(kLtLong * kLtStride <= kHistPartMax, "histogram part overflow");
bool lightning_long(const sparse_index_args& a) {
  const int64_t long_wgs =
      (int64_t)a.batch * ((a.n + kLtLong * kLtStride - 1) / (kLtLong * kLtStride));
  return long_wgs >= 448;
}
int lightning_parts(const sparse_index_args& a) {
  const int span = (lightning_long(a) ? kLtLong : kLtShort) * kLtStride;
  return (a.n + span - 1) / span;
}

hipError_t launch_score_lightning(const ScorePlan& p, hipStream_t s) {
  const sparse_index_args& a = *p.a;
  constexpr int kLong = kLtLong, kShort = kLtShort;
  const bool use_long = lightning_long(a);
  dim3 grid(lightning_parts(a), a.batch);
  if (a.n_heads == 64) {
    if (use_long) score_lightning_kernel<64, kLong><<<grid, kLtThreads, 0, s>>>(a, p.scores, p.hist, p.n_units);
    else score_lightning_kernel<64, kShort><<<grid, kLtThreads, 0, s>>>(a, p.scores, p.hist, p.n_units);
  } else {
    if (use_long) score_lightning_kernel<32, kLong><<<grid, kLtThreads, 0, s>>>(a, p.scores, p.hist, p.n_units);
    else score_lightning_kernel<32, kShort><<<grid, kLtThreads, 0, s>>>(a, p.scores, p.hist, p.n_units);
  }
  return hipGetLastError();
}

// ========================================================================
// Fathom read depth: the selection of one (request, KV head) in one
// workgroup, one thread per (channel, plane) gain.  All arithmetic that
// decides the allocation is float64 with a fixed operation order: q_bar =
// ((q_0 + q_1) + ...), imp = (q_bar * q_bar) * var, gain = imp * 4^-j (an
// exact power-of-two scaling); those are exact for bf16 queries and fp32
// variances, so the ranking (gain desc, channel asc, plane asc) is
// reproducible bit for bit.  read_depth_kernel (sparse_read_depth) writes
// the depths t_c; the bit-plane scan makes the same selection in its
// prologue and turns it into the plane weights W_{c,j} = q_bar_c * cell_c *
// 2^(3-j) of the read planes and the constant sum_c q_bar_c * (zero_c +
// cell_c * 2^(3 - t_c)).
// ========================================================================
constexpr int kDepthThreads = 512;  // D = 128 channels x 4 planes

// LDS of the read-depth selection of one (request, KV head).
struct DepthLds {
  double gain[kDepthThreads];
  double xkey[kDepthThreads];  // second exchange buffer of the sort
  int xid[2][kDepthThreads];   // indices of the two exchange buffers
  double qbar[128];
  double cterm[128];
  int taken[kDepthThreads];
  int scan[kDepthThreads / 64 + 1];
};

// The read depth of (request b, KV head h), left in LDS: L.taken[4c + j] is
// 1 when plane j of channel c is read, L.qbar[c] is q_bar_c and L.cterm[c]
// the channel's score constant q_bar_c * (zero_c + cell_c * 2^(3 - t_c)).
// Thread tid < 512 stands for (channel tid / 4, plane tid % 4) and gets that
// channel's cell width in cell; depth (nullable) receives t_c.  Every thread
// of the NT-thread workgroup must call it (it holds block barriers); it
// ends with a barrier.
template <int NT>
__device__ void depth_select(const sparse_index_args& a, int b, int h, DepthLds& L,
                             float& cell, int8_t* depth) {
  static_assert(NT >= kDepthThreads, "one thread per (channel, plane)");
  const int D = a.head_dim;
  const int Hkv = a.n_kv_heads;
  const int G = a.n_heads / Hkv;
  const int tid = threadIdx.x;
  // waves past the 512 (channel, plane) threads only join the barriers; the
  // test is on the wave's first lane, so those waves branch around the work
  const bool act = __builtin_amdgcn_readfirstlane(tid) < kDepthThreads;
  const int c = (tid & (kDepthThreads - 1)) >> 2;
  const int j = tid & 3;
  const int64_t hd = ((int64_t)b * Hkv + h) * D;
  // every global input first (one round trip): this thread's channel c
  // (variance, or the given depth) and, for tid < D, channel tid's cell and
  // zero point
  const bool fixed = a.depth_in != nullptr;
  const float var_c = (act && !fixed && c < D) ? a.chan_var[hd + c] : 0.f;
  const int din_c = (act && fixed && c < D) ? (int)a.depth_in[hd + c] : 0;
  cell = (act && c < D) ? a.chan_scale[hd + c] : 0.f;
  const float cell_t = tid < D ? a.chan_scale[hd + tid] : 0.f;
  const float zero_t = tid < D ? a.chan_zero[hd + tid] : 0.f;
  if (tid < D) {
    const uint16_t* q0 = (const uint16_t*)a.q + (int64_t)b * a.q_stride_b +
                         (int64_t)(h * G) * a.q_stride_h;
    double acc = (double)bf16_bits_to_f32(q0[tid]);
    for (int gq = 1; gq < G; ++gq)
      acc = __dadd_rn(acc, (double)bf16_bits_to_f32(q0[(int64_t)gq * a.q_stride_h + tid]));
    L.qbar[tid] = acc;
  }
  __syncthreads();
  if (act && !fixed && c < D) {
    double qb = L.qbar[c];
    double imp = __dmul_rn(__dmul_rn(qb, qb), (double)var_c);
    L.gain[tid] = ldexp(imp, -2 * j);
  }
  __syncthreads();
  if (fixed) {
    // a fixed allocation from the caller: planes j < t_c of channel c
    const int tc = c < D ? min(max(din_c, 0), 4) : 0;
    if (act) L.taken[tid] = j < tc;
    __syncthreads();
  } else {
    // Rank every gain in the total order (gain desc, channel asc, plane asc)
    // -- index order tid = 4c + j is (channel, plane) ascending -- with a
    // bitonic sort of (gain, index) pairs: position r of the sorted list
    // holds the gain of rank r.  Slots past 4D hold -1 (below every gain).
    // Steps between lanes of one wave exchange through DPP and lane swaps;
    // only the six steps that cross waves go through LDS and a barrier.
    // (Sorting each wave's 64 pairs and ranking by binary searches in the
    // other waves' sorted lists measured slower.)
    // The steps across waves alternate between two exchange buffers, so
    // each needs one barrier: a buffer is written again two such steps
    // later, after every wave has passed the barrier of the step between.
    double key = (act && c < D) ? L.gain[tid] : -1.0;
    int id = tid;
    int xs = 0;  // steps across waves so far (resolved at compile time)
#pragma unroll
    for (int k = 2; k <= kDepthThreads; k <<= 1) {
#pragma unroll
      for (int jj = k >> 1; jj > 0; jj >>= 1) {
        const int o = tid ^ jj;
        double ko = key;
        int io = id;
        if (jj >= kWave) {  // partner in another wave: through LDS
          double* xk = (xs & 1) ? L.xkey : L.gain;
          int* xi = L.xid[xs & 1];
          if (act) {
            xk[tid] = key;
            xi[tid] = id;
          }
          __syncthreads();
          if (act) {
            ko = xk[o];
            io = xi[o];
          }
          ++xs;
        } else if (act) {  // partner in this wave: DPP / lane swaps, no barrier
          const uint2 kb = __builtin_bit_cast(uint2, key);
          ko = __builtin_bit_cast(double, make_uint2(lane_xor_u32(kb.x, jj), lane_xor_u32(kb.y, jj)));
          io = (int)lane_xor_u32((uint32_t)id, jj);
        }
        if (act) {
          const bool mine_first = (key > ko) || (key == ko && id < io);
          // the lower slot of an ascending block keeps the earlier element
          const bool keep_first = ((tid & k) == 0) == (tid < o);
          if (mine_first != keep_first) { key = ko; id = io; }
        }
      }
    }
    if (act) L.taken[id] = tid < a.bit_budget;  // element id has rank tid
    __syncthreads();
  }
  if (tid < D) {
    const int t = L.taken[4 * tid] + L.taken[4 * tid + 1] + L.taken[4 * tid + 2] +
                  L.taken[4 * tid + 3];
    if (depth) depth[hd + tid] = (int8_t)t;
    L.cterm[tid] = L.qbar[tid] * ((double)zero_t + (double)cell_t * ldexp(1.0, 3 - t));
  }
  __syncthreads();
}

// sum_c cterm_c as a fixed pairwise tree over the 128 channels (level w
// adds entry t + w into entry t), left in L.cterm[0].  Every thread calls
// it; it ends with a barrier.  With D = 128 the first wave holds the
// level-64 sums, one per lane, and the lower levels pair lanes l and l + w
// with lane swaps: the same additions in the same order, without barriers.
__device__ __forceinline__ double lane_xor_f64(double v, int m) {
  const uint2 u = __builtin_bit_cast(uint2, v);
  return __builtin_bit_cast(double, make_uint2(lane_xor_u32(u.x, m), lane_xor_u32(u.y, m)));
}
__device__ __forceinline__ void depth_constant(DepthLds& L, int D) {
  if (D == 2 * kWave) {
    if (threadIdx.x < kWave) {
      double x = L.cterm[threadIdx.x] + L.cterm[threadIdx.x + kWave];
#pragma unroll
      for (int w = kWave / 2; w >= 1; w >>= 1) {
        const double other = lane_xor_f64(x, w);  // lane l + w for l < w
        x = x + other;
      }
      if (threadIdx.x == 0) L.cterm[0] = x;
    }
    __syncthreads();
    return;
  }
  for (int w = D / 2; w >= 1; w >>= 1) {
    if ((int)threadIdx.x < w) L.cterm[threadIdx.x] += L.cterm[threadIdx.x + w];
    __syncthreads();
  }
}

// The depths alone (sparse_read_depth): one workgroup per (request, KV head).
__global__ __launch_bounds__(kDepthThreads) void read_depth_kernel(sparse_index_args a,
                                                                   int8_t* __restrict__ depth) {
  __shared__ DepthLds L;
  float cell_c;
  depth_select<kDepthThreads>(a, blockIdx.y, blockIdx.x, L, cell_c, depth);
}

hipError_t launch_read_depth(const sparse_index_args* a, int8_t* depth, hipStream_t s) {
  dim3 grid(a->n_kv_heads, a->batch);
  read_depth_kernel<<<grid, kDepthThreads, 0, s>>>(*a, depth);
  return hipGetLastError();
}

// ========================================================================
// Fathom plane-prefix scan.  A thread owns one 32-bit word column of a
// (request, KV head): 32 consecutive tokens.  The workgroup first selects
// the read depths itself (depth_select, the same selection as
// read_depth_kernel, repeated by every workgroup of the (request, KV head):
// cheaper than a launch of its own) and turns them into the list of read
// planes (c, j) with their weights and the score constant.  The read planes
// are taken six at a time.  For each group
// of six the workgroup tabulates the 64 sums of their weights W_{c,j} over
// every subset; a thread loads the six plane words (buffer loads, coalesced
// across the workgroup), transposes the 8 x 8 bit blocks of two zero words
// and those six words in registers, after which byte q of word k is four
// times the 6-bit subset index of token 8q + k, and adds one table entry
// per token.  A 64-entry
// table puts every entry in its own LDS bank, so the lookups of a wave
// never conflict: lanes either read different banks or share one entry.
// (Tables of eight-plane groups, 256 entries, cost four to five LDS cycles
// per lookup instruction from bank conflicts, which bounded the scan.)
// The groups are taken sixteen at a time, 96 planes: their sixteen tables
// sit at fixed LDS offsets and are rebuilt between blocks of sixteen
// groups, so every lookup address is the token's index plus a constant.
// ========================================================================
constexpr int kBpThreads = 1024;
constexpr int kBpPassTok = kBpThreads * 32;             // 32768 tokens per workgroup pass
constexpr int kBpMaxPasses = kHistPartMax / kBpPassTok;  // per workgroup (histogram part)
constexpr int kBpGroup = 6;                             // planes per table lookup
constexpr int kBpBlockGroups = 16;                      // groups with resident tables
constexpr int kBpBlockPlanes = kBpGroup * kBpBlockGroups;  // 96
static_assert(kBpBlockGroups * 64 == kBpThreads, "one table entry per thread");

int bitplane_parts(const sparse_index_args& a) {
  const int passes = (a.n + kBpPassTok - 1) / kBpPassTok;
  const int rows = a.batch * a.n_kv_heads;
  // about 256 workgroups (one per compute unit) in all, each within one
  // histogram part's capacity
  int parts = (int)std::max<int64_t>(1, (256 + rows - 1) / std::max(rows, 1));
  parts = std::min(parts, passes);
  parts = std::max(parts, (passes + kBpMaxPasses - 1) / kBpMaxPasses);
  return std::max(parts, 1);
}

// In place: word k of eight, seen as four 8 x 8 bit matrices (byte q of
// the eight words), is replaced by column k of each matrix, i.e. afterwards
// bit j of byte q of w[k] is the old bit 8q + k of w[j].
__device__ __forceinline__ void transpose_bytes8(uint32_t (&w)[8]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t t = ((w[k] >> 4) ^ w[k + 4]) & 0x0F0F0F0Fu;
    w[k + 4] ^= t;
    w[k] ^= t << 4;
  }
#pragma unroll
  for (int k = 0; k < 8; k += (k & 1) ? 3 : 1) {  // 0, 1, 4, 5
    const uint32_t t = ((w[k] >> 2) ^ w[k + 2]) & 0x33333333u;
    w[k + 2] ^= t;
    w[k] ^= t << 2;
  }
#pragma unroll
  for (int k = 0; k < 8; k += 2) {
    const uint32_t t = ((w[k] >> 1) ^ w[k + 1]) & 0x55555555u;
    w[k + 1] ^= t;
    w[k] ^= t << 1;
  }
}

// One LDS buffer carved by hand, so that the tables start at address 0 and
// a group's table base fits the LDS instructions' immediate offset.
constexpr int kBpLdsLut = 0;                                     // [16][64] fp32
constexpr int kBpLdsHist = kBpLdsLut + kBpBlockGroups * 64 * 4;  // [4096] u32
constexpr int kBpLdsPoff = kBpLdsHist + kHistBins * 4;           // [512] u32
constexpr int kBpLdsPw = kBpLdsPoff + 512 * 4;                   // [512] fp32
constexpr int kBpLdsStage = kBpLdsPw + 512 * 4;                  // [16][1024] fp32
constexpr int kBpLdsBytes = kBpLdsStage + (kBpThreads / 64) * 1024 * 4;
static_assert(sizeof(DepthLds) <= kBpLdsBytes - kBpLdsStage && kBpLdsStage % 8 == 0,
              "the read-depth selection fits the staging LDS");

__global__ __launch_bounds__(kBpThreads) void score_bitplane_kernel(
    sparse_index_args a, float* __restrict__ scores, uint32_t* hist, int n_units) {
  __shared__ __attribute__((aligned(16))) char lds[kBpLdsBytes];
  float* lut_s = (float*)(lds + kBpLdsLut);
  uint32_t* poff_s = (uint32_t*)(lds + kBpLdsPoff);  // byte offset of each read plane
  float* pw_s = (float*)(lds + kBpLdsPw);
  LdsHist lh{(uint32_t*)(lds + kBpLdsHist)};
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int D = a.head_dim;
  const int Hkv = a.n_kv_heads;
  const int n = a.n;
  const int nw = (n + 31) / 32;
  const int valid = valid_len(a.seq_lens, b, n);
  const int64_t bh = (int64_t)b * Hkv + h;
  // planes of one (request, KV head) span 4 D nw words (at most 16 MiB), so
  // a plane's byte offset fits 32 bits
  int np;
  float c0;
  {
    // the read depth computed here, in the LDS the score staging uses later:
    // every workgroup of the (request, KV head) repeats the same selection,
    // which costs less than a launch of its own
    DepthLds& L = *(DepthLds*)(lds + kBpLdsStage);
    float cell;
    depth_select<kBpThreads>(a, b, h, L, cell, nullptr);
    const int tid = threadIdx.x;
    const int taken = tid < kDepthThreads && (tid >> 2) < D ? L.taken[tid] : 0;
    int total;
    const int incl = block_inclusive_scan<kBpThreads>(taken, L.scan, &total);
    if (taken) {
      poff_s[incl - 1] = (uint32_t)tid * (uint32_t)nw * 4u;
      pw_s[incl - 1] = (float)(L.qbar[tid >> 2] * (double)cell * ldexp(1.0, 3 - (tid & 3)));
    }
    np = total;
    depth_constant(L, D);
    c0 = (float)L.cterm[0];
    if (hist) lh.clear(kBpThreads);  // (ends with a barrier)
    else __syncthreads();
  }
  // the (request, KV head)'s planes as a buffer: a load takes the plane's
  // byte offset as its scalar offset and the lane's word column as its
  // vector offset, so forming an address costs no vector instruction
  const __amdgpu_buffer_rsrc_t prsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.planes + bh * 4 * D * (int64_t)nw), (short)0, (int)(4u * D * (uint32_t)nw * 4u),
      0x00020000);
  float* srow = scores + bh * n_units;
  const int passes = (n + kBpPassTok - 1) / kBpPassTok;
  const int nblocks = (np + kBpBlockPlanes - 1) / kBpBlockPlanes;
  for (int ps = blockIdx.x; ps < passes; ps += gridDim.x) {
    const int w = ps * kBpThreads + threadIdx.x;
    const int wc = w < nw ? w : nw - 1;  // ragged end: a valid word, result unused
    const uint32_t wcb = 4u * (uint32_t)wc;  // the lane's byte offset in a plane
    float acc[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) acc[i] = c0;
    for (int blk = 0; blk < nblocks; ++blk) {
      const int pb = blk * kBpBlockPlanes;  // first plane of the block
      // the six words of group g of the block: every lane reads the same
      // plane (a wave-uniform base) at its own word column; planes past np
      // (the last group's tail) repeat the last read plane, whose table
      // bits weigh 0
      auto load_group = [&](uint32_t (&wd)[kBpGroup], int g) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < kBpGroup; ++k) {
          const int pi = min(pb + kBpGroup * g + k, np - 1);
          const uint32_t off = __builtin_amdgcn_readfirstlane(poff_s[pi]);
          wd[k] = __builtin_amdgcn_raw_buffer_load_b32(prsrc, wcb, off, 2 /* nt */);
        }
      };
      const int ng = min(kBpBlockGroups, (np - pb + kBpGroup - 1) / kBpGroup);
      // the first two groups' loads go out before the tables are built
      uint32_t ring[3][kBpGroup];
      load_group(ring[0], 0);
      if (ng > 1) load_group(ring[1], 1);
      __syncthreads();  // the previous block's lookups are done
      {
        // table entry e = group e / 64, subset e % 64 of its six planes
        const int g = threadIdx.x >> 6, m = threadIdx.x & 63;
        float x = 0.f;
#pragma unroll
        for (int j = 0; j < kBpGroup; ++j) {
          const int pi = pb + kBpGroup * g + j;
          if (((m >> j) & 1) && pi < np) x += pw_s[pi];
        }
        lut_s[threadIdx.x] = x;
      }
      __syncthreads();
#pragma unroll
      for (int g = 0; g < kBpBlockGroups; ++g) {
        if (g < ng) {
          if (g + 2 < ng) load_group(ring[(g + 2) % 3], g + 2);
          // two zero words, then the six planes: after the transpose bit
          // j + 2 of byte q of w8[k] is plane j's bit of token 8q + k and
          // bits 0 and 1 are zero, so the byte is four times the token's
          // subset index, i.e. its byte offset in group g's table, which
          // starts at LDS address 256 g
          uint32_t w8[8];
          w8[0] = 0u;
          w8[1] = 0u;
#pragma unroll
          for (int k = 0; k < kBpGroup; ++k) w8[2 + k] = ring[g % 3][k];
          transpose_bytes8(w8);
#pragma unroll
          for (int k = 0; k < 8; ++k)
#pragma unroll
            for (int q = 0; q < 4; ++q)
              acc[8 * q + k] +=
                  *(const float*)(lds + kBpLdsLut + 256 * g + ((w8[k] >> (8 * q)) & 0xFFu));
        }
      }
    }
    // A lane holds 32 consecutive tokens, so stores straight from acc would
    // touch 64 cache lines per instruction.  The wave's 2048 tokens pass
    // through its LDS slot instead, 1024 at a time (the lanes of one half,
    // rows of 32 tokens, 16-byte chunks XOR-swizzled by row), and leave as
    // coalesced 256-byte stores.
    float* st = (float*)(lds + kBpLdsStage) + (threadIdx.x >> 6) * 1024;
    const int lane = threadIdx.x & 63;
    const int t_wave = 32 * (w - lane);  // first token of the wave
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      if ((lane >> 5) == r) {
        const int row = lane & 31;
#pragma unroll
        for (int c = 0; c < 8; ++c)
          *(f32x4*)(st + 32 * row + 4 * (c ^ (row & 7))) =
              f32x4{acc[4 * c], acc[4 * c + 1], acc[4 * c + 2], acc[4 * c + 3]};
      }
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int row = 2 * j + (lane >> 5), col = lane & 31;
        const float v = st[32 * row + 4 * ((col >> 2) ^ (row & 7)) + (col & 3)];
        const int t = t_wave + 1024 * r + 64 * j + lane;
        const float sc = t < valid ? v : -__builtin_huge_valf();
        if (t < n) {
          srow[t] = sc;
          if (hist && t < valid) lh.add(sc);
        }
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
  if (hist) {
    __syncthreads();
    lh.store(hist + (bh * gridDim.x + blockIdx.x) * kHistPartWords, kBpThreads);
  }
}

hipError_t launch_score_bitplane(const ScorePlan& p, hipStream_t s) {
  const sparse_index_args& a = *p.a;
  dim3 grid(bitplane_parts(a), a.n_kv_heads, a.batch);
  score_bitplane_kernel<<<grid, kBpThreads, 0, s>>>(a, p.scores, p.hist, p.n_units);
  return hipGetLastError();
}

int score_part_span(const sparse_index_args& a) {
  switch (a.kind) {
    case SPARSE_SCORE_DOT:
      return dot_rounds(a) * kDotRound / (a.block_size == 1 ? 1 : kDotTile);
    case SPARSE_SCORE_LIGHTNING:
      return (lightning_long(a) ? kLtLong : kLtShort) * kLtStride;
    default:
      // a part holds at most one pass, so bitplane_parts gives one part per
      // pass and workgroup x scores the contiguous tokens of pass x
      static_assert(kBpMaxPasses == 1, "one pass per histogram part");
      return kBpPassTok;
  }
}

int score_hist_parts(const sparse_index_args& a) {
  switch (a.kind) {
    case SPARSE_SCORE_DOT: return dot_parts(a);
    case SPARSE_SCORE_LIGHTNING: return lightning_parts(a);
    default: return bitplane_parts(a);
  }
}

}  // namespace sd
