// Sparse decode attention over the selected KV rows (steps a4, a5, a6).
//
// "XM-Sparse" blog, opening paragraph: each decode step attends over only
// the selected KV entries.  out_h = sum_i softmax_i(scale * q_h . k_i) v_i
// over the selected rows i, lse_h = log sum_i exp(scale * q_h . k_i).
//
// bf16 path (MFMA): a workgroup owns (request, head group, token split) and
// walks the split's selected tokens in tiles of 32.  Each tile is gathered
// row by row (page table / hot buffer / staging) into LDS with 16-byte
// loads, prefetched into registers one tile ahead.  S = q K^T runs on
// v_mfma_f32_16x16x32_bf16 with q held in registers; an online softmax
// keeps per-head running max and sum; P V runs on the same MFMA with V read
// from LDS as 8-token column strips re-packed in registers.  Splits write
// unnormalised partials that a combine kernel merges by log-sum-exp.
#include "select.hpp"

namespace sd {

struct RowAddr {
  // Resolves token t of request b (KV head h) to its K and V row pointers.
  const sparse_attn_args& a;
  __device__ __forceinline__ const char* k_row(int b, int h, int t, int64_t stage_row,
                                               const uint16_t* staging, int esize) const {
    if (a.hot_slot) {
      int slot = a.hot_slot[(int64_t)b * a.hs_stride_b + t];
      if (slot >= 0)
        return (const char*)a.hot_kv +
               ((int64_t)b * a.hot_stride_b + (int64_t)slot * a.hot_stride_s) * esize;
      return (const char*)(staging + stage_row * a.d_qk);
    }
    int64_t off;
    if (a.page_table) {
      int pg = a.page_table[(int64_t)b * a.pt_stride_b + t / a.page_size];
      off = ((int64_t)pg * a.page_size + t % a.page_size) * a.kv_stride_t;
    } else {
      off = (int64_t)b * a.kv_stride_b + (int64_t)t * a.kv_stride_t;
    }
    off += (int64_t)h * a.kv_stride_h;
    return (const char*)a.k_cache + off * esize;
  }
  __device__ __forceinline__ const char* v_row(int b, int h, int t, int esize) const {
    int64_t off;
    if (a.page_table) {
      int pg = a.page_table[(int64_t)b * a.pt_stride_b + t / a.page_size];
      off = ((int64_t)pg * a.page_size + t % a.page_size) * a.kv_stride_t;
    } else {
      off = (int64_t)b * a.kv_stride_b + (int64_t)t * a.kv_stride_t;
    }
    off += (int64_t)h * a.kv_stride_h;
    return (const char*)a.v_cache + off * esize;
  }
};


// A row of zeros owned by the library, as wide as the widest row the
// kernels read (a 576-element bf16 latent row, a 128-element fp32 row).
// Masked positions (padding entries, tokens past seq_len, the prefetch pad
// past a split's end) point here instead of at caller memory, so that the
// zero probability they get multiplies finite zeros: 0 * NaN would turn a
// whole head's output into NaN when the caller's row holds NaN or infinity
// (an unfilled hot-buffer slot or an unused page).
__device__ __attribute__((aligned(256))) uint16_t g_zero_row[576] = {0};

__device__ __forceinline__ const char* zero_row() { return (const char*)g_zero_row; }

// One halving step of a reduce-scatter over N partials: partner lanes
// (given by xch) exchange halves; a lane with `up` keeps the upper half.
template <int N, typename F>
__device__ __forceinline__ void rs_halve(float* p, bool up, F xch) {
#pragma unroll
  for (int i = 0; i < N / 2; ++i) {
    const float keep = up ? p[i + N / 2] : p[i];
    const float send = up ? p[i] : p[i + N / 2];
    p[i] = keep + xch(send);
  }
}


// =================================================================== fp32
// One workgroup per (request, KV head, group of up to 8 query heads, split);
// d_qk = d_v = 128.  Each K row is read once for all heads of the group:
//   QK: a wave takes one token at a time, lane l holds dims 2l, 2l + 1, and a
//       reduce-scatter over the wave leaves head h's dot in lanes 8h .. 8h+7
//   softmax per head over the split (waves own heads)
//   PV: thread (head, column quad) accumulates p_i v_i over the split.
constexpr int kF32Threads = 256;
constexpr int kF32Heads = 8;
constexpr int kF32MaxTok = 2048;

__device__ __forceinline__ float wave_sum_f(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));
  {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x += __uint_as_float((threadIdx.x & 16) ? r[0] : r[1]);
  }
  return x + swap_halves(x);
}
__device__ __forceinline__ float wave_max_f(float x) {
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false)));
  {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(x, __uint_as_float((threadIdx.x & 16) ? r[0] : r[1]));
  }
  return fmaxf(x, swap_halves(x));
}

__global__ __launch_bounds__(kF32Threads) void attn_f32_kernel(AttnPlan p) {
  __shared__ float q_s[kF32Heads][128];
  __shared__ float logit_s[kF32Heads][kF32MaxTok];
  __shared__ int tok_s[kF32MaxTok];
  __shared__ float ml_s[kF32Heads][2];
  const sparse_attn_args& A = p.a;
  const int split = blockIdx.x;
  const int G = A.n_q_heads / A.n_kv_heads;
  const int ngrp = (G + kF32Heads - 1) / kF32Heads;
  const int kvh = blockIdx.y / ngrp;
  const int hg = blockIdx.y % ngrp;
  const int h0 = kvh * G + hg * kF32Heads;        // first query head
  const int nh = min(kF32Heads, G - hg * kF32Heads);
  const int b = blockIdx.z;
  const int selrow_i = p.sel_heads == 1 ? 0 : kvh;
  const int32_t* selrow = p.sel + ((int64_t)b * p.sel_heads + selrow_i) * p.k;
  const int valid = valid_tokens(A, b);
  const int tps = (p.k_tokens + p.splits - 1) / p.splits;
  const int j0 = split * tps;
  const int j1 = min(j0 + tps, p.k_tokens);
  const int cnt = max(0, j1 - j0);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  RowAddr ra{A};
  const float* qb = (const float*)A.q + (int64_t)b * A.q_stride_b;
  for (int i = tid; i < kF32Heads * 128; i += kF32Threads) {
    const int h = i >> 7;
    q_s[h][i & 127] = h < nh ? qb[(int64_t)(h0 + h) * A.q_stride_h + (i & 127)] : 0.f;
  }
  for (int i = tid; i < cnt; i += kF32Threads) tok_s[i] = sel_token(selrow, j0 + i, p.sel_unit, valid);
  __syncthreads();

  float qr[kF32Heads][2];
#pragma unroll
  for (int h = 0; h < kF32Heads; ++h) {
    qr[h][0] = q_s[h][2 * lane];
    qr[h][1] = q_s[h][2 * lane + 1];
  }
  const int hl = (lane >> 3) & 7;  // head whose dot this lane ends with
  constexpr int kU = 4;  // tokens per wave step, their rows loaded together
  constexpr int kWavesF = kF32Threads / 64;
  for (int i0 = wid * kU; i0 < cnt; i0 += kWavesF * kU) {
    f32x2 kvs[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i = min(i0 + u, cnt - 1);
      const int t = tok_s[i];  // masked positions read the zero row
      const float* kr = t >= 0 ? (const float*)ra.k_row(b, kvh, t, 0, nullptr, 4)
                               : (const float*)zero_row();
      kvs[u] = *(const f32x2*)(kr + 2 * lane);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
    const int i = i0 + u;
    const int t = i < cnt ? tok_s[i] : -1;
    const f32x2 kv = kvs[u];
    float part[kF32Heads];
#pragma unroll
    for (int h = 0; h < kF32Heads; ++h) part[h] = fmaf(qr[h][0], kv[0], qr[h][1] * kv[1]);
    // reduce-scatter over lane bits 5, 4, 3 (upper half kept when set), then
    // sum over lane bits 0..2
    rs_halve<8>(part, lane & 32, [](float v) { return swap_halves(v); });
    rs_halve<4>(part, lane & 16, [](float v) {
      auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
      return __uint_as_float((threadIdx.x & 16) ? r[0] : r[1]);
    });
    rs_halve<2>(part, lane & 8, [](float v) {
      return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));
    });
    float d = part[0];
    d += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(d), 0xB1, 0xF, 0xF, false));
    d += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(d), 0x4E, 0xF, 0xF, false));
    d += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(d), 0x141, 0xF, 0xF, false));
    if ((lane & 7) == 0 && hl < nh && i < cnt)
      logit_s[hl][i] = t >= 0 ? d * A.sm_scale : -__builtin_huge_valf();
    }
  }
  __syncthreads();
  for (int h = wid; h < nh; h += kF32Threads / 64) {
    float m = -__builtin_huge_valf();
    for (int i = lane; i < cnt; i += 64) m = fmaxf(m, logit_s[h][i]);
    m = wave_max_f(m);
    float l = 0.f;
    for (int i = lane; i < cnt; i += 64) {
      const float e = m == -__builtin_huge_valf() ? 0.f : __expf(logit_s[h][i] - m);
      logit_s[h][i] = e;
      l += e;
    }
    l = wave_sum_f(l);
    if (lane == 0) { ml_s[h][0] = m; ml_s[h][1] = l; }
  }
  __syncthreads();
  const int h = tid >> 5;   // head of this thread's output quad
  const int qd = tid & 31;  // columns 4 qd .. 4 qd + 3
  if (h < nh) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int i = 0; i < cnt; ++i) {
      // a masked position has probability 0 and reads the zero row
      const int t = tok_s[i];
      const float* vr = t < 0 ? (const float*)zero_row()
                              : A.v_cache ? (const float*)ra.v_row(b, kvh, t, 4)
                                          : (const float*)ra.k_row(b, kvh, t, 0, nullptr, 4);
      acc += *(const f32x4*)(vr + 4 * qd) * logit_s[h][i];
    }
    const float m = ml_s[h][0], l = ml_s[h][1];
    const int64_t oh = (int64_t)b * A.n_q_heads + h0 + h;
    if (p.splits == 1) {
      *(f32x4*)(p.out + oh * 128 + 4 * qd) = l > 0.f ? acc * (1.f / l) : f32x4{0.f, 0.f, 0.f, 0.f};
      if (qd == 0 && p.lse) p.lse[oh] = l > 0.f ? m + __logf(l) : -__builtin_huge_valf();
    } else {
      float* pp = p.part + (oh * p.splits + split) * (128 + 4);
      *(f32x4*)(pp + 4 * qd) = acc;
      if (qd == 0) { pp[128] = m; pp[129] = l; }
    }
  }
}

hipError_t launch_attn_f32(const AttnPlan& p, hipStream_t s) {
  const int G = p.a.n_q_heads / p.a.n_kv_heads;
  dim3 grid(p.splits, p.a.n_kv_heads * ((G + kF32Heads - 1) / kF32Heads), p.a.batch);
  attn_f32_kernel<<<grid, kF32Threads, 0, s>>>(p);
  return hipGetLastError();
}

// =================================================================== bf16
constexpr int kTT = 32;            // tokens per tile
constexpr int kMaxSplitTok = 2048;  // row-table entries of one split

// ============================================================ latent (MLA)
// Latent rows (d_qk 576, values = the first 512 dims of the same row), one
// KV head, 64 query heads per workgroup in four 16-head blocks.  The eight
// waves split by role, so that on every SIMD a score wave and a P V wave
// overlap instead of running the two phases back to back:
//   score waves 0..3, head block w:
//     S^T[32 tokens x 16 heads] = K_tile Q^T over all 576 dims (A = K rows
//       from LDS, B = q in registers)
//     online softmax per head in the base-2 domain (scores scaled by
//       sm_scale * log2(e)); lane l holds head l % 16 and the four lanes of
//       a head combine with permlane swaps; the bf16 probabilities and the
//       factor that rescales each head's O go to LDS
//   P V waves 4..7, columns [128 c, +128) of all 64 heads:
//     O^T[128 x 16] += V^T P^T per head block (A = V^T read from the
//       row-major tile with the LDS transpose load ds_read_b64_tr_b16, shared
//       by the four head blocks; B = the block's probabilities)
// The token order of the P V contraction is permuted so that the eight
// probabilities a score lane holds (tokens 4g..4g+3 and 16+4g..16+4g+3,
// g = lane / 16) are exactly one lane's B operand.  K tiles rotate through
// three LDS buffers with one more tile in flight in registers, copied by
// all eight waves (a P V thread twice the chunks of a score thread); the
// score waves run one tile ahead of the P V waves.  Probabilities are taken
// relative to a per-head reference max that moves (rescaling O and the
// sum) only when a tile's max exceeds it by more than 2^8.  In the fused
// step the kernel first makes the request's top-k selection itself (FSEL).
constexpr int kMlaWaves = 8;
constexpr int kMlaHeadsWG = 64;
constexpr int kMlaThreads = 64 * kMlaWaves;
// floats in one split record of a (request, 64-head group): 64 x 512 partial
// outputs, then (m, l) per head (m in the base-2 domain)
constexpr int kMlaRec = kMlaHeadsWG * 512 + 2 * kMlaHeadsWG;

// The latent layout the MLA kernel serves (the API validates the head count).
__host__ __device__ inline bool mla_shape(const sparse_attn_args& a) {
  return a.d_qk == 576 && a.d_v == 512 && a.v_cache == nullptr && a.n_kv_heads == 1;
}
constexpr int kMlaRow = 576 + 8;                   // LDS row stride (elements)
constexpr int kMlaChunks = kTT * 72;               // 16-byte chunks per tile
constexpr int kMlaNchS = 3, kMlaNchP = 6;          // per score / P V thread
constexpr int kMlaNch = kMlaNchP;
static_assert(256 * (kMlaNchS + kMlaNchP) == kMlaChunks, "the two roles copy a whole tile");
constexpr int kMlaPad = 3 * kTT;  // row-table entries past a split (prefetch)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float xlane16(float v) {  // value of lane l ^ 16
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v),
                                            false, false);
  return __uint_as_float((threadIdx.x & 16) ? r[0] : r[1]);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
// LDS transpose load: within each 16-lane group, lane i receives element
// i % 4 of the 8-byte pieces addressed by lanes i / 4, 4 + i / 4, 8 + i / 4
// and 12 + i / 4 (in that order).
__device__ __forceinline__ s16x4 lds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(uint16_t*)p);
}

// FSEL: the fused step's selection is made here (see the row table below).
constexpr int kMlaSelCap = 11264;  // candidates of the fused selection staged in LDS
template <bool FSEL>
__global__ __launch_bounds__(kMlaThreads, 1) void attn_mla_kernel(AttnPlan p) {
  __shared__ __attribute__((aligned(16))) uint16_t ks_s[3][kTT * kMlaRow];
  // probabilities of a tile as the P V waves' B operands, [buffer][head block][lane]
  // [buffer][high part, residual][head block][lane]
  __shared__ __attribute__((aligned(16))) bf16x8 pb_s[2][2][4][64];
  __shared__ float alpha_s[2][4][16];  // rescale factor of each head's O for that tile
  __shared__ float ml_s[kMlaHeadsWG][2];
  __shared__ uint64_t rowp_s[kMaxSplitTok + kMlaPad];
  __shared__ uint32_t vmask_s[kMaxSplitTok / kTT];  // valid tokens of each tile

  const sparse_attn_args& A = p.a;
  const int ngrp = A.n_q_heads / kMlaHeadsWG;
  const int unit = (int)(blockIdx.x % 8) + 8 * (int)(blockIdx.x / (8 * ngrp));
  const int grp = (int)(blockIdx.x / 8) % ngrp;
  if (unit >= p.splits * A.batch) return;
  const int split = unit % p.splits;
  const int b = unit / p.splits;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int g = lane >> 4;
  const int n = lane & 15;
  const bool qk_wave = wid < 4;  // waves 0..3: scores and softmax of head block wid
  const int cq = wid & 3;        // waves 4..7: P V for columns [128 cq, +128)
  const int32_t* selrow = p.sel + (int64_t)b * p.sel_heads * p.k;
  const int valid = valid_tokens(A, b);
  const int tps = (p.k_tokens + p.splits - 1) / p.splits;
  const int j0 = split * tps;
  const int j1 = min(j0 + tps, p.k_tokens);
  const int cnt = max(0, j1 - j0);
  const int ntiles = (cnt + kTT - 1) / kTT;
  const int64_t stage_base = (int64_t)b * p.sel_heads * p.k_tokens;
  RowAddr ra{A};

  if constexpr (FSEL) {
    // The fused step's top-k of request b, from the fused filter's candidate
    // list: every workgroup of the request selects the whole row (the tile
    // buffers, unused until the first gather, hold the select's LDS) and
    // keeps the tokens of its split's positions in rowp_s, which the row
    // table below turns into row addresses in place; head group 0 writes the
    // split's positions of the caller's top-k buffer.  This takes the place
    // of the select kernel and of the round trip through that buffer.
    static_assert(sizeof(SelectLds<kMlaThreads, kMlaSelCap>) <= sizeof(ks_s),
                  "the select's LDS fits in the tile buffers");
    auto& SL = *reinterpret_cast<SelectLds<kMlaThreads, kMlaSelCap>*>(&ks_s[0][0]);
    int32_t* so = p.sel_out + (int64_t)b * p.k;
    select_row<kMlaThreads, kMlaSelCap, 8>(
        p.tk, b, SL,
        [&](int pos, int32_t unit_idx, uint32_t) {
          if (pos >= j0 && pos < j1) {
            rowp_s[pos - j0] = (uint64_t)(uint32_t)unit_idx;
            if (grp == 0) so[pos] = unit_idx;
          }
        },
        [&](int pos) {
          if (pos >= j0 && pos < j1) {
            rowp_s[pos - j0] = ~0ull;
            if (grp == 0) so[pos] = -1;
          }
        });
    __syncthreads();
  }

  // Row table: the K row address of every split position (masked positions
  // and the prefetch pad point at the library's zero row, so every load in
  // the pipeline is unconditional) and, per 32-token tile, the valid-token
  // bits.
  const uint64_t dummy = (uint64_t)zero_row();
  for (int base = 0; base < cnt; base += kMlaThreads) {
    const int i = base + tid;
    int t = -1;
    if (i < cnt) {
      if constexpr (FSEL) {
        t = (int32_t)(uint32_t)rowp_s[i];  // the selected token, or -1
        if (t >= valid) t = -1;
      } else {
        t = sel_token(selrow, j0 + i, p.sel_unit, valid);
      }
      rowp_s[i] = t >= 0 ? (uint64_t)ra.k_row(b, 0, t, stage_base + j0 + i, p.staging, 2)
                         : dummy;
    }
    const uint64_t bal = __builtin_amdgcn_ballot_w64(t >= 0);
    const int tile = (base >> 5) + 2 * wid;  // lanes 0..31: tile, 32..63: tile + 1
    if (lane == 0 && tile < ntiles) vmask_s[tile] = (uint32_t)bal;
    if (lane == 0 && tile + 1 < ntiles) vmask_s[tile + 1] = (uint32_t)(bal >> 32);
  }
  for (int i = cnt + tid; i < (ntiles + 3) * kTT; i += kMlaThreads) rowp_s[i] = dummy;

  // gather coordinates: chunk i of this thread is row crow[i], byte offset
  // coff[i] of the row.  A score thread copies kMlaNchS of a tile's 16-byte
  // chunks and a P V thread kMlaNchP: the score waves set the pace of a tile
  // step, so the P V waves take two thirds of the copying (lightning_128k
  // level, hot_16k without misses 2735-2749 -> 2802-2835 steps/s against an
  // even split; 1 : 8 and 2 : 7 were slower than 3 : 6)
  const int nch = qk_wave ? kMlaNchS : kMlaNchP;
  int crow[kMlaNch], coff[kMlaNch];
#pragma unroll
  for (int i = 0; i < kMlaNch; ++i) {
    const int q = qk_wave ? tid + 256 * i : 256 * kMlaNchS + (tid - 256) + 256 * i;
    const int qc = i < nch ? q : 0;
    crow[i] = qc / 72;
    coff[i] = 16 * (qc % 72);
  }

  // Row gathers are non-temporal: the rows are read once per head group,
  // and the two head groups of a split share them through L2 all the same
  // (lightning_128k 5852-5915 -> 6101-6153 steps/s against plain loads).
  auto gather = [&](u32x4 (&pre)[kMlaNch], int tile) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kMlaNch; ++i)
      if (i < nch)
        pre[i] = __builtin_nontemporal_load(
            (gptr<const u32x4>)((const char*)rowp_s[tile * kTT + crow[i]] + coff[i]));
  };
  auto commit = [&](const u32x4 (&pre)[kMlaNch], int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kMlaNch; ++i)
      if (i < nch)
        *(u32x4*)(&ks_s[buf][crow[i] * kMlaRow + (coff[i] >> 1)]) = pre[i];
  };
  // the first three tiles: two in LDS, one in registers
  u32x4 pre[kMlaNch];
  auto prologue = [&]() __attribute__((always_inline)) {
    __syncthreads();  // row table ready
    if (ntiles > 0) {
      u32x4 pre1[kMlaNch];
      gather(pre, 0);
      gather(pre1, 1);
      commit(pre, 0);
      commit(pre1, 1);
      gather(pre, 2);
    }
    __syncthreads();
  };

  // ---- pipeline, one barrier per tile.  In step t the score waves compute
  // the scores and probabilities of tile t+1 (LDS buffer (t+1) % 3) into
  // probability buffer (t+1) % 2 while the P V waves consume tile t (buffer
  // t % 3, probabilities t % 2); every thread writes tile t+2 from
  // registers into buffer (t+2) % 3 and starts loading tile t+3.
  if (qk_wave) {
    // q of head block wid as the B operand: B[k = dim 32 s + 8g + e][n = head]
    const int head = grp * kMlaHeadsWG + 16 * wid + n;
    bf16x8 qb[18];
    {
      const uint16_t* qp = (const uint16_t*)A.q + (int64_t)b * A.q_stride_b +
                           (int64_t)head * A.q_stride_h + 8 * g;
#pragma unroll
      for (int s = 0; s < 18; ++s) qb[s] = *(const bf16x8*)(qp + 32 * s);
    }
    const float qk_scale = A.sm_scale * kLog2e;
    float m_run = -__builtin_huge_valf();  // base-2 reference max
    float l_run = 0.f;
    // S^T[32 tokens x 16 heads] of one tile, online softmax, probabilities
    // into LDS
    auto scores = [&](int tile, int buf, int sb) __attribute__((always_inline)) {
      const uint16_t* kt = ks_s[buf];
      float sv[8];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
        const uint16_t* kr = kt + (16 * mt + n) * kMlaRow + 8 * g;
#pragma unroll
        for (int s = 0; s < 18; ++s) {
          const bf16x8 kv = *(const bf16x8*)(kr + 32 * s);
          if (s & 1) a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, qb[s], a1, 0, 0, 0);
          else a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, qb[s], a0, 0, 0, 0);
          if ((s % 6) == 5) __builtin_amdgcn_sched_barrier(0);  // bound the live K fragments
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) sv[4 * mt + i] = (a0[i] + a1[i]) * qk_scale;
      }
      const uint32_t vm = __builtin_amdgcn_readfirstlane(vmask_s[tile]);
      if (vm != 0xFFFFFFFFu) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (!((vm >> (16 * (e >> 2) + 4 * g + (e & 3))) & 1u)) sv[e] = -__builtin_huge_valf();
      }
      float tmax = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])),
                         fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
      tmax = fmaxf(tmax, xlane16(tmax));
      tmax = fmaxf(tmax, swap_halves(tmax));
      constexpr float kSlack = 8.0f;
      float alpha = 1.f;
      if (__builtin_amdgcn_ballot_w64(tmax > m_run + kSlack)) {
        const float m_new = fmaxf(m_run, tmax);
        alpha = (m_run == -__builtin_huge_valf()) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
        m_run = m_new;
      }
      if (g == 0) alpha_s[sb][wid][n] = alpha;
      const bool none = (m_run == -__builtin_huge_valf());
      float psum = 0.f;
      uint32_t ph[4], pl[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p0 = none ? 0.f : __builtin_amdgcn_exp2f(sv[2 * e] - m_run);
        const float p1 = none ? 0.f : __builtin_amdgcn_exp2f(sv[2 * e + 1] - m_run);
        psum += p0 + p1;
        const bf16x2 hi = bf16x2{(__bf16)p0, (__bf16)p1};
        const bf16x2 lo = bf16x2{(__bf16)(p0 - (float)hi[0]), (__bf16)(p1 - (float)hi[1])};
        ph[e] = __builtin_bit_cast(uint32_t, hi);
        pl[e] = __builtin_bit_cast(uint32_t, lo);
      }
      psum += xlane16(psum);
      psum += swap_halves(psum);
      l_run += psum;
      // B operands of P V, high part and residual (p = hi + lo to 2^-17):
      // k = 8g + e  <->  token (e < 4 ? 4g + e : 16 + 4g + e - 4)
      pb_s[sb][0][wid][lane] = __builtin_bit_cast(bf16x8, make_uint4(ph[0], ph[1], ph[2], ph[3]));
      pb_s[sb][1][wid][lane] = __builtin_bit_cast(bf16x8, make_uint4(pl[0], pl[1], pl[2], pl[3]));
    };
    prologue();
    if (ntiles > 0) {
      scores(0, 0, 0);
      __syncthreads();
      for (int t = 0; t < ntiles; ++t) {
        commit(pre, (t + 2) % 3);
        gather(pre, t + 3);
        if (t + 1 < ntiles) scores(t + 1, (t + 1) % 3, (t + 1) & 1);
        __syncthreads();
      }
    }
    if (g == 0) {
      ml_s[16 * wid + n][0] = m_run;
      ml_s[16 * wid + n][1] = l_run;
    }
    __syncthreads();
    const int64_t oh = (int64_t)b * A.n_q_heads + head;
    if (p.splits == 1) {
      if (g == 0 && p.lse)
        p.lse[oh] = l_run > 0.f ? (m_run + __log2f(l_run)) * kLn2 : -__builtin_huge_valf();
    } else if (g == 0) {
      float* pr = p.part + (((int64_t)b * ngrp + grp) * p.splits + split) * kMlaRec;
      pr[kMlaHeadsWG * 512 + 2 * (16 * wid + n)] = m_run;
      pr[kMlaHeadsWG * 512 + 2 * (16 * wid + n) + 1] = l_run;
    }
  } else {
    // O^T accumulators: o[hb][mc] holds columns 128 cq + 16 mc + 4g + i of
    // head 16 hb + n of the group
    f32x4 o[4][8];
#pragma unroll
    for (int hb = 0; hb < 4; ++hb)
#pragma unroll
      for (int mc = 0; mc < 8; ++mc) o[hb][mc] = f32x4{0.f, 0.f, 0.f, 0.f};
    // O^T[128 x 64] += V^T P^T for one tile; each V fragment feeds the four
    // head blocks
    auto pv = [&](int buf, int sb) __attribute__((always_inline)) {
      const uint16_t* kt = ks_s[buf];
      bf16x8 pbk[4], pbl[4];
#pragma unroll
      for (int hb = 0; hb < 4; ++hb) {
        const float alpha = alpha_s[sb][hb][n];
        if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
          for (int mc = 0; mc < 8; ++mc) o[hb][mc] *= alpha;
        }
        pbk[hb] = pb_s[sb][0][hb][lane];
        pbl[hb] = pb_s[sb][1][hb][lane];
      }
      // A operand, m-tile mc: lane (g, n) needs column 128 cq + 16 mc + n of
      // the eight tokens of its k range; lane n of each group addresses
      // token row n / 4 of the four and columns 4 (n % 4) .. +3
      const uint16_t* vb = kt + (4 * g + (n >> 2)) * kMlaRow + 128 * cq + 4 * (n & 3);
      bf16x8 vas[8];
#pragma unroll
      for (int mc = 0; mc < 8; ++mc) {
        const s16x4 r0 = lds_read_tr16(vb + 16 * mc);
        const s16x4 r1 = lds_read_tr16(vb + 16 * kMlaRow + 16 * mc);
        vas[mc] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7));
      }
#pragma unroll
      for (int mc = 0; mc < 8; ++mc) {
#pragma unroll
        for (int hb = 0; hb < 4; ++hb)
          o[hb][mc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vas[mc], pbk[hb], o[hb][mc], 0, 0, 0);
#pragma unroll
        for (int hb = 0; hb < 4; ++hb)
          o[hb][mc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vas[mc], pbl[hb], o[hb][mc], 0, 0, 0);
      }
    };
    prologue();
    if (ntiles > 0) {
      __syncthreads();
      for (int t = 0; t < ntiles; ++t) {
        // the P V MFMAs first: the score waves commit and gather while
        // these issue, and the P V waves commit and gather while the score
        // MFMAs issue (lightning_128k 6178 -> 6200-6211 steps/s, hot_16k
        // without misses 2706 -> 2748 against committing first)
        pv(t % 3, t & 1);
        commit(pre, (t + 2) % 3);
        gather(pre, t + 3);
        __syncthreads();
      }
    }
    __syncthreads();  // (m, l) of every head in LDS
    // epilogue: o[hb][mc] = O^T[col 128 cq + 16 mc + 4g + i][head 16 hb + n]
    if (p.splits == 1) {
#pragma unroll
      for (int hb = 0; hb < 4; ++hb) {
        const float l = ml_s[16 * hb + n][1];
        const float inv = l > 0.f ? 1.f / l : 0.f;
        const int64_t oh = (int64_t)b * A.n_q_heads + grp * kMlaHeadsWG + 16 * hb + n;
        float* op = p.out + oh * 512 + 128 * cq + 4 * g;
#pragma unroll
        for (int mc = 0; mc < 8; ++mc) *(f32x4*)(op + 16 * mc) = o[hb][mc] * inv;
      }
    } else {
      // record of (request, head group, split) in register order: slot
      // (cq * 4 + hb) * 8 + mc holds one f32x4 per lane, so that every store
      // writes 1 KiB contiguously; (m, l) per head follow
      float* pr = p.part + (((int64_t)b * ngrp + grp) * p.splits + split) * kMlaRec;
#pragma unroll
      for (int hb = 0; hb < 4; ++hb)
#pragma unroll
        for (int mc = 0; mc < 8; ++mc)
          *(f32x4*)(pr + ((((cq * 4 + hb) * 8) + mc) * 64 + lane) * 4) = o[hb][mc];
    }
  }
}

// ==================================================================== GQA
// d_qk = d_v = 128, up to 16 query heads per KV head, bf16.  One workgroup of
// kGqaWaves waves per (request, KV head, token split); the waves take the
// split's 32-token tiles in turn, each wave with its own online-softmax
// state, and merge through LDS once at the end, so the tile loop has no
// barrier.  Per tile a wave computes
//   S^T[32 tokens x 16 heads] = K Q^T  (A = K rows loaded from global memory
//       straight into the MFMA layout, B = q in registers; heads past the
//       group's G are zero),
//   the online softmax per head in the base-2 domain, with the lazy
//       rescale of the latent kernel (lane l holds head l % 16),
//   O^T[128 x 16] += V^T P^T  (A = V^T read from the wave's LDS copy of the
//       tile with ds_read_b64_tr_b16, B = the lane's own probabilities, in
//       the token order of the latent kernel).
// The K and V loads of a wave's next tile are in flight while it works on
// the current one.
constexpr int kGqaWaves = 4;
constexpr int kGqaRowV = 128 + 8;  // LDS row stride of a V tile (elements)

struct GqaTile {
  u32x4 k[2][4];  // K[token 16 mt + n][32 s + 8 g ..], lane (g, n)
  u32x4 v[8];     // V row (lane / 16) + 4 u, 16-byte chunk lane % 16
};

// (At most 256 VGPRs, so that two workgroups share a compute unit: at 260
// the kernel ran one workgroup per unit.)
// NT: the K/V rows are loaded non-temporally (chosen by the launch when the
// step gathers more than the last-level cache could keep for the next step).
template <bool NT>
__global__ __launch_bounds__(64 * kGqaWaves, 2) void attn_gqa_kernel(AttnPlan p) {
  __shared__ __attribute__((aligned(16))) uint16_t vs_s[kGqaWaves][kTT * kGqaRowV];
  __shared__ uint64_t rowp_s[kMaxSplitTok];
  __shared__ uint32_t vmask_s[kMaxSplitTok / kTT];
  __shared__ float ml_s[kGqaWaves][16][2];

  const sparse_attn_args& A = p.a;
  const int ngrp = A.n_kv_heads;
  const int unit = (int)(blockIdx.x % 8) + 8 * (int)(blockIdx.x / (8 * ngrp));
  const int kvh = (int)(blockIdx.x / 8) % ngrp;
  if (unit >= p.splits * A.batch) return;
  const int split = unit % p.splits;
  const int b = unit / p.splits;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int g = lane >> 4;
  const int n = lane & 15;
  const int G = A.n_q_heads / A.n_kv_heads;
  const int head0 = kvh * G;
  const int selrow_i = p.sel_heads == 1 ? 0 : kvh;
  const int32_t* selrow = p.sel + ((int64_t)b * p.sel_heads + selrow_i) * p.k;
  const int valid = valid_tokens(A, b);
  const int tps = (p.k_tokens + p.splits - 1) / p.splits;
  const int j0 = split * tps;
  const int j1 = min(j0 + tps, p.k_tokens);
  const int cnt = max(0, j1 - j0);
  const int ntiles = (cnt + kTT - 1) / kTT;
  RowAddr ra{A};
  const int64_t vdelta = (const char*)A.v_cache - (const char*)A.k_cache;

  // q of head n as the B operand: B[k = 32 s + 8 g + e][n]; zero past G
  bf16x8 qb[4];
  {
    const bool real = n < G;
    const uint16_t* qp = (const uint16_t*)A.q + (int64_t)b * A.q_stride_b +
                         (int64_t)(head0 + (real ? n : 0)) * A.q_stride_h + 8 * g;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const bf16x8 x = *(const bf16x8*)(qp + 32 * s);
      qb[s] = real ? x : bf16x8{};
    }
  }

  // row table (K rows; masked positions point at the library's zero row,
  // for K and V alike) and the valid-token bits of every tile
  const uint64_t dummy = (uint64_t)zero_row();
  for (int base = 0; base < ntiles * kTT; base += 64 * kGqaWaves) {
    const int i = base + tid;
    int t = -1;
    if (i < cnt) t = sel_token(selrow, j0 + i, p.sel_unit, valid);
    if (i < ntiles * kTT)
      rowp_s[i] = t >= 0 ? (uint64_t)ra.k_row(b, kvh, t, 0, nullptr, 2) : dummy;
    const uint64_t bal = __builtin_amdgcn_ballot_w64(t >= 0);
    const int tile = (base >> 5) + 2 * wid;  // lanes 0..31: tile, 32..63: tile + 1
    if (lane == 0 && tile < ntiles) vmask_s[tile] = (uint32_t)bal;
    if (lane == 0 && tile + 1 < ntiles) vmask_s[tile + 1] = (uint32_t)(bal >> 32);
  }
  __syncthreads();

  auto load = [&](GqaTile& T, int tile) __attribute__((always_inline)) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const char* kr = (const char*)rowp_s[tile * kTT + 16 * mt + n] + 16 * g;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        gptr<const u32x4> ka = (gptr<const u32x4>)(kr + 64 * s);
        T.k[mt][s] = NT ? __builtin_nontemporal_load(ka) : *ka;
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint64_t kp = rowp_s[tile * kTT + g + 4 * u];
      const char* vp = kp == dummy ? (const char*)kp : (const char*)kp + vdelta;
      gptr<const u32x4> va = (gptr<const u32x4>)(vp + 16 * n);
      T.v[u] = NT ? __builtin_nontemporal_load(va) : *va;
    }
  };

  const float qk_scale = A.sm_scale * kLog2e;
  float m_run = -__builtin_huge_valf();  // base-2 reference max of head n
  float l_run = 0.f;
  f32x4 o[8];  // O^T: o[mc][i] = column 16 mc + 4 g + i of head n
#pragma unroll
  for (int mc = 0; mc < 8; ++mc) o[mc] = f32x4{0.f, 0.f, 0.f, 0.f};
  uint16_t* vs = vs_s[wid];

  auto process = [&](const GqaTile& T, int tile) __attribute__((always_inline)) {
    f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, T.k[0][s]), qb[s], a0, 0, 0, 0);
      a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, T.k[1][s]), qb[s], a1, 0, 0, 0);
    }
    // the tile's V rows into this wave's LDS copy (read back transposed below)
#pragma unroll
    for (int u = 0; u < 8; ++u) *(u32x4*)(vs + (g + 4 * u) * kGqaRowV + 8 * n) = T.v[u];
    float sv[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sv[i] = a0[i] * qk_scale;
      sv[4 + i] = a1[i] * qk_scale;
    }
    const uint32_t vm = __builtin_amdgcn_readfirstlane(vmask_s[tile]);
    if (vm != 0xFFFFFFFFu) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (!((vm >> (16 * (e >> 2) + 4 * g + (e & 3))) & 1u)) sv[e] = -__builtin_huge_valf();
    }
    float tmax = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])),
                       fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
    tmax = fmaxf(tmax, xlane16(tmax));
    tmax = fmaxf(tmax, swap_halves(tmax));
    constexpr float kSlack = 8.0f;
    if (__builtin_amdgcn_ballot_w64(tmax > m_run + kSlack)) {
      const float m_new = fmaxf(m_run, tmax);
      const float alpha =
          (m_run == -__builtin_huge_valf()) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
      for (int mc = 0; mc < 8; ++mc) o[mc] *= alpha;
      l_run *= alpha;
      m_run = m_new;
    }
    const bool none = (m_run == -__builtin_huge_valf());
    float psum = 0.f;
    uint32_t ph[4], pl[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float p0 = none ? 0.f : __builtin_amdgcn_exp2f(sv[2 * e] - m_run);
      const float p1 = none ? 0.f : __builtin_amdgcn_exp2f(sv[2 * e + 1] - m_run);
      psum += p0 + p1;
      const bf16x2 hi = bf16x2{(__bf16)p0, (__bf16)p1};
      const bf16x2 lo = bf16x2{(__bf16)(p0 - (float)hi[0]), (__bf16)(p1 - (float)hi[1])};
      ph[e] = __builtin_bit_cast(uint32_t, hi);
      pl[e] = __builtin_bit_cast(uint32_t, lo);
    }
    psum += xlane16(psum);
    psum += swap_halves(psum);
    l_run += psum;
    // B operands of P V, high part and residual (p = hi + lo to 2^-17):
    // k = 8g + e  <->  token (e < 4 ? 4g + e : 16 + 4g + e - 4)
    const bf16x8 pb = __builtin_bit_cast(bf16x8, make_uint4(ph[0], ph[1], ph[2], ph[3]));
    const bf16x8 pbl = __builtin_bit_cast(bf16x8, make_uint4(pl[0], pl[1], pl[2], pl[3]));
    // A operand, m-tile mc: lane (g, n) needs column 16 mc + n of those
    // eight tokens; lane n of each group addresses token row n / 4 of the
    // four and columns 4 (n % 4) .. +3
    const uint16_t* vb = vs + (4 * g + (n >> 2)) * kGqaRowV + 4 * (n & 3);
#pragma unroll
    for (int mc = 0; mc < 8; ++mc) {
      const s16x4 r0 = lds_read_tr16(vb + 16 * mc);
      const s16x4 r1 = lds_read_tr16(vb + 16 * kGqaRowV + 16 * mc);
      const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7));
      o[mc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, o[mc], 0, 0, 0);
      o[mc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pbl, o[mc], 0, 0, 0);
    }
  };

  // this wave's tiles: wid, wid + kGqaWaves, ...; the next one in flight
  {
    GqaTile ta, tb;
    int t = wid;
    if (t < ntiles) load(ta, t);
    while (t < ntiles) {
      if (t + kGqaWaves < ntiles) load(tb, t + kGqaWaves);
      process(ta, t);
      t += kGqaWaves;
      if (t >= ntiles) break;
      if (t + kGqaWaves < ntiles) load(ta, t + kGqaWaves);
      process(tb, t);
      t += kGqaWaves;
    }
  }

  // ---- merge the waves: M = max m_w, f_w = 2^(m_w - M), L = sum l_w f_w,
  // O = sum f_w O_w (through LDS, reusing the V copies)
  if (g == 0) {
    ml_s[wid][n][0] = m_run;
    ml_s[wid][n][1] = l_run;
  }
  __syncthreads();
  float M = -__builtin_huge_valf();
#pragma unroll
  for (int w = 0; w < kGqaWaves; ++w)
    if (ml_s[w][n][1] > 0.f) M = fmaxf(M, ml_s[w][n][0]);
  float L = 0.f, f_own = 0.f;
#pragma unroll
  for (int w = 0; w < kGqaWaves; ++w) {
    const float lw = ml_s[w][n][1];
    const float fw = lw > 0.f ? __builtin_amdgcn_exp2f(ml_s[w][n][0] - M) : 0.f;
    L += lw * fw;
    if (w == wid) f_own = fw;
  }
  f32x4* os = (f32x4*)vs;  // 8 KiB of this wave's region: slot mc * 64 + lane
#pragma unroll
  for (int mc = 0; mc < 8; ++mc) os[mc * 64 + lane] = o[mc] * f_own;
  __syncthreads();
  // thread (wave wid, lane) sums m-tiles 2 wid and 2 wid + 1 of that lane
  const int64_t oh = (int64_t)b * A.n_q_heads + head0 + n;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int mc = 2 * wid + h;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kGqaWaves; ++w) acc += ((const f32x4*)vs_s[w])[mc * 64 + lane];
    if (n < G) {
      const int col = 16 * mc + 4 * g;
      if (p.splits == 1) {
        const float inv = L > 0.f ? 1.f / L : 0.f;
        *(f32x4*)(p.out + oh * 128 + col) = acc * inv;
      } else {
        *(f32x4*)(p.part + (oh * p.splits + split) * (128 + 4) + col) = acc;
      }
    }
  }
  if (wid == 0 && g == 0 && n < G) {
    const float m_nat = M * kLn2;  // natural-log domain of the combine
    if (p.splits == 1) {
      if (p.lse) p.lse[oh] = L > 0.f ? m_nat + __logf(L) : -__builtin_huge_valf();
    } else {
      float* pp = p.part + (oh * p.splits + split) * (128 + 4);
      pp[128] = m_nat;
      pp[129] = L;
    }
  }
}

bool attn_selects(const sparse_attn_args& a) {
  return a.dtype == SPARSE_BF16 && mla_shape(a) && a.hot_slot == nullptr;
}

hipError_t launch_attn_bf16(const AttnPlan& p, hipStream_t s) {
  const sparse_attn_args& a = p.a;
  // 8 * groups * ceil(units / 8) workgroup ids (the kernel decodes them)
  const int64_t units = (int64_t)p.splits * a.batch;
  const int64_t rounds = (units + 7) / 8;
  if (mla_shape(a)) {
    const int groups = a.n_q_heads / kMlaHeadsWG;
    dim3 grid((unsigned)(8 * groups * rounds), 1, 1);
    if (p.fsel) attn_mla_kernel<true><<<grid, kMlaThreads, 0, s>>>(p);
    else attn_mla_kernel<false><<<grid, kMlaThreads, 0, s>>>(p);
  } else if (a.d_qk == 128 && a.d_v == 128 && a.v_cache != nullptr) {
    const int groups = a.n_kv_heads;
    dim3 grid((unsigned)(8 * groups * rounds), 1, 1);
    // K and V rows gathered by this launch; from a quarter of the 256 MB
    // last-level cache up they would not stay there for the next step (the
    // other layers and the index stream pass through it too), so they stream
    // (block_sparse_80k, 128 MiB per layer: 7708 -> 7846 steps/s); smaller
    // gathers stay cacheable for the overlapping selection of the next step
    // (fathom_1m, 8 MiB: non-temporal loads measured 13890 -> 13583)
    const int64_t gathered = (int64_t)a.batch * p.k_tokens * a.n_kv_heads * (a.d_qk + a.d_v) * 2;
    if (gathered >= ((int64_t)64 << 20))
      attn_gqa_kernel<true><<<grid, 64 * kGqaWaves, 0, s>>>(p);
    else
      attn_gqa_kernel<false><<<grid, 64 * kGqaWaves, 0, s>>>(p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ================================================================ combine
// Merge split partials of one (request, head): M = max m_s,
// L = sum l_s exp(m_s - M), out = sum o_s exp(m_s - M) / L, lse = M + log L.
constexpr int kCombThreads = 256;

// One workgroup per (request, head); thread (q, sl) merges column quad q
// (d_v / 4 quads, d_v <= 512) over splits sl, sl + SL, ... (SL = threads per
// quad), and the SL partial results are summed through LDS.
__global__ __launch_bounds__(kCombThreads) void attn_combine_kernel(AttnPlan p) {
  __shared__ float m_s[kCombThreads];
  __shared__ f32x4 acc_s[kCombThreads];
  __shared__ float l_s[kCombThreads];
  const sparse_attn_args& A = p.a;
  const int dv = A.d_v;
  const int S = p.splits;
  const int64_t oh = blockIdx.x;
  const float* pp = p.part + oh * S * (dv + 4);
  const int tid = threadIdx.x;
  const int Q = dv / 4;
  const int SL = kCombThreads / Q;
  const int q = tid % Q, sl = tid / Q;
  // M = max over splits of the split maxima
  float mloc = -__builtin_huge_valf();
  for (int sp = tid; sp < S; sp += kCombThreads) mloc = fmaxf(mloc, pp[(int64_t)sp * (dv + 4) + dv]);
  m_s[tid] = mloc;
  __syncthreads();
  for (int off = kCombThreads / 2; off >= 1; off >>= 1) {
    if (tid < off) m_s[tid] = fmaxf(m_s[tid], m_s[tid + off]);
    __syncthreads();
  }
  const float M = m_s[0];
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
  if (sl < SL) {
#pragma unroll 4
    for (int sp = sl; sp < S; sp += SL) {
      const float* ps = pp + (int64_t)sp * (dv + 4);
      const float l = ps[dv + 1];
      const float f = l > 0.f ? __expf(ps[dv] - M) : 0.f;
      const f32x4 v = *(const f32x4*)(ps + 4 * q);
      acc += v * f;
      L += l * f;
    }
  }
  acc_s[tid] = acc;
  l_s[tid] = L;
  __syncthreads();
  if (tid < Q) {
    f32x4 a = acc_s[tid];
    float Lt = l_s[tid];
    for (int k = 1; k < SL; ++k) {
      a += acc_s[tid + k * Q];
      Lt += l_s[tid + k * Q];
    }
    const float inv = Lt > 0.f ? 1.f / Lt : 0.f;
    *(f32x4*)(p.out + oh * dv + 4 * tid) = a * inv;
    if (tid == 0 && p.lse) p.lse[oh] = Lt > 0.f ? M + __logf(Lt) : -__builtin_huge_valf();
  }
}

// Latent records (register order of the attention kernel, base-2 m): one
// workgroup per (request, head group, column quarter cq); thread (q, lane)
// merges slots 4q .. 4q + 3 of quarter cq: head block q / 2, column m-tiles
// 4 (q % 2) .. +3.
__global__ __launch_bounds__(512) void attn_combine_mla_kernel(AttnPlan p) {
  const sparse_attn_args& A = p.a;
  const int ngrp = A.n_q_heads / kMlaHeadsWG;
  const int cq = (int)(blockIdx.x % 4);
  const int64_t bg = blockIdx.x / 4;  // request * ngrp + group
  const int b = (int)(bg / ngrp), grp = (int)(bg % ngrp);
  const int tid = threadIdx.x, lane = tid & 63, q = tid >> 6;
  const int g = lane >> 4, n = lane & 15;
  const int hb = q >> 1, mc0 = 4 * (q & 1);
  const int hl = 16 * hb + n;
  const int S = p.splits;
  const float* base = p.part + bg * S * kMlaRec;
  const int slot = (cq * 4 + hb) * 8 + mc0;
  // splits in batches of four, every load of a batch issued before any is
  // used; the batches merge online (running max M, sum L, output acc)
  float M = -__builtin_huge_valf(), L = 0.f;
  f32x4 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < S; s0 += 4) {
    float mv[4], lv[4];
    f32x4 pv[4][4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float* ps = base + (int64_t)min(s0 + u, S - 1) * kMlaRec;
      mv[u] = ps[kMlaHeadsWG * 512 + 2 * hl];
      lv[u] = s0 + u < S ? ps[kMlaHeadsWG * 512 + 2 * hl + 1] : 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j)  // each record is read once: non-temporal
        pv[u][j] = __builtin_nontemporal_load((const f32x4*)(ps + ((slot + j) * 64 + lane) * 4));
    }
    float mb = M;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (lv[u] > 0.f) mb = fmaxf(mb, mv[u]);
    const float r = M == -__builtin_huge_valf() ? 0.f : __builtin_amdgcn_exp2f(M - mb);
    L *= r;
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] *= r;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float f = lv[u] > 0.f ? __builtin_amdgcn_exp2f(mv[u] - mb) : 0.f;
      L += lv[u] * f;
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] += pv[u][j] * f;
    }
    M = mb;
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  const int64_t oh = (int64_t)b * A.n_q_heads + grp * kMlaHeadsWG + hl;
  float* op = p.out + oh * 512 + 128 * cq + 16 * mc0 + 4 * g;
#pragma unroll
  for (int j = 0; j < 4; ++j) *(f32x4*)(op + 16 * j) = acc[j] * inv;
  if ((q & 1) == 0 && cq == 0 && g == 0 && p.lse)
    p.lse[oh] = L > 0.f ? (M + __log2f(L)) * kLn2 : -__builtin_huge_valf();
}

hipError_t launch_attn_combine(const AttnPlan& p, hipStream_t s) {
  const sparse_attn_args& a = p.a;
  if (a.dtype == SPARSE_BF16 && mla_shape(a)) {
    const int64_t wgs = (int64_t)a.batch * (a.n_q_heads / kMlaHeadsWG) * 4;
    attn_combine_mla_kernel<<<(unsigned)wgs, 512, 0, s>>>(p);
  } else {
    attn_combine_kernel<<<(unsigned)((int64_t)a.batch * a.n_q_heads), kCombThreads, 0, s>>>(p);
  }
  return hipGetLastError();
}

// ============================================================ miss fetch
// "XM-Sparse" blog, Figure 1 caption and KV-lifecycle list: selected
// entries that are not in the HBM hot buffer are fetched from host memory.
// One workgroup per 256 selection positions of a request: each thread checks
// one position once (token, then hot slot), the missed rows are compacted
// into an LDS list (wave ballots), and the workgroup then copies those rows
// 16 bytes per thread and item, eight items in flight, through the
// device-visible alias of the pinned host buffer (PCIe) into the workspace
// staging slots of their selection positions.
constexpr int kMfRows = 256;
constexpr int kMfUnroll = 8;

__global__ __launch_bounds__(kMfRows) void miss_fetch_kernel(AttnPlan p) {
  __shared__ int32_t mj_s[kMfRows];
  __shared__ const char* msrc_s[kMfRows];
  __shared__ int nm_s;
  const sparse_attn_args& A = p.a;
  const int b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int cpr = A.d_qk * 2 / 16;
  if (tid == 0) nm_s = 0;
  __syncthreads();
  const int j = blockIdx.x * kMfRows + tid;
  bool miss = false;
  const char* src = nullptr;
  if (j < p.k_tokens) {
    const int32_t* selrow = p.sel + (int64_t)b * p.sel_heads * p.k;
    const int t = sel_token(selrow, j, p.sel_unit, valid_tokens(A, b));
    if (t >= 0 && A.hot_slot[(int64_t)b * A.hs_stride_b + t] < 0) {
      miss = true;
      src = (const char*)A.host_kv + ((int64_t)b * A.host_stride_b + (int64_t)t * A.host_stride_t) * 2;
    }
  }
  const uint64_t bal = __builtin_amdgcn_ballot_w64(miss);
  int base = 0;
  if (lane == 0 && bal) base = atomicAdd(&nm_s, __builtin_popcountll(bal));
  base = __shfl(base, 0, 64);
  if (miss) {
    const int slot = base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                           __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
    mj_s[slot] = j;
    msrc_s[slot] = src;
  }
  __syncthreads();
  const int items = nm_s * cpr;
  char* stage = (char*)(p.staging + (int64_t)b * p.k_tokens * A.d_qk);
  for (int i0 = tid; i0 < items; i0 += kMfRows * kMfUnroll) {
    uint4 v[kMfUnroll];
#pragma unroll
    for (int u = 0; u < kMfUnroll; ++u) {
      const int i = i0 + u * kMfRows;
      if (i < items) v[u] = *(const uint4*)(msrc_s[i / cpr] + 16 * (i % cpr));
    }
#pragma unroll
    for (int u = 0; u < kMfUnroll; ++u) {
      const int i = i0 + u * kMfRows;
      if (i < items)
        *(uint4*)(stage + (int64_t)mj_s[i / cpr] * A.d_qk * 2 + 16 * (i % cpr)) = v[u];
    }
  }
}

hipError_t launch_miss_fetch(const AttnPlan& p, hipStream_t s) {
  dim3 grid((unsigned)((p.k_tokens + kMfRows - 1) / kMfRows), p.a.batch);
  miss_fetch_kernel<<<grid, kMfRows, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace sd
