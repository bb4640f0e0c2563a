// Decode-side append: the new token of each request joins the KV history,
// the K-index and the bit planes that the next step reads.
//
// "XM-Sparse" blog, KV-lifecycle list: the KV a decode step generates is
// appended to the history.  "MiniMax-M3: share the sparse index top-k ..."
// description: the decode path's sparse-KV store writes the step's entries
// once (idempotently).  "Fathom" abstract: the 4-bit K is stored
// channel-major as bit planes, so a new key is one bit in each of its
// channel's four planes.
//
// One workgroup per (request, part): part 0 writes the KV rows, the others
// the index entry (one per KV head for bit planes).  Every word is written by
// exactly one thread.
#include <string.h>

#include "common.hpp"

namespace sd {

constexpr int kAppThreads = 256;

// OCP E4M3FN byte nearest to x (|x| <= 448), ties to the even code.
__device__ __forceinline__ uint32_t e4m3fn_rne(float x) {
  const uint32_t sign = __float_as_uint(x) >> 31;
  const float a = fabsf(x);
  uint32_t code;
  if (a < 0.015625f) {
    // subnormal range: steps of 2^-9; 8 steps is the first normal (0x08)
    code = (uint32_t)__builtin_rintf(a * 512.0f);
  } else {
    int e = (int)((__float_as_uint(a) >> 23) & 0xFFu) - 127;  // floor(log2 a)
    uint32_t m = (uint32_t)__builtin_rintf(ldexpf(a, 3 - e));  // 8 .. 16
    if (m == 16u) { m = 8u; e += 1; }
    code = ((uint32_t)(e + 7) << 3) | (m - 8u);
  }
  if (code > 0x7Eu) code = 0x7Eu;
  return code | (sign << 7);
}

__device__ __forceinline__ uint16_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

struct AppendPlan {
  sparse_index_args ia;
  sparse_attn_args aa;
  int has_ia, has_aa;
  const int32_t* pos;
  const float* key_new;  // index key, fp32
  const void* k_new;     // attention K (or latent) rows, aa.dtype
  const void* v_new;     // attention V rows (NULL when latent)
};

__device__ void append_kv(const AppendPlan& p, int b) {
  const sparse_attn_args& A = p.aa;
  const int t = p.pos[b];
  if (t < 0 || t >= A.n) return;
  const int es = A.dtype == SPARSE_F32 ? 4 : 2;
  const int kchunks = A.d_qk * es / 16;
  const int vchunks = A.v_cache ? A.d_v * es / 16 : 0;
  const int per_head = kchunks + vchunks;
  for (int i = threadIdx.x; i < A.n_kv_heads * per_head; i += kAppThreads) {
    const int h = i / per_head;
    const int c = i % per_head;
    const bool isv = c >= kchunks;
    const int cc = isv ? c - kchunks : c;
    const char* src;
    char* dst;
    if (!isv) {
      src = (const char*)p.k_new + (((int64_t)b * A.n_kv_heads + h) * A.d_qk) * es;
      if (A.hot_slot) {
        dst = (char*)A.host_kv + ((int64_t)b * A.host_stride_b + (int64_t)t * A.host_stride_t) * es;
      } else {
        int64_t off;
        if (A.page_table) {
          const int pg = A.page_table[(int64_t)b * A.pt_stride_b + t / A.page_size];
          off = ((int64_t)pg * A.page_size + t % A.page_size) * A.kv_stride_t;
        } else {
          off = (int64_t)b * A.kv_stride_b + (int64_t)t * A.kv_stride_t;
        }
        dst = (char*)A.k_cache + (off + (int64_t)h * A.kv_stride_h) * es;
      }
    } else {
      src = (const char*)p.v_new + (((int64_t)b * A.n_kv_heads + h) * A.d_v) * es;
      int64_t off;
      if (A.page_table) {
        const int pg = A.page_table[(int64_t)b * A.pt_stride_b + t / A.page_size];
        off = ((int64_t)pg * A.page_size + t % A.page_size) * A.kv_stride_t;
      } else {
        off = (int64_t)b * A.kv_stride_b + (int64_t)t * A.kv_stride_t;
      }
      dst = (char*)A.v_cache + (off + (int64_t)h * A.kv_stride_h) * es;
    }
    *(u32x4*)(dst + 16 * cc) = *(const u32x4*)(src + 16 * cc);
  }
}

// part: 0 for the one-wave kinds; for bit planes the KV head this
// workgroup writes (one workgroup per KV head).
__device__ void append_index(const AppendPlan& p, int b, int part) {
  const sparse_index_args& I = p.ia;
  const int t = p.pos[b];
  if (t < 0 || t >= I.n) return;
  const int D = I.head_dim;  // 128
  const int tid = threadIdx.x;
  if (I.kind == SPARSE_SCORE_DOT) {
    const float* k = p.key_new + (int64_t)b * D;
    for (int d = tid; d < D; d += kAppThreads) {
      const int64_t o = (int64_t)b * I.k_stride_b + (int64_t)t * I.k_stride_t + d;
      if (I.k_dtype == SPARSE_F32) ((float*)I.keys)[o] = k[d];
      else ((uint16_t*)I.keys)[o] = bf16_rne(k[d]);
    }
  } else if (I.kind == SPARSE_SCORE_LIGHTNING) {
    if (tid >= 64) return;  // one wave; lane l holds dims 2l, 2l + 1
    const float* k = p.key_new + (int64_t)b * D;
    const float k0 = k[2 * tid], k1 = k[2 * tid + 1];
    float amax = fmaxf(fabsf(k0), fabsf(k1));
    for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
    const float sc = amax > 0.f ? __fdiv_rn(amax, 448.0f) : 1.0f;
    const float x0 = fminf(fmaxf(__fdiv_rn(k0, sc), -448.0f), 448.0f);
    const float x1 = fminf(fmaxf(__fdiv_rn(k1, sc), -448.0f), 448.0f);
    uint8_t* row = (uint8_t*)I.keys + (int64_t)b * I.k_stride_b + (int64_t)t * I.k_stride_t;
    *(uint16_t*)(row + 2 * tid) = (uint16_t)(e4m3fn_rne(x0) | (e4m3fn_rne(x1) << 8));
    if (tid == 0) ((float*)I.k_scale)[(int64_t)b * I.ks_stride_b + t] = sc;
  } else {
    // bit planes: thread per channel of this workgroup's KV head; it owns
    // the channel's four words
    const int Hkv = I.n_kv_heads;
    const int nw = (I.n + 31) / 32;
    const int w = t >> 5;
    const uint32_t bit = 1u << (t & 31);
    for (int i = tid; i < D; i += kAppThreads) {
      const int64_t hc = ((int64_t)b * Hkv + part) * D + i;  // [b][h][c]
      const double kv = (double)p.key_new[hc];
      const double z = (double)I.chan_zero[hc];
      const double cell = (double)I.chan_scale[hc];
      int code = 0;
      if (cell > 0.0) {
        const double f = floor(__ddiv_rn(__dsub_rn(kv, z), cell));
        code = f < 0.0 ? 0 : (f > 15.0 ? 15 : (int)f);
      }
      uint32_t* pl = (uint32_t*)I.planes + hc * 4 * (int64_t)nw + w;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t* wp = pl + (int64_t)j * nw;
        const uint32_t v = *wp;
        *wp = ((code >> (3 - j)) & 1) ? (v | bit) : (v & ~bit);
      }
    }
  }
}

__global__ __launch_bounds__(kAppThreads) void append_kernel(AppendPlan p) {
  const int b = blockIdx.x;
  if (blockIdx.y == 0) {
    if (p.has_aa) append_kv(p, b);
  } else {
    if (p.has_ia) append_index(p, b, blockIdx.y - 1);
  }
}

hipError_t launch_append(const sparse_index_args* ia, const sparse_attn_args* aa,
                         const int32_t* pos, const float* key_new, const void* k_new,
                         const void* v_new, int batch, hipStream_t s) {
  AppendPlan p;
  memset(&p, 0, sizeof(p));
  if (ia) p.ia = *ia;
  if (aa) p.aa = *aa;
  p.has_ia = ia != nullptr;
  p.has_aa = aa != nullptr;
  p.pos = pos;
  p.key_new = key_new;
  p.k_new = k_new;
  p.v_new = v_new;
  const int parts = (ia && ia->kind == SPARSE_SCORE_BITPLANE) ? ia->n_kv_heads : 1;
  append_kernel<<<dim3(batch, 1 + parts), kAppThreads, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace sd
