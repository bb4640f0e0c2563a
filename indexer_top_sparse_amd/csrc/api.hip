// extern "C" entry points: argument validation, workspace layout, dispatch.
// No entry point allocates, frees or synchronises; all scratch lives in the
// caller's workspace (sparse_decode_step_noalloc: in a fixed device array)
// and all work goes on the caller's stream.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "common.hpp"

// Scratch of sparse_decode_step_noalloc: device memory of this code object,
// held by every GPU the library runs on until the process ends.  Its name
// is a host-side stand-in in host code: host code uses only the device
// address hipGetSymbolAddress returns for the current device.
static constexpr size_t kNoAllocScratchBytes = SPARSE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

namespace {

thread_local char g_err[512];

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

#define CHECK(cond, code, ...) \
  do {                         \
    if (!(cond)) return fail(code, __VA_ARGS__); \
  } while (0)

#define HIPCHECK(expr)                                                   \
  do {                                                                   \
    hipError_t e_ = (expr);                                              \
    if (e_ != hipSuccess)                                                \
      return fail(SPARSE_EHIP, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int64_t esize(int dt) { return dt == SPARSE_F32 ? 4 : (dt == SPARSE_BF16 ? 2 : 1); }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Device address of `scratch` on each device, looked up once per device
// with that device current.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// ------------------------------------------------------------------ layout
struct IndexLayout {
  int rows_per_b = 1;  // R
  int rows = 0;        // B * R
  int n_units = 0;
  int n_chunks = 0;
  int hist_parts = 0;   // histogram parts per row the score kernel writes
  size_t scores = 0, hist = 0, bstar = 0, cand_key = 0, cand_idx = 0, chunk_cnt = 0,
         cand_total = 0, end = 0;
};

IndexLayout index_layout(const sparse_index_args& a, bool with_scores) {
  IndexLayout L;
  L.rows_per_b = a.kind == SPARSE_SCORE_BITPLANE ? a.n_kv_heads : 1;
  L.rows = a.batch * L.rows_per_b;
  const int bs = a.kind == SPARSE_SCORE_DOT ? a.block_size : 1;
  L.n_units = (int)ceil_div(a.n, bs);
  L.n_chunks = (int)ceil_div(L.n_units, sd::kTopkChunk);
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += align256(bytes); return o; };
  const size_t cells = (size_t)L.rows * L.n_units;
  L.scores = with_scores ? take(cells * 4) : 0;
  // room for the score kernel's parts and for one part per chunk (the
  // standalone top-k)
  L.hist_parts = sd::score_hist_parts(a);
  const int parts = std::max(L.hist_parts, std::max(L.n_chunks, 1));
  L.hist = take((size_t)L.rows * parts * sd::kHistPartWords * 4);
  L.bstar = take((size_t)L.rows * 2 * 4);
  L.cand_key = take(cells * 4);
  L.cand_idx = take(cells * 4);
  L.chunk_cnt = take((size_t)L.rows * std::max(L.n_chunks, 1) * 4);
  L.cand_total = take((size_t)L.rows * 4);
  L.end = off;
  return L;
}

// Fixed split heuristic (no runtime tuning): enough workgroups to fill the
// 256 compute units (512 for the lighter 4-wave kernels), never fewer than
// min_tok tokens per split, and never more than 2048 tokens per split (the
// kernels resolve a split's rows into a 2048-entry LDS table).
int attn_splits(const sparse_attn_args& a, int k_tokens) {
  if (k_tokens <= 0) return 1;
  int groups, min_tok, target;
  if (a.dtype == SPARSE_F32) {
    // workgroups of up to 8 query heads sharing a KV head
    const int G = a.n_q_heads / std::max(a.n_kv_heads, 1);
    groups = a.n_kv_heads * ((G + 7) / 8);
    min_tok = 16;
    target = 256;
  } else if (a.d_qk == 576) {
    // One 8-wave workgroup per compute unit (its LDS), 64 heads each, so the
    // workgroups run in rounds of one per CU.  A workgroup costs about six
    // 32-token tiles of fixed time (row table, pipeline fill, epilogue) plus
    // its tiles, and any split adds the combine (about four tiles): take the
    // split count with the least rounds x per-workgroup time.
    constexpr int kCUs = 256;  // MI355X
    const int64_t base = (int64_t)std::max(a.batch, 1) * std::max(a.n_q_heads / 64, 1);
    const int64_t tiles = ceil_div(k_tokens, 32);
    const int64_t s_min = std::max<int64_t>(1, ceil_div(k_tokens, 2048));
    const int64_t s_max = std::max<int64_t>(s_min, std::min<int64_t>(64, k_tokens / 256));
    int64_t best = s_min, best_cost = -1;
    for (int64_t sp = s_min; sp <= s_max; ++sp) {
      const int64_t rounds = ceil_div(base * sp, kCUs);
      const int64_t cost = rounds * (ceil_div(tiles, sp) + 6) + (sp > 1 ? 4 : 0);
      if (best_cost < 0 || cost < best_cost) {
        best = sp;
        best_cost = cost;
      }
    }
    return (int)best;
  } else {
    // 4-wave workgroups, one KV head each, two fit a compute unit.  About
    // 256 workgroups with at least 128 tokens (one tile per wave) each beat
    // filling all 512 slots: fewer splits mean less fixed time per token
    // and a smaller combine (block_sparse_80k 7610 -> 7720 steps/s, fathom_1m
    // 14170 -> 14280).
    groups = a.n_kv_heads;
    min_tok = 128;
    target = 256;
  }
  const int64_t base = (int64_t)std::max(a.batch, 1) * std::max(groups, 1);
  int64_t s = ceil_div(target, base);
  s = std::min<int64_t>(s, std::max<int64_t>(1, k_tokens / min_tok));
  s = std::max<int64_t>(s, ceil_div(k_tokens, 2048));
  return (int)std::max<int64_t>(s, 1);
}

struct AttnLayout {
  int k_tokens = 0, splits = 1;
  size_t part = 0, staging = 0, end = 0;
};

AttnLayout attn_layout(const sparse_attn_args& a, int k_tokens, size_t base) {
  AttnLayout L;
  L.k_tokens = k_tokens;
  L.splits = attn_splits(a, k_tokens);
  size_t off = base;
  auto take = [&](size_t bytes) { size_t o = off; off += align256(bytes); return o; };
  if (L.splits > 1)
    L.part = take((size_t)a.batch * a.n_q_heads * L.splits * (a.d_v + 4) * 4);
  if (a.hot_slot) L.staging = take((size_t)a.batch * k_tokens * a.d_qk * 2);
  L.end = off;
  return L;
}

// -------------------------------------------------------------- validation
int check_index(const sparse_index_args* a) {
  CHECK(a, SPARSE_EINVAL, "index args is NULL");
  CHECK(a->batch >= 0 && a->n >= 0, SPARSE_EINVAL, "negative batch or n");
  CHECK(a->kind >= 0 && a->kind <= 2, SPARSE_EINVAL, "unknown score kind %d", a->kind);
  CHECK(a->head_dim == 128, SPARSE_EUNSUPPORTED, "head_dim %d (only 128)", a->head_dim);
  CHECK(a->n <= (1 << 22) * 1, SPARSE_EUNSUPPORTED, "n %d above 4194304", a->n);
  if (a->batch == 0 || a->n == 0) return SPARSE_OK;
  CHECK(a->q && aligned16(a->q), SPARSE_EINVAL, "q NULL or not 16-byte aligned");
  CHECK(a->n_heads >= 1, SPARSE_EINVAL, "n_heads %d", a->n_heads);
  const int64_t qe = esize(a->q_dtype);
  CHECK((a->q_stride_h * qe) % 16 == 0 && (a->q_stride_b * qe) % 16 == 0,
        SPARSE_EINVAL, "q strides must be multiples of 16 bytes");
  CHECK(a->q_stride_h >= a->head_dim, SPARSE_EINVAL, "q_stride_h < head_dim");
  if (a->kind == SPARSE_SCORE_DOT) {
    CHECK(a->q_dtype == SPARSE_F32 || a->q_dtype == SPARSE_BF16, SPARSE_EUNSUPPORTED,
          "DOT q dtype");
    CHECK(a->k_dtype == a->q_dtype, SPARSE_EUNSUPPORTED, "DOT needs q and keys of one dtype");
    CHECK(a->block_size == 1 || a->block_size == 64, SPARSE_EUNSUPPORTED,
          "block_size %d (1 or 64)", a->block_size);
  } else {
    CHECK(a->block_size == 1, SPARSE_EUNSUPPORTED, "block_size must be 1 for this kind");
    CHECK(a->q_dtype == SPARSE_BF16, SPARSE_EUNSUPPORTED, "q must be bf16 for this kind");
  }
  if (a->kind != SPARSE_SCORE_BITPLANE) {
    CHECK(a->keys && aligned16(a->keys), SPARSE_EINVAL, "keys NULL or not 16-byte aligned");
    const int64_t ke = esize(a->k_dtype);
    CHECK((a->k_stride_t * ke) % 16 == 0 && (a->k_stride_b * ke) % 16 == 0,
          SPARSE_EINVAL, "key strides must be multiples of 16 bytes");
    CHECK(a->k_stride_t >= a->head_dim, SPARSE_EINVAL, "k_stride_t < head_dim");
  }
  if (a->kind == SPARSE_SCORE_LIGHTNING) {
    CHECK(a->k_dtype == SPARSE_E4M3FN, SPARSE_EUNSUPPORTED, "LIGHTNING keys must be e4m3fn");
    CHECK(a->n_heads == 32 || a->n_heads == 64, SPARSE_EUNSUPPORTED,
          "LIGHTNING n_heads %d (32 or 64)", a->n_heads);
    CHECK(a->head_w && a->k_scale, SPARSE_EINVAL, "head_w / k_scale NULL");
    // the scan addresses a request's keys with 32-bit byte offsets
    CHECK((int64_t)a->n * a->k_stride_t <= INT32_MAX, SPARSE_EUNSUPPORTED,
          "n * k_stride_t = %lld bytes of keys per request, above 2^31 - 1",
          (long long)a->n * a->k_stride_t);
  }
  CHECK(a->depth_in == nullptr || a->kind == SPARSE_SCORE_BITPLANE, SPARSE_EINVAL,
        "depth_in is for kind BITPLANE only");
  if (a->kind == SPARSE_SCORE_BITPLANE) {
    CHECK(a->n_kv_heads >= 1 && a->n_heads % a->n_kv_heads == 0, SPARSE_EINVAL,
          "n_heads %d not a multiple of n_kv_heads %d", a->n_heads, a->n_kv_heads);
    CHECK(a->planes && a->chan_zero && a->chan_scale && (a->chan_var || a->depth_in),
          SPARSE_EINVAL, "planes / chan_zero / chan_scale / chan_var NULL");
    CHECK(a->bit_budget >= 0 && a->bit_budget <= 4 * a->head_dim, SPARSE_EINVAL,
          "bit_budget %d outside 0..%d", a->bit_budget, 4 * a->head_dim);
  }
  return SPARSE_OK;
}

int check_attn(const sparse_attn_args* a, int sel_heads, int k, int sel_unit) {
  CHECK(a, SPARSE_EINVAL, "attn args is NULL");
  CHECK(a->batch >= 0 && a->n >= 0, SPARSE_EINVAL, "negative batch or n");
  CHECK(k >= 1, SPARSE_EINVAL, "k %d < 1", k);
  CHECK(sel_unit == 1 || sel_unit == 64, SPARSE_EUNSUPPORTED, "sel_unit %d", sel_unit);
  CHECK(a->n_q_heads >= 1 && a->n_kv_heads >= 1 && a->n_q_heads % a->n_kv_heads == 0,
        SPARSE_EINVAL, "heads %d / %d", a->n_q_heads, a->n_kv_heads);
  CHECK(sel_heads == 1 || sel_heads == a->n_kv_heads, SPARSE_EINVAL,
        "sel_heads %d must be 1 or n_kv_heads", sel_heads);
  const int G = a->n_q_heads / a->n_kv_heads;
  if (a->dtype == SPARSE_F32) {
    CHECK(a->d_qk == 128 && a->d_v == 128, SPARSE_EUNSUPPORTED, "f32 attention needs 128/128");
    CHECK(a->hot_slot == nullptr, SPARSE_EUNSUPPORTED, "hot buffer needs bf16 latent rows");
  } else if (a->dtype == SPARSE_BF16) {
    const bool mla = a->d_qk == 576 && a->d_v == 512 && a->v_cache == nullptr &&
                     a->n_kv_heads == 1 && a->n_q_heads % 64 == 0;
    const bool gqa = a->d_qk == 128 && a->d_v == 128 && a->v_cache != nullptr && G <= 16;
    CHECK(mla || gqa, SPARSE_EUNSUPPORTED,
          "bf16 attention shapes: latent 576/512 (1 KV head, Hq %% 64 == 0) or "
          "128/128 with <= 16 query heads per KV head");
  } else {
    return fail(SPARSE_EUNSUPPORTED, "attention dtype %d", a->dtype);
  }
  if (a->batch == 0) return SPARSE_OK;
  CHECK(a->q && aligned16(a->q), SPARSE_EINVAL, "q NULL or not 16-byte aligned");
  const int64_t e = esize(a->dtype);
  CHECK((a->q_stride_h * e) % 16 == 0 && (a->q_stride_b * e) % 16 == 0, SPARSE_EINVAL,
        "q strides must be multiples of 16 bytes");
  // an empty context: every selected position resolves to no token, so no
  // KV row is read and those pointers may be NULL
  if (a->n == 0) return SPARSE_OK;
  if (a->hot_slot) {
    CHECK(a->v_cache == nullptr && a->page_table == nullptr, SPARSE_EUNSUPPORTED,
          "hot buffer: latent contiguous rows only");
    CHECK(sel_heads == 1, SPARSE_EUNSUPPORTED, "hot buffer: one selection per request");
    CHECK(a->hot_kv && aligned16(a->hot_kv) && a->host_kv && aligned16(a->host_kv),
          SPARSE_EINVAL, "hot_kv / host_kv NULL or misaligned");
    CHECK((a->hot_stride_s * 2) % 16 == 0 && (a->hot_stride_b * 2) % 16 == 0 &&
              (a->host_stride_t * 2) % 16 == 0 && (a->host_stride_b * 2) % 16 == 0,
          SPARSE_EINVAL, "hot/host strides must be multiples of 16 bytes");
  } else {
    CHECK(a->k_cache && aligned16(a->k_cache), SPARSE_EINVAL,
          "k_cache NULL or not 16-byte aligned");
    CHECK(a->v_cache == nullptr || aligned16(a->v_cache), SPARSE_EINVAL,
          "v_cache not 16-byte aligned");
    CHECK((a->kv_stride_t * e) % 16 == 0 && (a->kv_stride_h * e) % 16 == 0 &&
              (a->kv_stride_b * e) % 16 == 0,
          SPARSE_EINVAL, "KV strides must be multiples of 16 bytes");
    if (a->page_table) CHECK(a->page_size >= 1, SPARSE_EINVAL, "page_size < 1");
  }
  return SPARSE_OK;
}

sd::TopkPlan make_topk_plan(const IndexLayout& L, char* ws, const float* scores,
                            int64_t row_stride, const int32_t* valid, int rows_per_valid,
                            int unit_div, int k, int32_t* idx_out, float* val_out,
                            int hist_parts, int part_span) {
  sd::TopkPlan p;
  p.rows = L.rows;
  p.n_units = L.n_units;
  p.k = k;
  p.n_chunks = L.n_chunks;
  p.rows_per_valid = rows_per_valid;
  p.row_stride = row_stride;
  p.scores = scores;
  p.valid = valid;
  p.unit_div = unit_div;
  p.hist = (uint32_t*)(ws + L.hist);
  p.parts = hist_parts;
  p.part_span = part_span;
  // one contiguous candidate list per row when the parts are few contiguous
  // spans that cover the row
  p.fused = part_span > 0 && hist_parts >= 1 && hist_parts <= sd::kFuseMaxParts &&
            (int64_t)hist_parts * part_span >= L.n_units;
  p.direct = L.n_units <= sd::kTopkDirectMax;
  p.bstar = (uint32_t*)(ws + L.bstar);
  p.cand_total = (uint32_t*)(ws + L.cand_total);
  p.cand_key = (uint32_t*)(ws + L.cand_key);
  p.cand_idx = (int32_t*)(ws + L.cand_idx);
  p.chunk_cnt = (uint32_t*)(ws + L.chunk_cnt);
  p.idx_out = idx_out;
  p.val_out = val_out;
  return p;
}

// with_select false: the latent attention makes the selection from the
// fused filter's candidates itself (the fused step only).
int run_topk(const sd::TopkPlan& p, bool hist_ready, hipStream_t s, bool with_select = true) {
  if (p.rows == 0) return SPARSE_OK;
  if (p.n_units == 0) {
    // nothing valid: the select kernel only pads
    HIPCHECK(sd::launch_topk_select(p, s));
    return SPARSE_OK;
  }
  if (!p.direct) {
    if (!hist_ready) HIPCHECK(sd::launch_topk_hist(p, s));
    if (p.fused) {
      HIPCHECK(sd::launch_topk_filter_fused(p, s));
    } else {
      HIPCHECK(sd::launch_topk_bin(p, s));
      HIPCHECK(sd::launch_topk_filter(p, s));
    }
  }
  if (with_select) HIPCHECK(sd::launch_topk_select(p, s));
  return SPARSE_OK;
}

int run_scores(const sparse_index_args& a, const IndexLayout& L, float* scores, uint32_t* hist,
               hipStream_t s) {
  sd::ScorePlan sp;
  sp.a = &a;
  sp.scores = scores;
  sp.hist = hist;
  sp.n_units = L.n_units;
  switch (a.kind) {
    case SPARSE_SCORE_DOT:
      HIPCHECK(sd::launch_score_dot(sp, s));
      break;
    case SPARSE_SCORE_LIGHTNING:
      HIPCHECK(sd::launch_score_lightning(sp, s));
      break;
    case SPARSE_SCORE_BITPLANE:
      // the scan selects the read depth in its own prologue (no plane list)
      HIPCHECK(sd::launch_score_bitplane(sp, s));
      break;
  }
  return SPARSE_OK;
}

// fused_tp: the fused filter's candidates, from which the attention selects
// (attn_selects) and writes the selection to sel_out; NULL: sel holds it.
int run_attn(const sparse_attn_args& a, const int32_t* sel, int sel_heads, int k,
             int sel_unit, float* out, float* lse, char* ws, size_t base, hipStream_t s,
             const sd::TopkPlan* fused_tp = nullptr, int32_t* sel_out = nullptr) {
  const int k_tokens = k * sel_unit;
  AttnLayout L = attn_layout(a, k_tokens, base);
  sd::AttnPlan p{};
  p.a = a;
  p.sel = sel;
  p.sel_heads = sel_heads;
  p.k = k;
  p.sel_unit = sel_unit;
  p.out = out;
  p.lse = lse;
  p.splits = L.splits;
  p.part = L.splits > 1 ? (float*)(ws + L.part) : nullptr;
  p.staging = a.hot_slot ? (uint16_t*)(ws + L.staging) : nullptr;
  p.k_tokens = k_tokens;
  p.fsel = fused_tp != nullptr;
  p.sel_out = sel_out;
  if (fused_tp) p.tk = *fused_tp;
  if (a.hot_slot) HIPCHECK(sd::launch_miss_fetch(p, s));
  if (a.dtype == SPARSE_F32) HIPCHECK(sd::launch_attn_f32(p, s));
  else HIPCHECK(sd::launch_attn_bf16(p, s));
  if (L.splits > 1) HIPCHECK(sd::launch_attn_combine(p, s));
  return SPARSE_OK;
}

// Argument checks of the fused step (before anything is launched) and the
// workspace it needs.
int check_step(const sparse_index_args* ia, const sparse_attn_args* aa, int32_t k,
               const int32_t* topk_out, const float* out, size_t* need) {
  int rc = check_index(ia);
  if (rc) return rc;
  const bool bitplane = ia->kind == SPARSE_SCORE_BITPLANE;
  const int sel_heads = bitplane ? ia->n_kv_heads : 1;
  const int unit = ia->kind == SPARSE_SCORE_DOT ? ia->block_size : 1;
  rc = check_attn(aa, sel_heads, k, unit);
  if (rc) return rc;
  CHECK(ia->batch == aa->batch, SPARSE_EINVAL, "index batch %d != attention batch %d",
        ia->batch, aa->batch);
  CHECK(ia->n <= aa->n, SPARSE_EINVAL, "index n %d > attention n %d", ia->n, aa->n);
  if (bitplane)
    CHECK(ia->n_kv_heads == aa->n_kv_heads, SPARSE_EINVAL, "KV heads differ");
  *need = 0;
  if (ia->batch == 0) return SPARSE_OK;
  CHECK(topk_out && out, SPARSE_EINVAL, "topk_out / out NULL");
  return sparse_workspace_size(ia, aa, k, need);
}

}  // namespace

extern "C" {

int sparse_abi_version(void) { return SPARSE_ABI_VERSION; }

const char* sparse_strerror(int status) {
  switch (status) {
    case SPARSE_OK: return "ok";
    case SPARSE_EINVAL: return "invalid argument";
    case SPARSE_EUNSUPPORTED: return "unsupported shape or dtype";
    case SPARSE_EWORKSPACE: return "workspace too small";
    case SPARSE_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* sparse_last_error(void) { return g_err; }

int sparse_workspace_size(const sparse_index_args* ia, const sparse_attn_args* aa,
                          int32_t k, size_t* bytes) {
  CHECK(bytes, SPARSE_EINVAL, "bytes is NULL");
  CHECK(ia || aa, SPARSE_EINVAL, "both args NULL");
  size_t total = 0;
  int unit = 1;
  if (ia) {
    int rc = check_index(ia);
    if (rc) return rc;
    total = index_layout(*ia, aa != nullptr).end;
    unit = ia->kind == SPARSE_SCORE_DOT ? ia->block_size : 1;
  }
  if (aa) {
    CHECK(k >= 1, SPARSE_EINVAL, "k %d < 1", k);
    total = attn_layout(*aa, k * unit, total).end;
  }
  *bytes = total;
  return SPARSE_OK;
}

int sparse_topk_workspace_size(int32_t rows, int32_t n_units, int32_t k, size_t* bytes) {
  CHECK(bytes, SPARSE_EINVAL, "bytes is NULL");
  CHECK(rows >= 0 && n_units >= 0 && k >= 1, SPARSE_EINVAL, "rows/n_units/k");
  sparse_index_args a;
  memset(&a, 0, sizeof(a));
  a.kind = SPARSE_SCORE_DOT;
  a.batch = rows;
  a.n = n_units;
  a.block_size = 1;
  *bytes = index_layout(a, false).end;
  return SPARSE_OK;
}

int sparse_read_depth(const sparse_index_args* ia, int8_t* depth_out, void* stream) {
  int rc = check_index(ia);
  if (rc) return rc;
  CHECK(ia->kind == SPARSE_SCORE_BITPLANE, SPARSE_EINVAL, "read depth needs kind BITPLANE");
  if (ia->batch == 0) return SPARSE_OK;
  CHECK(depth_out, SPARSE_EINVAL, "depth_out NULL");
  CHECK(ia->q, SPARSE_EINVAL, "q NULL");
  hipStream_t s = (hipStream_t)stream;
  HIPCHECK(sd::launch_read_depth(ia, depth_out, s));
  return SPARSE_OK;
}

int sparse_index_score(const sparse_index_args* ia, float* scores, void* ws,
                       size_t ws_bytes, void* stream) {
  int rc = check_index(ia);
  if (rc) return rc;
  if (ia->batch == 0 || ia->n == 0) return SPARSE_OK;
  CHECK(scores, SPARSE_EINVAL, "scores NULL");
  (void)ws;
  (void)ws_bytes;
  IndexLayout L = index_layout(*ia, false);
  return run_scores(*ia, L, scores, nullptr, (hipStream_t)stream);
}

int sparse_topk(const float* scores, int32_t rows, int32_t n_units, int64_t row_stride,
                const int32_t* valid_units, int32_t rows_per_valid, int32_t k,
                int32_t* idx_out, float* val_out, void* ws, size_t ws_bytes, void* stream) {
  CHECK(rows >= 0 && n_units >= 0, SPARSE_EINVAL, "negative rows or n_units");
  CHECK(k >= 1 && k <= (1 << 20), SPARSE_EINVAL, "k %d outside 1..1048576", k);
  CHECK(n_units <= sd::kTopkChunk * 1024, SPARSE_EUNSUPPORTED, "n_units above 4194304");
  if (rows == 0) return SPARSE_OK;
  CHECK(idx_out, SPARSE_EINVAL, "idx_out NULL");
  CHECK(n_units == 0 || scores, SPARSE_EINVAL, "scores NULL");
  CHECK(row_stride >= n_units, SPARSE_EINVAL, "row_stride < n_units");
  CHECK(!valid_units || rows_per_valid >= 1, SPARSE_EINVAL, "rows_per_valid < 1");
  size_t need = 0;
  sparse_topk_workspace_size(rows, n_units, k, &need);
  CHECK(ws && ws_bytes >= need, SPARSE_EWORKSPACE, "workspace %zu < %zu", ws_bytes, need);
  sparse_index_args a;
  memset(&a, 0, sizeof(a));
  a.kind = SPARSE_SCORE_DOT;
  a.batch = rows;
  a.n = n_units;
  a.block_size = 1;
  IndexLayout L = index_layout(a, false);
  sd::TopkPlan p = make_topk_plan(L, (char*)ws, scores, row_stride, valid_units,
                                  valid_units ? rows_per_valid : 1, 1, k, idx_out, val_out,
                                  L.n_chunks, sd::kTopkChunk);
  return run_topk(p, false, (hipStream_t)stream);
}

int sparse_gather_attn_decode(const sparse_attn_args* aa, const int32_t* sel,
                              int32_t sel_heads, int32_t k, int32_t sel_unit, float* out,
                              float* lse, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_attn(aa, sel_heads, k, sel_unit);
  if (rc) return rc;
  if (aa->batch == 0) return SPARSE_OK;
  CHECK(sel && out, SPARSE_EINVAL, "sel / out NULL");
  AttnLayout L = attn_layout(*aa, k * sel_unit, 0);
  CHECK(L.end == 0 || (ws && ws_bytes >= L.end), SPARSE_EWORKSPACE, "workspace %zu < %zu",
        ws_bytes, L.end);
  return run_attn(*aa, sel, sel_heads, k, sel_unit, out, lse, (char*)ws, 0,
                  (hipStream_t)stream);
}

int sparse_decode_step(const sparse_index_args* ia, const sparse_attn_args* aa, int32_t k,
                       int32_t* topk_out, float* out, float* lse, void* ws,
                       size_t ws_bytes, void* stream) {
  size_t need = 0;
  int rc = check_step(ia, aa, k, topk_out, out, &need);
  if (rc) return rc;
  if (ia->batch == 0) return SPARSE_OK;
  CHECK(ws && ws_bytes >= need, SPARSE_EWORKSPACE, "workspace %zu < %zu", ws_bytes, need);
  const bool bitplane = ia->kind == SPARSE_SCORE_BITPLANE;
  const int sel_heads = bitplane ? ia->n_kv_heads : 1;
  const int unit = ia->kind == SPARSE_SCORE_DOT ? ia->block_size : 1;
  hipStream_t s = (hipStream_t)stream;
  char* w = (char*)ws;
  IndexLayout L = index_layout(*ia, true);
  float* scores = (float*)(w + L.scores);
  sd::TopkPlan tp = make_topk_plan(L, w, scores, L.n_units, ia->seq_lens, L.rows_per_b,
                                   unit, k, topk_out, nullptr, L.hist_parts,
                                   sd::score_part_span(*ia));
  if (ia->n > 0) {
    rc = run_scores(*ia, L, scores, tp.direct ? nullptr : tp.hist, s);
    if (rc) return rc;
  }
  // Latent rows without a hot buffer: the attention selects from the fused
  // filter's candidates in its prologue and writes topk_out itself, instead
  // of a select launch whose output it would read back (lightning_128k:
  // see the latent attention's row table).
  const bool fsel = tp.fused && !tp.direct && tp.n_units > 0 && sel_heads == 1 &&
                    unit == 1 && sd::attn_selects(*aa);
  rc = run_topk(tp, true, s, !fsel);
  if (rc) return rc;
  return run_attn(*aa, topk_out, sel_heads, k, unit, out, lse, w, L.end, s,
                  fsel ? &tp : nullptr, topk_out);
}

int sparse_decode_step_noalloc(const sparse_index_args* ia, const sparse_attn_args* aa,
                               int32_t k, int32_t* topk_out, float* out, float* lse,
                               void* stream) {
  size_t need = 0;
  int rc = check_step(ia, aa, k, topk_out, out, &need);
  if (rc) return rc;
  if (ia->batch == 0) return SPARSE_OK;
  CHECK(need <= kNoAllocScratchBytes, SPARSE_EWORKSPACE,
        "this step needs %zu bytes of scratch, above the %zu bytes the no-allocation "
        "entry point holds per device; use sparse_decode_step with a workspace",
        need, kNoAllocScratchBytes);
  int dev = 0;
  HIPCHECK(hipGetDevice(&dev));
  CHECK(dev >= 0 && dev < kMaxDevices, SPARSE_EUNSUPPORTED, "device %d above %d", dev,
        kMaxDevices - 1);
  void* ptr = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
      void* p = nullptr;
      HIPCHECK(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
      CHECK(p != nullptr, SPARSE_EHIP, "no device address for the scratch array");
      g_scratch_ptr[dev] = p;
    }
    ptr = g_scratch_ptr[dev];
  }
  return sparse_decode_step(ia, aa, k, topk_out, out, lse, ptr, kNoAllocScratchBytes,
                            stream);
}

int sparse_append_token(const sparse_index_args* ia, const sparse_attn_args* aa,
                        const int32_t* pos, const float* index_key_new, const void* k_new,
                        const void* v_new, void* stream) {
  CHECK(ia || aa, SPARSE_EINVAL, "both args NULL");
  int batch = -1;
  if (ia) {
    CHECK(ia->kind >= 0 && ia->kind <= 2, SPARSE_EINVAL, "unknown score kind %d", ia->kind);
    CHECK(ia->batch >= 0 && ia->n >= 0, SPARSE_EINVAL, "negative batch or n");
    CHECK(ia->head_dim == 128, SPARSE_EUNSUPPORTED, "head_dim %d (only 128)", ia->head_dim);
    batch = ia->batch;
    if (ia->batch > 0) {
      CHECK(index_key_new, SPARSE_EINVAL, "index_key_new NULL");
      if (ia->kind == SPARSE_SCORE_DOT) {
        CHECK(ia->keys && (ia->k_dtype == SPARSE_F32 || ia->k_dtype == SPARSE_BF16),
              SPARSE_EINVAL, "DOT keys NULL or not f32/bf16");
      } else if (ia->kind == SPARSE_SCORE_LIGHTNING) {
        CHECK(ia->keys && ia->k_scale && ia->k_dtype == SPARSE_E4M3FN, SPARSE_EINVAL,
              "LIGHTNING keys / k_scale NULL or keys not e4m3fn");
        CHECK(ia->k_stride_t % 2 == 0 && ia->k_stride_b % 2 == 0 &&
                  ((uintptr_t)ia->keys & 1u) == 0,
              SPARSE_EINVAL, "LIGHTNING key rows must be 2-byte aligned");
      } else {
        CHECK(ia->n_kv_heads >= 1 && ia->planes && ia->chan_zero && ia->chan_scale,
              SPARSE_EINVAL, "BITPLANE planes / chan_zero / chan_scale NULL");
      }
    }
  }
  if (aa) {
    CHECK(aa->batch >= 0 && aa->n >= 0 && aa->n_kv_heads >= 1, SPARSE_EINVAL,
          "attention batch / n / n_kv_heads");
    CHECK(batch < 0 || batch == aa->batch, SPARSE_EINVAL, "batch differs between args");
    batch = aa->batch;
    CHECK(aa->dtype == SPARSE_F32 || aa->dtype == SPARSE_BF16, SPARSE_EUNSUPPORTED,
          "attention dtype %d", aa->dtype);
    const int64_t e = esize(aa->dtype);
    CHECK((aa->d_qk * e) % 16 == 0 && (aa->v_cache == nullptr || (aa->d_v * e) % 16 == 0),
          SPARSE_EUNSUPPORTED, "row widths must be multiples of 16 bytes");
    if (aa->batch > 0) {
      CHECK(k_new && aligned16(k_new), SPARSE_EINVAL, "k_new NULL or not 16-byte aligned");
      CHECK(aa->v_cache == nullptr || (v_new && aligned16(v_new)), SPARSE_EINVAL,
            "v_new NULL or not 16-byte aligned");
      if (aa->hot_slot) {
        CHECK(aa->v_cache == nullptr, SPARSE_EUNSUPPORTED, "hot buffer: latent rows only");
        CHECK(aa->host_kv && aligned16(aa->host_kv) && (aa->host_stride_t * e) % 16 == 0 &&
                  (aa->host_stride_b * e) % 16 == 0,
              SPARSE_EINVAL, "host_kv NULL or misaligned");
      } else {
        CHECK(aa->k_cache && aligned16(aa->k_cache), SPARSE_EINVAL,
              "k_cache NULL or not 16-byte aligned");
        CHECK(aa->v_cache == nullptr || aligned16(aa->v_cache), SPARSE_EINVAL,
              "v_cache not 16-byte aligned");
        CHECK((aa->kv_stride_t * e) % 16 == 0 && (aa->kv_stride_h * e) % 16 == 0 &&
                  (aa->kv_stride_b * e) % 16 == 0,
              SPARSE_EINVAL, "KV strides must be multiples of 16 bytes");
        if (aa->page_table) CHECK(aa->page_size >= 1, SPARSE_EINVAL, "page_size < 1");
      }
    }
  }
  if (batch == 0) return SPARSE_OK;
  CHECK(pos, SPARSE_EINVAL, "pos NULL");
  HIPCHECK(sd::launch_append(ia, aa, pos, index_key_new, k_new, v_new, batch,
                             (hipStream_t)stream));
  return SPARSE_OK;
}

int sparse_hot_update(const sparse_index_args* ia, const sparse_attn_args* aa,
                      const int32_t* sel, int32_t k, int32_t sel_unit, int32_t n_slots,
                      int32_t step, int32_t* slot_token, int32_t* slot_stamp, void* ws,
                      size_t ws_bytes, void* stream) {
  int rc = check_attn(aa, 1, k, sel_unit);
  if (rc) return rc;
  CHECK(aa->hot_slot, SPARSE_EINVAL, "hot_slot NULL: no hot buffer to update");
  CHECK(n_slots >= 1 && n_slots <= sd::kHotMaxSlots, SPARSE_EUNSUPPORTED,
        "n_slots %d outside 1..%d", n_slots, sd::kHotMaxSlots);
  CHECK(step >= 0, SPARSE_EINVAL, "step %d < 0", step);
  CHECK((int64_t)k * sel_unit <= sd::kHotMaxSel, SPARSE_EUNSUPPORTED,
        "%d selected tokens above %d", k * sel_unit, sd::kHotMaxSel);
  size_t base = 0;
  if (ia) {
    rc = check_index(ia);
    if (rc) return rc;
    const int unit = ia->kind == SPARSE_SCORE_DOT ? ia->block_size : 1;
    CHECK(unit == sel_unit, SPARSE_EINVAL, "sel_unit %d differs from the index unit %d",
          sel_unit, unit);
    CHECK(ia->batch == aa->batch, SPARSE_EINVAL, "index batch %d != attention batch %d",
          ia->batch, aa->batch);
    base = index_layout(*ia, true).end;
  }
  if (aa->batch == 0) return SPARSE_OK;
  CHECK(sel && slot_token && slot_stamp, SPARSE_EINVAL, "sel / slot_token / slot_stamp NULL");
  AttnLayout L = attn_layout(*aa, k * sel_unit, base);
  CHECK(ws && ws_bytes >= L.end, SPARSE_EWORKSPACE, "workspace %zu < %zu", ws_bytes, L.end);
  sd::HotPlan p;
  p.a = *aa;
  p.sel = sel;
  p.k = k;
  p.sel_unit = sel_unit;
  p.k_tokens = k * sel_unit;
  p.n_slots = n_slots;
  p.step = step;
  p.slot_token = slot_token;
  p.slot_stamp = slot_stamp;
  p.staging = (const uint16_t*)((const char*)ws + L.staging);
  HIPCHECK(sd::launch_hot_update(p, (hipStream_t)stream));
  return SPARSE_OK;
}

int sparse_hot_prefetch(const sparse_attn_args* aa, const int32_t* cand, int32_t m,
                        int32_t n_slots, int32_t step, int32_t* slot_token,
                        int32_t* slot_stamp, void* stream) {
  int rc = check_attn(aa, 1, m, 1);
  if (rc) return rc;
  CHECK(aa->hot_slot, SPARSE_EINVAL, "hot_slot NULL: no hot buffer to prefetch into");
  CHECK(n_slots >= 1 && n_slots <= sd::kHotMaxSlots, SPARSE_EUNSUPPORTED,
        "n_slots %d outside 1..%d", n_slots, sd::kHotMaxSlots);
  CHECK(step >= 0, SPARSE_EINVAL, "step %d < 0", step);
  CHECK(m <= sd::kHotMaxSel, SPARSE_EUNSUPPORTED, "%d candidates above %d", m,
        sd::kHotMaxSel);
  if (aa->batch == 0) return SPARSE_OK;
  CHECK(cand && slot_token && slot_stamp, SPARSE_EINVAL, "cand / slot_token / slot_stamp NULL");
  sd::HotPlan p;
  p.a = *aa;
  p.sel = cand;
  p.k = m;
  p.sel_unit = 1;
  p.k_tokens = m;
  p.n_slots = n_slots;
  p.step = step;
  p.slot_token = slot_token;
  p.slot_stamp = slot_stamp;
  p.staging = nullptr;  // prefetch: rows from host_kv
  HIPCHECK(sd::launch_hot_update(p, (hipStream_t)stream));
  return SPARSE_OK;
}

int sparse_host_device_pointer(void* host_ptr, void** dev_ptr) {
  CHECK(host_ptr && dev_ptr, SPARSE_EINVAL, "NULL pointer");
  HIPCHECK(hipHostGetDevicePointer(dev_ptr, host_ptr, 0));
  return SPARSE_OK;
}

}  // extern "C"
