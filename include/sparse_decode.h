/*
 * sparse_decode.h -- C ABI of a decode step of indexer-driven sparse
 * attention on AMD Instinct MI355X (gfx950).
 *
 * Per request (and per KV head where stated) one decode step
 *   1. scores every cached key against the current query (the indexer pass),
 *   2. selects the top-k tokens or 64-token blocks,
 *   3. runs exact softmax attention over only the selected KV rows.
 *
 * Sources, cited by page title and passage:
 *   [XM] "XM-Sparse: Pushing the Throughput Frontier of Sparse Attention with
 *        Netpreme X-Mem": opening paragraph (each decode step reads only the
 *        selected KV entries; the indexer key cache, the K-index, stays in
 *        HBM), Figure 1 caption (missing selected entries are fetched from
 *        host memory into HBM), the modelling paragraphs (2,048 selected
 *        entries per layer and step, a 4,096-token hot KV buffer per request)
 *        and the KV-lifecycle list (only the selected KV is fetched).
 *   [MM] "MiniMax-M3: share the sparse index top-k across layers and reuse
 *        the decode top-k buffer": description (a lightning-indexer pass
 *        picks the top-k KV blocks; the first layer of a group writes the
 *        selection into a persistent int32 buffer that later layers reuse;
 *        no allocation, so graph capture never allocates; on ROCm a fixed
 *        tile configuration instead of runtime autotuning).
 *   [FA] "Fathom: Per-Query Read Depth for Sparse Decoding over Offloaded KV
 *        Caches": abstract (4-bit K stored channel-major as bit planes; the
 *        first t planes of a channel form its t-bit quantizer; a query
 *        divides its per-key bit budget among the channels by reverse
 *        water-filling on variance-weighted channel importance).
 *
 * Conventions shared by every entry point
 *   - All pointers are device pointers owned by the caller unless stated.
 *     The library never allocates, frees or synchronises; all scratch comes
 *     from the caller's workspace `ws` of `ws_bytes` bytes (256-byte aligned).
 *   - All work is enqueued on `stream` (a hipStream_t passed as void*; NULL =
 *     the default stream), so every call can be captured in a HIP graph.
 *   - Strides are in elements of the tensor's own type.  The innermost
 *     dimension (head_dim, row width) is always contiguous.
 *   - Return value: SPARSE_OK, or an error code.  Arguments are validated
 *     before anything is launched; on an error nothing is launched and no
 *     output is written.  A failed launch returns SPARSE_EHIP.
 *     sparse_last_error() gives a thread-local message for the last error.
 *   - Same inputs give bit-identical outputs (fixed reduction orders, no
 *     floating-point atomics on any result).
 */
#ifndef SPARSE_DECODE_H
#define SPARSE_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPARSE_ABI_VERSION 2

enum sparse_status {
  SPARSE_OK = 0,
  SPARSE_EINVAL = 1,       /* a null pointer, a negative or inconsistent size */
  SPARSE_EUNSUPPORTED = 2, /* a valid shape or dtype with no kernel here */
  SPARSE_EWORKSPACE = 3,   /* ws too small (see sparse_workspace_size) */
  SPARSE_EHIP = 4          /* the HIP runtime reported an error */
};

enum sparse_dtype {
  SPARSE_F32 = 0,
  SPARSE_BF16 = 1,
  SPARSE_E4M3FN = 2 /* OCP FP8 E4M3 (no infinities, 0x7F/0xFF = NaN) */
};

enum sparse_score_kind {
  /* s_t = sum_h q_h . k_t over the index heads (no weights, no ReLU).
   * With block_size 64 the unit score is the max over the block's valid
   * tokens: the block-level selection of [MM].                            */
  SPARSE_SCORE_DOT = 0,
  /* Lightning indexer over an fp8 K-index with a per-token fp32 scale:
   * s_t = sum_h w_h * max(0, q_h . (scale_t * k8_t)).  [XM] opening
   * paragraph (K-index in HBM), [MM] description (the indexer pass).      */
  SPARSE_SCORE_LIGHTNING = 1,
  /* Fathom scan [FA]: per (request, KV head), q_bar = sum of the group's
   * query heads; read depth t_c by reverse water-filling (sparse_read_depth);
   * s_t = sum_c q_bar_c * (zero_c + scale_c * (P_c(t) + 2^(3 - t_c))) where
   * P_c(t) = sum_{j < t_c} plane_{c,j}(t) * 2^(3-j).  One score row per KV
   * head.                                                                  */
  SPARSE_SCORE_BITPLANE = 2
};

/* Arguments of the indexer pass. */
typedef struct sparse_index_args {
  int32_t kind;            /* enum sparse_score_kind */
  int32_t batch;           /* B >= 0 */
  int32_t n;               /* token capacity per request, 0 <= n <= 4194304
                              (EUNSUPPORTED above) */
  const int32_t* seq_lens; /* [B] valid tokens per request (<= n); NULL = n */

  int32_t n_heads;  /* DOT/LIGHTNING: index query heads H.  BITPLANE: the
                       attention query heads Hq (a multiple of n_kv_heads) */
  int32_t head_dim; /* D; 128 is the size with kernels                    */

  const void* q;      /* [B][H][D] at q_stride_b / q_stride_h             */
  int32_t q_dtype;    /* DOT: F32 or BF16.  LIGHTNING/BITPLANE: BF16      */
  int64_t q_stride_b;
  int64_t q_stride_h;

  const float* head_w; /* LIGHTNING: [B][H] weights w_h (w_stride_b)      */
  int64_t w_stride_b;

  const void* keys;   /* DOT: [B][n][D] F32/BF16; LIGHTNING: [B][n][D]
                         E4M3FN; rows at k_stride_b / k_stride_t.
                         LIGHTNING: n * k_stride_t must stay below 2^31
                         bytes (EUNSUPPORTED otherwise)                   */
  int32_t k_dtype;
  int64_t k_stride_b;
  int64_t k_stride_t;

  const float* k_scale; /* LIGHTNING: [B][n] per-token fp32 scale (> 0)  */
  int64_t ks_stride_b;

  int32_t block_size; /* DOT: 1 (token units) or 64 (block units); others 1 */

  /* BITPLANE */
  int32_t n_kv_heads;       /* Hkv                                        */
  const uint32_t* planes;   /* [B][Hkv][D][4][ceil(n/32)]: plane j of a
                               channel holds bit (3-j) of the 4-bit code;
                               bit i of word w is token 32w + i            */
  const float* chan_zero;   /* [B][Hkv][D] quantizer zero (channel min)   */
  const float* chan_scale;  /* [B][Hkv][D] 4-bit cell width ((max-min)/16) */
  const float* chan_var;    /* [B][Hkv][D] channel variance var_c (unused
                               with depth_in)                              */
  int32_t bit_budget;       /* bits read per key per KV head, 0..4*D      */
  /* BITPLANE, nullable: [B][Hkv][D] int8 read depths t_c given by the
   * caller (values clamped to 0..4), in place of the reverse water-filling
   * over chan_var and bit_budget -- a fixed allocation, e.g. the same
   * prefix for every query.  The scan, its score constant and the plane
   * weights follow these depths exactly as they follow computed ones.     */
  const int8_t* depth_in;
} sparse_index_args;

/* Arguments of the sparse attention. */
typedef struct sparse_attn_args {
  int32_t batch;           /* B (equal to the index pass's B in the fused step) */
  int32_t n;               /* token capacity per request; with n == 0 no row
                              is ever read: k_cache, page_table and the
                              hot-buffer pointers may be NULL (v_cache still
                              tells K/V rows from latent rows), and every
                              output row is 0 with log-sum-exp -inf         */
  const int32_t* seq_lens; /* [B] valid tokens; NULL = n                    */
  int32_t n_q_heads;       /* Hq                                            */
  int32_t n_kv_heads;      /* Hkv, Hq % Hkv == 0                            */
  int32_t d_qk;            /* query/key width: 128 or 576                   */
  int32_t d_v;             /* value width: 128, or 512 with d_qk 576        */
  int32_t dtype;           /* F32 (d_qk = d_v = 128) or BF16                */

  const void* q;           /* [B][Hq][d_qk] at q_stride_b / q_stride_h      */
  int64_t q_stride_b;
  int64_t q_stride_h;

  /* KV rows.  Token t of request b, KV head h starts at
   *   contiguous: k_cache + b*kv_stride_b + t*kv_stride_t + h*kv_stride_h
   *   paged:      k_cache + (page_table[b*pt_stride_b + t/page_size]
   *                          * page_size + t%page_size) * kv_stride_t
   *                       + h*kv_stride_h                                  */
  const void* k_cache;
  const void* v_cache;     /* NULL: latent (MLA) rows, value = the first d_v
                              elements of the key row (read once)          */
  int64_t kv_stride_b;
  int64_t kv_stride_t;
  int64_t kv_stride_h;
  const int32_t* page_table; /* NULL = contiguous                         */
  int64_t pt_stride_b;
  int32_t page_size;

  float sm_scale;          /* softmax scale, e.g. 1/sqrt(d_qk)              */

  /* Hot buffer ([XM] Figure 1): when hot_slot is not NULL the full latent
   * KV lives in host memory and only hot rows are in HBM.  The step reads a
   * selected token from hot_kv[b][hot_slot[b][t]] when the slot is >= 0,
   * else it fetches the row from host_kv (a device-visible pointer of
   * pinned host memory, see sparse_host_device_pointer) into workspace
   * staging first.  Latent (v_cache NULL), contiguous layout only.        */
  const int32_t* hot_slot; /* [B][n] slot or -1, at hs_stride_b            */
  int64_t hs_stride_b;
  const void* hot_kv;      /* [B][slots][d_qk] at hot_stride_b/hot_stride_s */
  int64_t hot_stride_b;
  int64_t hot_stride_s;
  const void* host_kv;     /* [B][n][d_qk] at host_stride_b/host_stride_t  */
  int64_t host_stride_b;
  int64_t host_stride_t;
} sparse_attn_args;

int sparse_abi_version(void);
const char* sparse_strerror(int status);
const char* sparse_last_error(void);

/* Bytes of workspace the calls below need.  [MM] description and ROCm
 * note: the decode top-k buffer is allocated once per batch size and never
 * inside a layer, so a captured graph never allocates; here every scratch
 * byte of a step (scores, histogram parts, candidate lists, attention
 * partials, miss staging) likewise lives in one caller-owned workspace,
 * sized once by this call and reused by every step.  Either args pointer
 * may be NULL: with only `ia`, enough for sparse_index_score +
 * sparse_topk of those scores; with only `aa`, enough for
 * sparse_gather_attn_decode; with both, enough for sparse_decode_step.  k is
 * the number of selected units (k >= 1).  bytes: out, the size.  Errors: the
 * argument checks of the matching entry points (nothing is launched). */
int sparse_workspace_size(const sparse_index_args* ia,
                          const sparse_attn_args* aa, int32_t k,
                          size_t* bytes);

/* Workspace for sparse_topk over `rows` rows of `n_units` scores (see
 * sparse_workspace_size for why scratch is the caller's). */
int sparse_topk_workspace_size(int32_t rows, int32_t n_units, int32_t k,
                               size_t* bytes);

/* Step a1 of [FA]: per (request, KV head) read depth t_c in 0..4 with
 * sum_c t_c = bit_budget.  q_bar_c = ((q_0 + q_1) + ...) over the group's
 * query heads in float64, importance imp_c = (q_bar_c * q_bar_c) * var_c,
 * gains imp_c * 4^-j for planes j = 0..3, the bit_budget largest gains are
 * taken (ties: lower channel, then lower plane); t_c counts the taken planes
 * of channel c.  With depth_in set, depth_out receives those depths
 * (clamped to 0..4).  depth_out: [B][Hkv][D] int8.  Only kind BITPLANE. */
int sparse_read_depth(const sparse_index_args* ia, int8_t* depth_out,
                      void* stream);

/* Step a2: index scores.  [XM] opening paragraph: the indexer scans the
 * K-index that stays in HBM and scores every cached key against the current
 * query; [MM] description: the lightning-indexer pass (and its reduction
 * to KV blocks) runs in the first layer of a group; [FA] abstract: the
 * per-token scan reads each channel's plane prefix (depths as for
 * sparse_read_depth).  scores: [B][R][n_units] fp32, device, caller-owned,
 * with R = 1 (DOT, LIGHTNING) or R = Hkv (BITPLANE) and n_units =
 * ceil(n / block_size).  Units at or past a request's valid length are
 * written as -inf.  ws, ws_bytes: not used by any kind (the bit-plane scan
 * selects its read depths in its own prologue); may be NULL / 0.  Errors:
 * EINVAL / EUNSUPPORTED from the argument checks, EHIP. */
int sparse_index_score(const sparse_index_args* ia, float* scores, void* ws,
                       size_t ws_bytes, void* stream);

/* Step a3: exact top-k of each score row.  [MM] description: the top-k
 * KV blocks are written into a persistent int32 buffer that later layers
 * read; [XM] modelling paragraphs: 2,048 entries per layer and step.  Row r
 * starts at scores + r*row_stride (device fp32) and has n_units entries of
 * which the first valid_units[r / rows_per_valid] are valid (valid_units
 * NULL = all; rows_per_valid lets the rows of one request -- e.g. its KV
 * heads -- share one length entry).  Ties go to the lower index.  idx_out:
 * [rows][k] int32, the selected unit indices in ascending order, -1-padded
 * when fewer than k are valid.  val_out (nullable): [rows][k] their scores
 * (-inf for padding).  Scores must not be NaN.  ws: sparse_topk_workspace_
 * size bytes.  Errors: EINVAL (sizes, NULL outputs), EUNSUPPORTED
 * (n_units above 4194304), EWORKSPACE, EHIP. */
int sparse_topk(const float* scores, int32_t rows, int32_t n_units,
                int64_t row_stride, const int32_t* valid_units,
                int32_t rows_per_valid, int32_t k, int32_t* idx_out,
                float* val_out, void* ws, size_t ws_bytes, void* stream);

/* Step a6 (with a4, and a5 when aa->hot_slot is set): attention of each
 * query head over the selected units ([XM] opening paragraph: a step reads
 * only the selected KV entries; Figure 1 caption: selected entries missing
 * from the hot buffer are fetched from host memory).  Padding entries and
 * tokens past seq_len read no caller memory.  sel: [B][sel_heads][k] int32 unit
 * ids (-1 = padding), sel_heads = 1 (shared by all KV heads) or Hkv (query
 * head h uses row h / (Hq/Hkv)).  sel_unit = 1 (tokens) or 64 (a unit u is
 * tokens 64u .. 64u+63; tokens past seq_len are skipped).
 * out: [B][Hq][d_v] fp32.  lse (nullable): [B][Hq] natural-log sum of
 * exp(sm_scale * q.k) over the attended rows; an empty selection gives
 * out = 0 and lse = -inf.  This is also the reuse path of [MM]: a later
 * layer passes the earlier layer's persistent top-k buffer as sel. */
int sparse_gather_attn_decode(const sparse_attn_args* aa, const int32_t* sel,
                              int32_t sel_heads, int32_t k, int32_t sel_unit,
                              float* out, float* lse, void* ws,
                              size_t ws_bytes, void* stream);

/* The fused step: index scores -> top-k -> attention.  topk_out:
 * [B][R][k] int32 (R as in sparse_index_score), the caller's persistent
 * selection buffer ([MM]); it is written and then read by the attention.
 * For BITPLANE the selection is per KV head (sel_heads = Hkv); otherwise
 * one selection per request.  The selection unit is ia->block_size. */
int sparse_decode_step(const sparse_index_args* ia, const sparse_attn_args* aa,
                       int32_t k, int32_t* topk_out, float* out, float* lse,
                       void* ws, size_t ws_bytes, void* stream);

/* sparse_decode_step without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.  The step's scratch lives in a
 * fixed device array of the library, SPARSE_NOALLOC_SCRATCH_BYTES (128 MiB)
 * per device, which each GPU the library runs on holds from its first use
 * until the process ends; nothing is allocated or freed by the call.  A step
 * whose sparse_workspace_size exceeds that returns SPARSE_EWORKSPACE before
 * anything is launched (at 128K context this covers batch 32 of the
 * lightning indexer, not the hot-buffer batches of 109 or 241).  Every call
 * on one GPU shares that GPU's array: calls that overlap on one GPU (two
 * streams, or two host threads) race and must be ordered by the caller.
 * The first call on each device looks the array's address up and should be
 * made outside graph capture.  Arguments, outputs and errors otherwise as
 * for sparse_decode_step. */
#define SPARSE_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
int sparse_decode_step_noalloc(const sparse_index_args* ia,
                               const sparse_attn_args* aa, int32_t k,
                               int32_t* topk_out, float* out, float* lse,
                               void* stream);

/* Decode-side append: after a step, the new token of each request joins
 * the history the next step reads -- [XM] KV-lifecycle list (generated KV
 * is appended to the history), [MM] the decode path's sparse-KV store (the
 * step's KV and index entries are written once; a repeated write is
 * idempotent), [FA] abstract (the 4-bit K is stored channel-major as bit
 * planes).  pos: [B] int32, the token position of the new entry; a request
 * whose pos is outside 0..n-1 is skipped.  Either struct may be NULL.
 *   aa (attention history): k_new [B][Hkv][d_qk] (aa->dtype) is written as
 *     the K row (the latent row when v_cache is NULL) of token pos[b] of
 *     each KV head, at the address the attention reads it from (contiguous,
 *     paged, or -- with a hot buffer -- the pinned host KV through host_kv;
 *     the hot buffer itself is not changed); v_new [B][Hkv][d_v] is the V
 *     row when v_cache is set (NULL otherwise).
 *   ia (index): index_key_new holds the new, unquantised key in fp32:
 *     DOT        [B][D]: stored in the keys' dtype (bf16: round to nearest
 *                even); block scores of a partly filled block change.
 *     LIGHTNING  [B][D]: scale = max|k| / 448 in fp32 (1 for an all-zero
 *                key) into k_scale, and each byte the OCP E4M3FN value
 *                nearest to clamp(k / scale, -448, 448) (fp32 division;
 *                ties to the even code).
 *     BITPLANE   [B][Hkv][D]: code = min(max(floor((k - zero) / cell), 0),
 *                15) in fp64 against chan_zero / chan_scale (0 when cell
 *                is 0); bit (3 - j) of the code goes to bit pos % 32 of word
 *                pos / 32 of plane j.  The quantizer is not refitted.
 * Only the head_dim 128 index layouts are written; q, head_w, chan_var and
 * seq_lens are not used.  Nothing else is read or written. */
int sparse_append_token(const sparse_index_args* ia, const sparse_attn_args* aa,
                        const int32_t* pos, const float* index_key_new,
                        const void* k_new, const void* v_new, void* stream);

/* Hot-buffer replacement, to run right after the step that used the hot
 * buffer ([XM] Figure 1 and decode-path list: the hot KV buffer in HBM and
 * the fetch of the missing selected rows; the page keeps HiSparse's cache
 * management without stating its rule, and this is least recently used).
 * Call it with the same ia (NULL after sparse_gather_attn_decode), aa, k,
 * sel_unit and workspace as that call, whose fetched rows the workspace
 * still holds, and with hot_slot unchanged since.  Per request:
 *   - a selected token held in a slot (a hit) stamps the slot with step;
 *   - the selected tokens not held (misses), in selection order, take the
 *     slots not stamped step that have the smallest (stamp, slot index),
 *     in ascending slot order: the slot's previous token loses its slot
 *     (hot_slot -1), the miss's row is copied into hot_kv, hot_slot of the
 *     miss becomes the slot, and the slot is stamped step;
 *   - misses beyond the slots available stay out.
 * sel: [B][k] the step's selection (distinct tokens, -1 padding); n_slots:
 * the hot_kv rows per request (1..8192); at most 4096 selected tokens per
 * request.  slot_token [B][n_slots] int32: the token a slot holds, or -1;
 * slot_stamp [B][n_slots] int32: the step of the slot's last hit or fill,
 * -1 for never (stamps >= -1; a stamp >= step marks a slot as kept this
 * time).  step >= 0 must grow from call to call for the order to be least
 * recently used.  hot_slot (aa) and hot_kv (aa) are written in place; it
 * is the caller's job to keep hot_slot and slot_token consistent (each the
 * other's inverse) between calls.  Prefetch is not done. */
int sparse_hot_update(const sparse_index_args* ia, const sparse_attn_args* aa,
                      const int32_t* sel, int32_t k, int32_t sel_unit,
                      int32_t n_slots, int32_t step, int32_t* slot_token,
                      int32_t* slot_stamp, void* ws, size_t ws_bytes,
                      void* stream);

/* Hot-buffer prefetch: preload rows the next steps are likely to select
 * ([XM] the paragraph on X-Mem's APIs: HiSparse's prefetch mechanism is
 * kept, without being stated, and every measured run has it off;
 * CXL-SpecKV's abstract: speculative preloading of the entries future
 * tokens will use).  The caller names the candidates, e.g. the tokens
 * ranked just below the step's top-k (a top-(k+m) selection holds them).
 * Run it after sparse_hot_update with the same step.  Per request:
 *   - a resident candidate is left as it is: not replaced by this call and
 *     not stamped;
 *   - the other candidates, in list order, take the slots that are neither
 *     stamped step nor holding a resident candidate, smallest (stamp, slot
 *     index) first, in ascending slot order: the slot's previous token
 *     loses its slot (hot_slot -1), the candidate's row is copied from
 *     host_kv (over PCIe) into hot_kv, hot_slot of the candidate becomes
 *     the slot, and the slot is stamped step;
 *   - candidates beyond the slots available stay out.
 * aa: the hot-buffer attention arguments (hot_slot, hot_kv, host_kv, n,
 * seq_lens); cand: [B][m] distinct token ids, -1 padding, tokens at or past
 * the valid length ignored; m: 1..4096; n_slots, step, slot_token and
 * slot_stamp as for sparse_hot_update, updated in place.  No workspace.
 * Errors as for sparse_hot_update; nothing is launched on an error. */
int sparse_hot_prefetch(const sparse_attn_args* aa, const int32_t* cand, int32_t m,
                        int32_t n_slots, int32_t step, int32_t* slot_token,
                        int32_t* slot_stamp, void* stream);

/* Device-visible address of pinned host memory allocated with
 * hipHostMalloc (e.g. a pinned torch tensor); used for host_kv. */
int sparse_host_device_pointer(void* host_ptr, void** dev_ptr);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_DECODE_H */
