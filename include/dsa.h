/*
 * dsa.h -- C ABI of a gfx950 (MI355X) implementation of the DeepSeek-style
 * sparse attention (DSA) step over a block-packed paged cache.
 *
 * Pages cited (title, then section):
 *   [ZH]     "vLLM 为 Kimi K3.1 Pro 提供 Day-0 支持"
 *   [EN]     "vLLM Adds Day-0 Support for Moonshot AI's Kimi K3.1 Pro"
 *   [RECIPE] "moonshotai/Kimi-K3.1-Pro"
 *
 * The step, per DSA layer ([ZH] "K3.1 Pro 中的稀疏注意力", figure 1):
 *   1. dsa_resolve_pages      block table -> kernel page addresses
 *   2. dsa_indexer_score      every earlier token scored by a 32-head indexer
 *   3. dsa_topk               the 2048 best tokens kept per query row
 *   4. dsa_sparse_mla_decode / dsa_sparse_mla_prefill
 *                             exact MLA attention over only those tokens
 * The fused decode path does steps 1-3 in one call and attends over physical rows:
 *   dsa_indexer_select        scores + exact top-k + physical rows, pages found
 *                             through the block table (no separate resolve)
 *   dsa_sparse_mla_decode_phys  attention over physical rows
 * The prefill indexer on FP8 MFMA with an exact top-k (a band of tokens rescored exactly):
 *   dsa_prefill_select        = dsa_prefill_score_fp8 (= dsa_prefill_prepare_fp8 +
 *                               dsa_prefill_gemm_fp8) + dsa_prefill_topk_band
 * and, for decode context parallelism emulated on one GPU:
 *   dsa_dcp_topk              the exact top-k merge across token shards
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Memory: every buffer is allocated by the caller.  Pointers documented
 *    as "device" must be device (HBM) memory; "host" means host memory.  The
 *    library allocates no device memory; scratch space is a caller buffer
 *    sized by the matching *_workspace_size call.
 *  - Streams: device calls enqueue asynchronously on `stream` (a hipStream_t
 *    passed as an opaque pointer; NULL = the null stream) and never block
 *    the host.  Calls hold no state between them and may be made from any
 *    thread; calls that share a workspace must not overlap.
 *  - Errors: arguments are checked on the host before anything is
 *    enqueued; a bad argument returns a non-zero dsa_status and enqueues
 *    nothing.  DSA_ERR_HIP means a launch failed (hipGetLastError).  Errors
 *    in device data (a block id outside the pool, an index past a request's
 *    context, ...) cannot be seen on the host: kernels OR a DSA_DEVERR_* bit
 *    into the optional device int32 `err_flag` (NULL = do not report), skip
 *    the offending element, and never trap.
 *  - Layouts are row-major; `*_ld` arguments are leading dimensions in
 *    elements.  bf16 values are passed as uint16_t bit patterns.
 *  - Floating-point data must be finite; NaN/Inf inputs give unspecified
 *    (but memory-safe) results.
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void *dsa_stream_t; /* hipStream_t */
typedef int32_t dsa_status;

#define DSA_OK 0
#define DSA_ERR_NULL_ARG 1            /* a required pointer is NULL */
#define DSA_ERR_BAD_SHAPE 2           /* a size, count or leading dimension is invalid */
#define DSA_ERR_MISALIGNED 3          /* a pointer lacks the alignment stated for it */
#define DSA_ERR_UNSUPPORTED 4         /* a format, head count or size the library does not run */
#define DSA_ERR_WORKSPACE_TOO_SMALL 5 /* workspace_bytes < the *_workspace_size answer */
#define DSA_ERR_HIP 6                 /* a HIP launch failed */
#define DSA_ERR_SCRATCH_LIMIT 7       /* needs more than the static scratch of the *_noalloc calls */

/* Bits kernels OR into *err_flag. */
#define DSA_DEVERR_BLOCK_RANGE 1u  /* block id outside [0, pool_rows) */
#define DSA_DEVERR_PAGE_COUNT 2u   /* n_pages outside [0, max_pages] */
#define DSA_DEVERR_PAGE_OFFSET 4u  /* page offset negative or page outside the pool */
#define DSA_DEVERR_ROW_LEN 8u      /* row_len outside [0, ld] or past the page table */
#define DSA_DEVERR_INDEX 16u       /* selected index outside [0, ctx_len) */
#define DSA_DEVERR_REQUEST 32u     /* q_req outside [0, n_req) */
#define DSA_DEVERR_BOUND 64u       /* dsa_prefill_select: a score outside its error bound */

/* Index-key row formats ([ZH] "K3.1 Pro 中的稀疏注意力" and "量化：原生 MXFP4 索引器"). */
#define DSA_KEY_FP8_E4M3_SCALED 0 /* 132 B: 128 OCP e4m3 codes, then a little-endian fp32 scale */
#define DSA_KEY_MXFP4 1           /* 68 B: 64 B of e2m1 pairs (element 2i in the low nibble),
                                     then 4 E8M0 scales (dims 0-31, 32-63, 64-95, 96-127) */
/* Latent row formats ([EN] "Sparse attention targets long-context costs"; [RECIPE] "NVFP4 KV cache"). */
#define DSA_LAT_FP8_E4M3 0 /* 576 B: 576 e4m3 codes; value = code * kv_scale */
#define DSA_LAT_NVFP4 1    /* 352 B: 256 B e2m1 pairs for dims 0-511, 32 e4m3 block scales
                              (one per 16 dims), 64 e4m3 rope dims 512-575;
                              value = code * block_scale * kv_scale (rope: code * kv_scale) */
/* Query formats. */
#define DSA_Q_BF16 0     /* bf16 values */
#define DSA_Q_FP8_E4M3 1 /* e4m3 codes plus one fp32 scale per (row, head): value = code * scale */
#define DSA_Q_MXFP4 2    /* 68 B per (row, head) in the MXFP4 key format: 64 B of e2m1 pairs
                            (element 2i in the low nibble), then four E8M0 scales, one per
                            32 elements; value = code * 2^(scale - 127) */

/* Block-packed cache layout ([ZH] "面向三种状态的 KV 缓存", figure 3): one
 * contiguous row per cache block holds, for each DSA layer in turn, the
 * layer's latent page (page_size latents) then its key page (page_size keys);
 * each layer slot is rounded up to 256 B and opaque per-block extra state
 * (e.g. recurrent state) follows the last layer:
 *   lat_page(row, layer) = row*row_stride + layer*layer_stride
 *   key_page(row, layer) = lat_page(row, layer) + lat_page_bytes
 *   token slot s of a page: + s*lat_bytes (latent) / + s*key_bytes (key)   */
typedef struct dsa_layout {
  int32_t page_size; /* tokens per page (64 in this library) */
  int32_t n_layers;
  int32_t key_fmt; /* DSA_KEY_* */
  int32_t lat_fmt; /* DSA_LAT_* */
  int32_t key_bytes;
  int32_t lat_bytes;
  int64_t lat_page_bytes;
  int64_t key_page_bytes;
  int64_t layer_stride;
  int64_t extra_row_bytes;
  int64_t row_stride;
} dsa_layout;

/* Static, NUL-terminated text for a status code / the library version. */
const char *dsa_status_str(dsa_status s);
const char *dsa_version(void);

/* Fill *out (host) for the given page size, layer count, formats and extra
 * per-row bytes.  Host only.  DSA_ERR_BAD_SHAPE for a non-positive page size
 * or layer count or negative extra bytes; DSA_ERR_UNSUPPORTED for an unknown
 * format. */
dsa_status dsa_layout_make(int32_t page_size, int32_t n_layers, int32_t key_fmt, int32_t lat_fmt,
                           int64_t extra_row_bytes, dsa_layout *out);

/* Page resolve ([ZH] "面向三种状态的 KV 缓存": before each step, block tables
 * and cache slots become the kernels' page addresses, so the kernels read the
 * packed cache unmodified).  Integer only.
 *   block_table  device int32 [n_req][bt_ld]   pool row of each logical page
 *   n_pages      device int32 [n_req]          pages in use per request
 *   lat_off, key_off  device int64 [n_req][off_ld]  (out) byte offsets from the
 *                pool base of layer `layer`'s latent / key page; for pages
 *                p < max_pages: p >= n_pages[b] or a bad block id gives -1
 *                (the latter also sets DSA_DEVERR_BLOCK_RANGE); columns
 *                >= max_pages are not written.
 * Requires max_pages <= bt_ld and max_pages <= off_ld, 0 <= layer < n_layers. */
dsa_status dsa_resolve_pages(const dsa_layout *layout, int32_t layer, const int32_t *block_table, int64_t bt_ld,
                             const int32_t *n_pages, int32_t n_req, int32_t max_pages, int64_t pool_rows,
                             int64_t *lat_off, int64_t *key_off, int64_t off_ld, int32_t *err_flag,
                             dsa_stream_t stream);

/* Indexer score ([ZH] "K3.1 Pro 中的稀疏注意力": one 132-byte FP8 key per token,
 * 32 light heads score every earlier token for each query; MXFP4 keys per
 * "量化：原生 MXFP4 索引器").  For query row r, request b = q_req[r], and every
 * token t < row_len[r] of request b:
 *     score[r][t] = sum_{j<32} w[r][j] * max(0, (q[r][j] . k_t) * scale_t)
 * with k_t the decoded key (MXFP4: E8M0 block scales included, scale_t = 1);
 * fp32 result, fp32 accumulation.  Decode: one row per request, row_len =
 * context length.  Prefill: row_len = position + 1 (causal).
 *   pool       device uint8, pool_bytes long, 16-B aligned
 *   key_off    device int64 [n_req][off_ld] from dsa_resolve_pages
 *   q          device [n_q][32][128]: bf16 (q_fmt DSA_Q_BF16) or e4m3 codes
 *              (DSA_Q_FP8_E4M3, with q_scale device fp32 [n_q][32]; else NULL),
 *              or device [n_q][32][68] bytes (DSA_Q_MXFP4, MXFP4 keys only)
 *   w          device fp32 [n_q][32]
 *   q_req, row_len  device int32 [n_q]
 *   scores     device fp32 [n_q][ld] (out): entries t < row_len[r] written,
 *              the rest untouched.
 *   workspace  device, >= dsa_indexer_score_workspace_size(n_q, q_fmt) bytes,
 *              256-B aligned (0 bytes, may be NULL, for bf16 queries)
 * The BF16 and MXFP4 paths stream each row's keys (decode); MXFP4 queries on
 * MXFP4 keys score on native FP4 MFMA with the E8M0 block scales of both
 * ([ZH] "量化：原生 MXFP4 索引器"; the query is quantised upstream, as in
 * "低延迟解码：融合的 DSA 解码路径"), so the result is the formula above for
 * the decoded MXFP4 query.  The FP8 path is an MFMA
 * GEMM over tiles of consecutive rows and is fastest when consecutive rows
 * share a request (a prefill chunk).  Both accept any q_req.  The FP8 path
 * first writes the rows' sign-folded bf16 query heads and head weights into
 * the workspace (about 8.2 KB per row). */
dsa_status dsa_indexer_score_workspace_size(int32_t n_q, int32_t q_fmt, size_t *bytes);

/* Prefill indexer and its exact top-k, scored on FP8 MFMA ([ZH] "低延迟解码：融合的 DSA
 * 解码路径": the indexer query is FP8 with its scale folded into the head weights;
 * "预填充：上下文并行稀疏注意力": each row keeps its top-k over the whole context).
 * The same problem as dsa_indexer_score (q_fmt DSA_Q_FP8_E4M3, FP8 keys) followed by dsa_topk,
 * with the same result: idx equals, bit for bit, what dsa_topk returns on dsa_indexer_score's
 * FP8 scores.  Both operands go to the FP8 MFMA as raw e4m3 codes; every product is exact, but
 * within each group of 8 consecutive dims the MFMA cuts the smaller products to 14 bits below
 * the group's largest, so the scores it writes are approximations s^ with
 *     |s^ - s| <= E_r = delta * sum_g U_rg * M_bg,   delta = 5.5 * 2^-13,
 * s the dsa_indexer_score value, g over the 16 groups of 8 dims,
 * U_rg = sum_j w[r][j] |q_scale[r][j]| max_{d in g} |q[r][j][d]| (code values) and
 * M_bg = max |scale_t| max_{d in g} |k_t[d]| over the request's first ctx_len[b] tokens.  The
 * top-k then finds the k-th largest s^, rescores exactly every token within 2 E_r of it (the
 * bf16 MFMA arithmetic of dsa_indexer_score), and selects from those and the tokens surely
 * above.
 *   pool, key_off, off_ld, n_req  as dsa_indexer_score (FP8 keys)
 *   ctx_len    device int32 [n_req]: tokens of each request; rows need row_len[r] <= ctx_len[q_req[r]]
 *   q          device e4m3 [n_q][32][128], 16-B aligned; q_scale, w device fp32 [n_q][32]
 *   q_req, row_len  device int32 [n_q] (prefill: row_len = position + 1)
 *   scores     device fp32 [n_q][ld] (out), 16-B aligned: s^ for t < row_len[r] (a row whose
 *              band holds more than 4096 tokens is rewritten with the exact s)
 *   idx        device int32 [n_q][idx_ld] (out): as dsa_topk, idx_ld >= k
 *   bound      device fp32 [n_q] (out, may be NULL): E_r
 *   workspace  device, >= dsa_prefill_select_workspace_size(...) bytes, 256-B aligned
 * 1 <= k <= 4096, ld <= 2^23, n_q and n_req <= 65535.  Errors as dsa_indexer_score and
 * dsa_topk; a row_len past ctx_len of its request is clamped and flags DSA_DEVERR_ROW_LEN.
 * DSA_DEVERR_BOUND would mean a score fell outside E_r (the bound rests on the measured
 * behaviour of the instruction; this flag reports a violation instead of a silent error). */
dsa_status dsa_prefill_select_workspace_size(int32_t n_q, int64_t ld, int32_t n_req, int64_t off_ld, int32_t k,
                                             size_t *bytes);
dsa_status dsa_prefill_select(const dsa_layout *layout, const uint8_t *pool, int64_t pool_bytes,
                              const int64_t *key_off, int64_t off_ld, int32_t n_req, const int32_t *ctx_len,
                              const uint8_t *q, const float *q_scale, const float *w, const int32_t *q_req,
                              const int32_t *row_len, int32_t n_q, int32_t k, float *scores, int64_t ld,
                              int32_t *idx, int64_t idx_ld, float *bound, void *workspace, size_t workspace_bytes,
                              int32_t *err_flag, dsa_stream_t stream);

/* The two halves of dsa_prefill_select, for callers that time or overlap them: the FP8 MFMA
 * scores (plus E_r and, in the workspace, the exact query rows the rescoring reads and, when
 * ld <= 2^18 and 64*off_ld >= ld, each long row's candidates at or above a threshold drawn from
 * 16 sampled 256-token tiles per 32 rows, written by the GEMM itself), then the band top-k.
 * Called in this order on the same workspace and arguments (the same k), they enqueue exactly
 * what dsa_prefill_select does; dsa_prefill_topk_band reads only what the score half left. */
dsa_status dsa_prefill_score_fp8(const dsa_layout *layout, const uint8_t *pool, int64_t pool_bytes,
                                 const int64_t *key_off, int64_t off_ld, int32_t n_req, const int32_t *ctx_len,
                                 const uint8_t *q, const float *q_scale, const float *w, const int32_t *q_req,
                                 const int32_t *row_len, int32_t n_q, int32_t k, float *scores, int64_t ld,
                                 float *bound, void *workspace, size_t workspace_bytes, int32_t *err_flag,
                                 dsa_stream_t stream);
/* dsa_prefill_score_fp8 in its two parts, same arguments, called in this order: the pre-pass,
 * the key bound and (candidate-list mode) the sampled tiles and thresholds; then the full
 * GEMM.  Together they enqueue exactly what dsa_prefill_score_fp8 does. */
dsa_status dsa_prefill_prepare_fp8(const dsa_layout *layout, const uint8_t *pool, int64_t pool_bytes,
                                   const int64_t *key_off, int64_t off_ld, int32_t n_req, const int32_t *ctx_len,
                                   const uint8_t *q, const float *q_scale, const float *w, const int32_t *q_req,
                                   const int32_t *row_len, int32_t n_q, int32_t k, float *scores, int64_t ld,
                                   float *bound, void *workspace, size_t workspace_bytes, int32_t *err_flag,
                                   dsa_stream_t stream);
dsa_status dsa_prefill_gemm_fp8(const dsa_layout *layout, const uint8_t *pool, int64_t pool_bytes,
                                const int64_t *key_off, int64_t off_ld, int32_t n_req, const int32_t *ctx_len,
                                const uint8_t *q, const float *q_scale, const float *w, const int32_t *q_req,
                                const int32_t *row_len, int32_t n_q, int32_t k, float *scores, int64_t ld,
                                float *bound, void *workspace, size_t workspace_bytes, int32_t *err_flag,
                                dsa_stream_t stream);
dsa_status dsa_prefill_topk_band(const dsa_layout *layout, const uint8_t *pool, int64_t pool_bytes,
                                 const int64_t *key_off, int64_t off_ld, int32_t n_req, const int32_t *q_req,
                                 const int32_t *row_len, int32_t n_q, int32_t k, float *scores, int64_t ld,
                                 int32_t *idx, int64_t idx_ld, void *workspace, size_t workspace_bytes,
                                 int32_t *err_flag, dsa_stream_t stream);
dsa_status dsa_indexer_score(const dsa_layout *layout, const uint8_t *pool, int64_t pool_bytes,
                             const int64_t *key_off, int64_t off_ld, int32_t n_req, const void *q, int32_t q_fmt,
                             const float *q_scale, const float *w, const int32_t *q_req, const int32_t *row_len,
                             int32_t n_q, float *scores, int64_t ld, void *workspace, size_t workspace_bytes,
                             int32_t *err_flag, dsa_stream_t stream);

/* Indexer score for speculative verification ([ZH] "量化：原生 MXFP4 索引器": while
 * draft tokens are verified, the keys are reused across the query rows instead of
 * being read again for each; "低延迟解码：融合的 DSA 解码路径": DSpark verifies 7
 * draft tokens, 8 rows per request).  Request b owns the rows_per_req consecutive
 * query rows r = b*rows_per_req + i; each row gets exactly the dsa_indexer_score
 * (bf16 query) result for q_req[r] = r / rows_per_req, bit for bit, but every
 * key page is read once for all rows of its request.  Row r scores tokens
 * t < row_len[r] (for causal verification of m rows at context L:
 * row_len = L - m + 1 + i).
 *   pool       device uint8, pool_bytes long, 16-B aligned
 *   key_off    device int64 [n_req][off_ld] from dsa_resolve_pages
 *   q          device bf16 [n_req*rows_per_req][32][128], 16-B aligned
 *   w          device fp32 [n_req*rows_per_req][32]
 *   row_len    device int32 [n_req*rows_per_req]
 *   scores     device fp32 [n_req*rows_per_req][ld] (out): entries t < row_len[r]
 *              written, the rest untouched.
 * rows_per_req < 1, n_req < 0, ld < 0 or off_ld < 1: DSA_ERR_BAD_SHAPE; rows_per_req
 * > 8 or n_req > 1024: DSA_ERR_UNSUPPORTED.  A row_len outside [0, min(ld, 64*off_ld)]
 * is clamped and flags DSA_DEVERR_ROW_LEN; a page a row needs whose offset is negative,
 * misaligned or past the pool is skipped (its scores are not written) and flags
 * DSA_DEVERR_PAGE_OFFSET. */
dsa_status dsa_indexer_score_verify(const dsa_layout *layout, const uint8_t *pool, int64_t pool_bytes,
                                    const int64_t *key_off, int64_t off_ld, int32_t n_req, int32_t rows_per_req,
                                    const uint16_t *q, const float *w, const int32_t *row_len, float *scores,
                                    int64_t ld, int32_t *err_flag, dsa_stream_t stream);

/* Top-k ([ZH] "K3.1 Pro 中的稀疏注意力": the top 2048 are kept; an exact top-k
 * per "低延迟解码：融合的 DSA 解码路径").  For each row r, the min(k, row_len[r])
 * tokens with the largest scores[r][t]; a tie goes to the lower token index
 * (one consistent tie-break, cf. "通信：高效的跨 GPU 通信"), -0 equals +0.
 * Output idx[r][0..k): the kept token indices in ascending order, then -1.
 * The result depends only on the row's own scores (batch-invariant, cf.
 * "day 0 零失配 RL") and is bitwise deterministic.
 *   scores  device fp32 [n_rows][ld]; row_len device int32 [n_rows]
 *   idx     device int32 [n_rows][idx_ld] (out), idx_ld >= k
 *   workspace  device, >= dsa_topk_workspace_size(n_rows, ld, k) bytes, 16-B aligned
 * 1 <= k <= 4096. */
dsa_status dsa_topk_workspace_size(int32_t n_rows, int64_t ld, int32_t k, size_t *bytes);
dsa_status dsa_topk(const float *scores, int64_t ld, const int32_t *row_len, int32_t n_rows, int32_t k, int32_t *idx,
                    int64_t idx_ld, void *workspace, size_t workspace_bytes, int32_t *err_flag, dsa_stream_t stream);

/* Sparse MLA decode ([ZH] "K3.1 Pro 中的稀疏注意力": every query head attends
 * exactly to the kept tokens' latents; partial results merged by
 * log-sum-exp as in "长上下文：带稀疏 indexer 的 decode 上下文并行").
 * For request b, head h and the non-negative entries t of idx[b] (each
 * entry one term; -1 entries are skipped):
 *     z_t = sm_scale * (q[b][h] . kv_t)                 kv_t includes kv_scale
 *     lse[b][h] = ln sum_t exp(z_t)
 *     out[b][h][c] = sum_t exp(z_t - lse) * kv_t[c]     c < 512 (values = first 512 dims)
 * An empty set writes out = 0, lse = -inf.  Entries >= ctx_len[b] are
 * skipped and flag DSA_DEVERR_INDEX.
 *   pool, lat_off (device, from dsa_resolve_pages), ctx_len device int32 [n_req]
 *   idx   device int32 [n_req][idx_ld] (logical token ids)
 *   q     device bf16 [n_req][n_heads][576]
 *   out   device bf16 [n_req][n_heads][512] (out); lse device fp32 [n_req][n_heads] (out)
 *   workspace  device, >= dsa_sparse_mla_decode_workspace_size(...) bytes
 * 1 <= n_heads <= 128. */
dsa_status dsa_sparse_mla_decode_workspace_size(int32_t n_req, int32_t n_heads, int32_t k, size_t *bytes);
dsa_status dsa_sparse_mla_decode(const dsa_layout *layout, const uint8_t *pool, int64_t pool_bytes,
                                 const int64_t *lat_off, int64_t off_ld, const int32_t *ctx_len, const int32_t *idx,
                                 int64_t idx_ld, int32_t k, const uint16_t *q, int32_t n_req, int32_t n_heads,
                                 float sm_scale, float kv_scale, uint16_t *out, float *lse, void *workspace,
                                 size_t workspace_bytes, int32_t *err_flag, dsa_stream_t stream);

/* Sparse MLA prefill ([ZH] "预填充：上下文并行稀疏注意力": each query row of a
 * prefill chunk attends over its own selected tokens, all local heads at
 * once).  Same definition as the decode call, per query row r with request
 * b = q_req[r] and set idx[r]; q is bf16 or e4m3 codes with q_scale device
 * fp32 [n_q][n_heads] (value = code * scale).
 *   q    device [n_q][n_heads][576];  q_req device int32 [n_q]
 *   out  device bf16 [n_q][n_heads][512] (out); lse device fp32 [n_q][n_heads] (out) */
dsa_status dsa_sparse_mla_prefill_workspace_size(int32_t n_q, int32_t n_heads, int32_t k, size_t *bytes);
dsa_status dsa_sparse_mla_prefill(const dsa_layout *layout, const uint8_t *pool, int64_t pool_bytes,
                                  const int64_t *lat_off, int64_t off_ld, int32_t n_req, const int32_t *ctx_len,
                                  const int32_t *idx, int64_t idx_ld, int32_t k, const void *q, int32_t q_fmt,
                                  const float *q_scale, const int32_t *q_req, int32_t n_q, int32_t n_heads,
                                  float sm_scale, float kv_scale, uint16_t *out, float *lse, void *workspace,
                                  size_t workspace_bytes, int32_t *err_flag, dsa_stream_t stream);

/* Fused indexer for decode: score -> exact top-k -> physical rows
 * ([ZH] "低延迟解码：融合的 DSA 解码路径": the fused indexer is a key-balanced
 * scorer and an exact top-k selection, and it outputs the physical KV rows
 * attention reads; "面向三种状态的 KV 缓存": the pages are found through the
 * block table).  For each row r (request b = q_req[r]):
 *   scores[r][t] for t < row_len[r] exactly as dsa_indexer_score with the same
 *   q_fmt (same kernel, bit for bit), with each key page read through the
 *   block table (pool row * row_stride + layer * layer_stride + the latent
 *   page's bytes) instead of resolved offsets;
 *   idx[r][0..k)  exactly the dsa_topk result on those scores: the
 *   min(k, row_len[r]) best tokens (lower index wins ties, -0 = +0),
 *   ascending, then -1;
 *   phys[r][i]    (optional, may be NULL) the physical row of idx[r][i]:
 *   block_table[b][t / 64] * 64 + t % 64, or -1 (padding; also for a block
 *   id outside [0, pool_rows), which flags DSA_DEVERR_BLOCK_RANGE), with
 *   pool_rows = pool_bytes / row_stride.
 * Launches on `stream`: the scan, then dsa_topk's kernels, whose last one
 * looks up each kept token's block as it writes it.  No page-offset table and
 * no separate resolve launch.
 *   pool         device uint8, pool_bytes long, 16-B aligned
 *   block_table  device int32 [n_req][bt_ld]; row_len[r] <= 64 * bt_ld (else
 *                DSA_DEVERR_ROW_LEN and the row is cut there)
 *   q, q_fmt     DSA_Q_BF16: device bf16 [n_q][32][128]; DSA_Q_MXFP4 (MXFP4
 *                keys only): device [n_q][32][68] bytes; 16-B aligned
 *   w            device fp32 [n_q][32]
 *   q_req, row_len  device int32 [n_q]
 *   scores       device fp32 [n_q][ld] (out)
 *   idx, phys    device int32 [n_q][idx_ld] (out), idx_ld >= k
 *   workspace    device, >= dsa_indexer_select_workspace_size(n_q, ld) bytes
 *                (the same as dsa_topk's), 16-B aligned
 * 1 <= k <= 4096, n_q <= 4096, ld <= 2^23 (else DSA_ERR_UNSUPPORTED); with
 * phys, pool_rows * 64 must fit int32. */
dsa_status dsa_indexer_select_workspace_size(int32_t n_q, int64_t ld, size_t *bytes);
dsa_status dsa_indexer_select(const dsa_layout *layout, int32_t layer, const uint8_t *pool, int64_t pool_bytes,
                              const int32_t *block_table, int64_t bt_ld, int32_t n_req, const void *q, int32_t q_fmt,
                              const float *w, const int32_t *q_req, const int32_t *row_len, int32_t n_q, int32_t k,
                              float *scores, int64_t ld, int32_t *idx, int32_t *phys, int64_t idx_ld,
                              void *workspace, size_t workspace_bytes, int32_t *err_flag, dsa_stream_t stream);
/* The two halves of dsa_indexer_select, for callers that time or reuse them
 * (arguments as there): dsa_indexer_score_pages is the scan alone (no
 * workspace); dsa_topk_pages is dsa_topk with the physical-row output. */
dsa_status dsa_indexer_score_pages(const dsa_layout *layout, int32_t layer, const uint8_t *pool, int64_t pool_bytes,
                                   const int32_t *block_table, int64_t bt_ld, int32_t n_req, const void *q,
                                   int32_t q_fmt, const float *w, const int32_t *q_req, const int32_t *row_len, int32_t n_q,
                                   float *scores, int64_t ld, int32_t *err_flag, dsa_stream_t stream);
dsa_status dsa_topk_pages(const dsa_layout *layout, int64_t pool_bytes, const int32_t *block_table, int64_t bt_ld,
                          int32_t n_req, const int32_t *q_req, const float *scores, int64_t ld,
                          const int32_t *row_len, int32_t n_q, int32_t k, void *workspace, size_t workspace_bytes,
                          int32_t *idx, int32_t *phys, int64_t idx_ld, int32_t *err_flag, dsa_stream_t stream);

/* Sparse MLA decode over physical rows ([ZH] "低延迟解码：融合的 DSA 解码路径":
 * attention reads the physical KV rows the fused indexer emits).  The result
 * of dsa_sparse_mla_decode (same kernel and split order, bit for bit) for the
 * set whose entries are phys[b][i] = pool_row * 64 + slot; the latent of an
 * entry is at pool_row * row_stride + layer * layer_stride + slot * lat_bytes.
 * -1 entries are skipped; a pool row outside [0, pool_bytes / row_stride)
 * flags DSA_DEVERR_BLOCK_RANGE and is skipped.
 *   phys  device int32 [n_req][idx_ld];  q device bf16 [n_req][n_heads][576]
 *   out   device bf16 [n_req][n_heads][512] (out); lse device fp32 [n_req][n_heads] (out)
 *   workspace  device, >= dsa_sparse_mla_decode_workspace_size(n_req, n_heads, k) bytes
 * 1 <= n_heads <= 128. */
dsa_status dsa_sparse_mla_decode_phys(const dsa_layout *layout, int32_t layer, const uint8_t *pool, int64_t pool_bytes,
                                      const int32_t *phys, int64_t idx_ld, int32_t k, const uint16_t *q,
                                      int32_t n_req, int32_t n_heads, float sm_scale, float kv_scale, uint16_t *out,
                                      float *lse, void *workspace, size_t workspace_bytes, int32_t *err_flag,
                                      dsa_stream_t stream);

/* Sparse MLA decode that allocates nothing and takes no workspace: for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  Same arguments and result
 * as dsa_sparse_mla_decode, bit for bit (the same kernels), minus the
 * workspace.  The split partials go to a static device array of
 * DSA_NOALLOC_SCRATCH_BYTES per GPU, held until the process ends; a call whose
 * partials would not fit (dsa_sparse_mla_decode_workspace_size answers more)
 * returns DSA_ERR_SCRATCH_LIMIT and enqueues nothing (32 MiB covers 64 requests
 * x 12 heads x k = 2048).  Every call on a GPU shares that GPU's array:
 * calls that overlap on one GPU (other streams, other threads) race and must
 * be serialised by the caller.  The array's device address is looked up with
 * hipGetSymbolAddress on a device's first call (DSA_ERR_HIP if that fails). */
#define DSA_NOALLOC_SCRATCH_BYTES (32 * 1024 * 1024)
dsa_status dsa_sparse_mla_decode_noalloc(const dsa_layout *layout, const uint8_t *pool, int64_t pool_bytes,
                                         const int64_t *lat_off, int64_t off_ld, const int32_t *ctx_len,
                                         const int32_t *idx, int64_t idx_ld, int32_t k, const uint16_t *q,
                                         int32_t n_req, int32_t n_heads, float sm_scale, float kv_scale,
                                         uint16_t *out, float *lse, int32_t *err_flag, dsa_stream_t stream);

/* Exact top-k merge across decode-context-parallel shards, emulated on one GPU
 * ([ZH] "长上下文：带稀疏 indexer 的 decode 上下文并行": shard s of W holds every
 * W-th token, t mod W = s; "流量减少 10× 的精确 top-k 合并": each shard sends
 * its best ceil(1.5 k / W) candidates taken from BF16 scores, each packed with
 * its score into 32 bits; the same radix select over the gathered candidates
 * gives the global top-k; a shard that may hold more of it than it sent
 * resends its full local top-k for the row).
 * Output idx[r][0..k): the min(k, row_len[r]) tokens first in the order
 * (BF16 of the score, round to nearest even, descending; token index
 * ascending), in ascending token order, then -1.  resend_mask[r] (optional,
 * device uint32): bit s set when shard s resent for row r, which is when
 * shard s holds more than c = ceil(1.5 k / W) of the row's tokens and its
 * c-th (last sent) candidate is among the min(k, row_len[r]) best of all
 * shards' candidates; that is the test a shard can make from the gathered
 * candidates alone, and it never misses a shard holding unsent top-k tokens
 * (it may flag shards that hold none).  Four
 * launches (candidates, merge, resend, merge of resent rows), all on `stream`.
 *   scores  device fp32 [n_rows][ld]; row_len device int32 [n_rows]
 *   idx     device int32 [n_rows][idx_ld] (out), idx_ld >= k
 *   workspace  device, >= dsa_dcp_topk_workspace_size(n_rows, k, n_shards)
 *              bytes, 16-B aligned
 * 1 <= n_shards <= 8, 1 <= k <= 2048, ld <= 65536 * n_shards (each shard's
 * local token index fits the 16 bits of a packed candidate), else
 * DSA_ERR_UNSUPPORTED. */
dsa_status dsa_dcp_topk_workspace_size(int32_t n_rows, int32_t k, int32_t n_shards, size_t *bytes);
dsa_status dsa_dcp_topk(const float *scores, int64_t ld, const int32_t *row_len, int32_t n_rows, int32_t k,
                        int32_t n_shards, int32_t *idx, int64_t idx_ld, uint32_t *resend_mask, void *workspace,
                        size_t workspace_bytes, int32_t *err_flag, dsa_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* DSA_H */
