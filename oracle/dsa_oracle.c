/*
 * dsa_oracle.c -- CPU oracle for the DeepSeek-style sparse attention (DSA) step.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load or call this library.  The product
 * path (libdsa.so and its Python binding) never does, and shares no code,
 * header, table or constant generator with it.
 *
 * Plain, slow and meant to be checked by eye: every quantity is computed in
 * double precision straight from its definition; the only concession to
 * speed is OpenMP over independent output rows, which changes no arithmetic.
 *
 * Pages cited (by title and section):
 *   [ZH]     "vLLM 为 Kimi K3.1 Pro 提供 Day-0 支持"
 *   [EN]     "vLLM Adds Day-0 Support for Moonshot AI's Kimi K3.1 Pro"
 *   [RECIPE] "moonshotai/Kimi-K3.1-Pro" (vLLM recipe page)
 *
 * What the step computes ([ZH] section "K3.1 Pro 中的稀疏注意力", figure 1):
 *   1. a small indexer scores every earlier token of the request against the
 *      query, from one 132-byte FP8 key per token and 32 light heads;
 *   2. the 2048 best-scoring tokens are kept;
 *   3. MLA attention then runs exactly, over only those tokens' latents.
 * The indexer score is not printed on the pages; this oracle uses the
 * DeepSeek-V3.2 lightning-indexer form that the section points to:
 *   score(t) = sum_j w_j * ReLU(q_j . k_t * scale_t).
 *
 * Status codes: 0 ok, 1 bad argument, 2 out-of-range block/token,
 * 3 non-finite value where the definition needs a finite one.
 */
#define _GNU_SOURCE
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_OK 0
#define OR_ERR_ARG 1
#define OR_ERR_RANGE 2
#define OR_ERR_NONFINITE 3

/* ------------------------------------------------------------------------ */
/* Number formats (public specifications, decoded from their definitions)   */
/* ------------------------------------------------------------------------ */

/* OCP OFP8 E4M3 ("E4M3FN"): sign, 4 exponent bits (bias 7), 3 mantissa bits.
 * Normal: (1 + m/8) * 2^(e-7).  Subnormal (e = 0): (m/8) * 2^-6.
 * S.1111.111 is NaN; there are no infinities; the largest finite is 448. */
double or_e4m3(unsigned code) {
  unsigned s = (code >> 7) & 1u, e = (code >> 3) & 15u, m = code & 7u;
  double v;
  if (e == 15u && m == 7u) return NAN;
  if (e == 0u)
    v = ldexp((double)m / 8.0, -6);
  else
    v = ldexp(1.0 + (double)m / 8.0, (int)e - 7);
  return s ? -v : v;
}

/* OCP MX FP4 E2M1 element: sign, 2 exponent bits (bias 1), 1 mantissa bit.
 * Normal: (1 + m/2) * 2^(e-1); subnormal (e = 0): m * 0.5. */
double or_e2m1(unsigned nib) {
  unsigned s = (nib >> 3) & 1u, e = (nib >> 1) & 3u, m = nib & 1u;
  double v = (e == 0u) ? 0.5 * (double)m : ldexp(1.0 + 0.5 * (double)m, (int)e - 1);
  return s ? -v : v;
}

/* OCP MX E8M0 shared scale: 2^(e-127); 0xFF is NaN. */
double or_e8m0(unsigned code) {
  if ((code & 0xFFu) == 0xFFu) return NAN;
  return ldexp(1.0, (int)(code & 0xFFu) - 127);
}

/* bfloat16: the upper 16 bits of an IEEE binary32. */
double or_bf16(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

static double f32_le(const uint8_t *p) {
  uint32_t u = (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* ------------------------------------------------------------------------ */
/* Block-packed cache layout                                                */
/* ------------------------------------------------------------------------ */
/* [ZH] section "面向三种状态的 KV 缓存": the cache is packed by block, not by
 * layer; one block is one contiguous row that holds, for every DSA layer, a
 * latent page (576 B/token FP8, 352 B NVFP4) and an index-key page (132 B/token
 * FP8, 68 B MXFP4), plus the recurrent state.  Pages inside a row may differ in
 * size; kernels still see small fixed-size pages.  Reading of the in-row
 * order taken here: per layer, latent page then key page, each layer slot
 * rounded up to 256 bytes, the opaque extra state after the last layer. */

typedef struct {
  int64_t page_size, n_layers, key_fmt, lat_fmt;
  int64_t key_bytes, lat_bytes, layer_stride, row_stride, extra_row_bytes;
} or_layout;

static int64_t round_up_256(int64_t x) { return (x + 255) / 256 * 256; }

int or_layout_make(int64_t page_size, int64_t n_layers, int64_t key_fmt, int64_t lat_fmt,
                   int64_t extra_row_bytes, or_layout *out) {
  if (!out || page_size <= 0 || n_layers <= 0 || extra_row_bytes < 0) return OR_ERR_ARG;
  if (key_fmt != 0 && key_fmt != 1) return OR_ERR_ARG;
  if (lat_fmt != 0 && lat_fmt != 1) return OR_ERR_ARG;
  out->page_size = page_size;
  out->n_layers = n_layers;
  out->key_fmt = key_fmt;
  out->lat_fmt = lat_fmt;
  /* FP8 key: 128 e4m3 + fp32 scale; MXFP4 key: 128 e2m1 (64 B) + 4 E8M0 ([ZH] "KV 缓存占用"). */
  out->key_bytes = key_fmt == 0 ? 128 + 4 : 64 + 4;
  /* FP8 latent: 576 e4m3; NVFP4 latent: 512 e2m1 (256 B) + 32 e4m3 block scales + 64 e4m3 rope. */
  out->lat_bytes = lat_fmt == 0 ? 576 : 256 + 32 + 64;
  out->layer_stride = round_up_256(page_size * out->lat_bytes + page_size * out->key_bytes);
  out->extra_row_bytes = extra_row_bytes;
  out->row_stride = round_up_256(n_layers * out->layer_stride + extra_row_bytes);
  return OR_OK;
}

/* Pool row holding token t of request b, found by walking the block table.
 * Returns OR_OK and sets *row, or OR_ERR_RANGE. */
static int token_row(const or_layout *L, const int32_t *bt, int64_t bt_ld, const int32_t *n_pages,
                     int64_t pool_rows, int64_t b, int64_t t, int64_t *row) {
  int64_t page = t / L->page_size;
  if (t < 0 || page >= n_pages[b] || page >= bt_ld) return OR_ERR_RANGE;
  int64_t r = bt[b * bt_ld + page];
  if (r < 0 || r >= pool_rows) return OR_ERR_RANGE;
  *row = r;
  return OR_OK;
}

static const uint8_t *key_row_ptr(const or_layout *L, const uint8_t *pool, int64_t layer, int64_t row,
                                  int64_t t) {
  return pool + row * L->row_stride + layer * L->layer_stride + L->page_size * L->lat_bytes +
         (t % L->page_size) * L->key_bytes;
}

static const uint8_t *lat_row_ptr(const or_layout *L, const uint8_t *pool, int64_t layer, int64_t row,
                                  int64_t t) {
  return pool + row * L->row_stride + layer * L->layer_stride + (t % L->page_size) * L->lat_bytes;
}

/* Page resolve: block table -> byte offsets of each (request, page)'s latent
 * and key pages in the pool ([ZH] "面向三种状态的 KV 缓存": block tables and
 * cache slots become kernel page addresses before each step).  Integer only.
 * Entries past n_pages[b] get -1; an out-of-range block id gets -1 and
 * makes the call return OR_ERR_RANGE. */
int or_resolve_pages(const or_layout *L, int64_t layer, const int32_t *bt, int64_t bt_ld,
                     const int32_t *n_pages, int64_t n_req, int64_t max_pages, int64_t pool_rows,
                     int64_t *lat_off, int64_t *key_off, int64_t off_ld) {
  int rc = OR_OK;
  if (!L || !bt || !n_pages || !lat_off || !key_off || layer < 0 || layer >= L->n_layers) return OR_ERR_ARG;
  for (int64_t b = 0; b < n_req; ++b) {
    for (int64_t p = 0; p < max_pages; ++p) {
      int64_t lo = -1, ko = -1;
      if (p < n_pages[b]) {
        int64_t r = bt[b * bt_ld + p];
        if (r >= 0 && r < pool_rows) {
          lo = r * L->row_stride + layer * L->layer_stride;
          ko = lo + L->page_size * L->lat_bytes;
        } else {
          rc = OR_ERR_RANGE;
        }
      }
      if (n_pages[b] > max_pages || n_pages[b] < 0) rc = OR_ERR_RANGE;
      lat_off[b * off_ld + p] = lo;
      key_off[b * off_ld + p] = ko;
    }
  }
  return rc;
}

/* One index key, decoded: k[0..127] and the per-token scale.
 * FP8 ([ZH] "K3.1 Pro 中的稀疏注意力": 132 bytes with its scale): 128 e4m3
 * codes then a little-endian fp32 scale.  MXFP4 ([ZH] "量化：原生 MXFP4 索引器":
 * 68 bytes with scales): 64 bytes of e2m1 pairs (element 2i in the low
 * nibble) then four E8M0 scales, one per 32 elements; its scale_t is 1. */
int or_key_decode(int64_t key_fmt, const uint8_t *row, double *k, double *scale) {
  if (key_fmt == 0) {
    for (int d = 0; d < 128; ++d) k[d] = or_e4m3(row[d]);
    *scale = f32_le(row + 128);
  } else if (key_fmt == 1) {
    for (int d = 0; d < 128; ++d) {
      unsigned byte = row[d / 2];
      unsigned nib = (d % 2 == 0) ? (byte & 15u) : (byte >> 4);
      k[d] = or_e2m1(nib) * or_e8m0(row[64 + d / 32]);
    }
    *scale = 1.0;
  } else {
    return OR_ERR_ARG;
  }
  return OR_OK;
}

/* One latent, decoded to 576 values including the per-tensor kv_scale.
 * FP8: 576 e4m3 codes ([EN] "Sparse attention targets long-context costs":
 * 576 bytes per token and layer).  NVFP4 ([RECIPE] "NVFP4 KV cache": 352
 * bytes): dims 0..511 are e2m1 (low nibble first) times the e4m3 scale of
 * their 16-element block; dims 512..575 (rope) are e4m3. */
int or_latent_decode(int64_t lat_fmt, const uint8_t *row, double kv_scale, double *kv) {
  if (lat_fmt == 0) {
    for (int d = 0; d < 576; ++d) kv[d] = or_e4m3(row[d]) * kv_scale;
  } else if (lat_fmt == 1) {
    for (int d = 0; d < 512; ++d) {
      unsigned byte = row[d / 2];
      unsigned nib = (d % 2 == 0) ? (byte & 15u) : (byte >> 4);
      kv[d] = or_e2m1(nib) * or_e4m3(row[256 + d / 16]) * kv_scale;
    }
    for (int d = 512; d < 576; ++d) kv[d] = or_e4m3(row[288 + (d - 512)]) * kv_scale;
  } else {
    return OR_ERR_ARG;
  }
  return OR_OK;
}

/* Query element (row r, head j, dim d): bf16, an e4m3 code times the fp32
 * scale of its (row, head), or (q_fmt 2, indexer queries only) element d of
 * a 68-byte MXFP4 row per (row, head) -- the MXFP4 key format ([ZH] "低延迟解码：融合的 DSA 解码路径": the indexer query
 * is quantised to FP8 or MXFP4 before scoring; "量化：原生 MXFP4 索引器"). */
static double q_elem(const void *q, int64_t q_fmt, const float *q_scale, int64_t heads, int64_t dim,
                     int64_t r, int64_t j, int64_t d) {
  int64_t i = (r * heads + j) * dim + d;
  if (q_fmt == 0) return or_bf16(((const uint16_t *)q)[i]);
  if (q_fmt == 2) {  /* the MXFP4 key row layout (see or_key_decode) */
    const uint8_t *row = (const uint8_t *)q + (r * heads + j) * 68;
    unsigned byte = row[d / 2];
    unsigned nib = (d % 2 == 0) ? (byte & 15u) : (byte >> 4);
    return or_e2m1(nib) * or_e8m0(row[64 + d / 32]);
  }
  return or_e4m3(((const uint8_t *)q)[i]) * (double)q_scale[r * heads + j];
}

/* ------------------------------------------------------------------------ */
/* Indexer score                                                            */
/* ------------------------------------------------------------------------ */
/* For query row r (request b = q_req[r]) and each token t < row_len[r]:
 *   x_j   = (sum_d q[r][j][d] * k_t[d]) * scale_t          j = 0..31
 *   score = sum_j w[r][j] * max(x_j, 0)
 * evaluated in double and rounded once to float.  A decode row scores the
 * whole context (row_len = context length, the new token included); a
 * prefill row at position p scores tokens 0..p (row_len = p + 1).
 * bytes_read[r] (optional) counts the key bytes read for row r. */
int or_indexer_score(const or_layout *L, int64_t layer, const uint8_t *pool, int64_t pool_rows,
                     const int32_t *bt, int64_t bt_ld, const int32_t *n_pages, int64_t n_req,
                     const void *q, int64_t q_fmt, const float *q_scale, const float *w,
                     const int32_t *q_req, const int32_t *row_len, int64_t n_q, float *scores, int64_t ld,
                     int64_t *bytes_read) {
  if (!L || !pool || !bt || !n_pages || !q || !w || !q_req || !row_len || !scores) return OR_ERR_ARG;
  if ((q_fmt == 1 && !q_scale) || q_fmt < 0 || q_fmt > 2) return OR_ERR_ARG;
  int rc = OR_OK;
  const int64_t BLK = 512;
  if (bytes_read)
    for (int64_t r = 0; r < n_q; ++r) bytes_read[r] = 0;
  int64_t nblk_max = (ld + BLK - 1) / BLK;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t task = 0; task < n_q * nblk_max; ++task) {
    int64_t r = task / nblk_max, t0 = (task % nblk_max) * BLK;
    int64_t len = row_len[r], b = q_req[r];
    if (t0 >= len) continue;
    if (len > ld || b < 0 || b >= n_req) {
#pragma omp atomic write
      rc = OR_ERR_ARG;
      continue;
    }
    double k[128], sc, qv[32][128];
    int64_t t1 = t0 + BLK < len ? t0 + BLK : len, counted = 0;
    for (int64_t j = 0; j < 32; ++j)
      for (int64_t d = 0; d < 128; ++d) qv[j][d] = q_elem(q, q_fmt, q_scale, 32, 128, r, j, d);
    for (int64_t t = t0; t < t1; ++t) {
      int64_t row;
      if (token_row(L, bt, bt_ld, n_pages, pool_rows, b, t, &row) != OR_OK) {
#pragma omp atomic write
        rc = OR_ERR_RANGE;
        continue;
      }
      or_key_decode(L->key_fmt, key_row_ptr(L, pool, layer, row, t), k, &sc);
      counted += L->key_bytes;
      double acc = 0.0;
      for (int64_t j = 0; j < 32; ++j) {
        double dot = 0.0;
        for (int64_t d = 0; d < 128; ++d) dot += qv[j][d] * k[d];
        double x = dot * sc;
        double relu = x > 0.0 ? x : 0.0;
        acc += (double)w[r * 32 + j] * relu;
      }
      if (!isfinite(acc)) {
#pragma omp atomic write
        rc = OR_ERR_NONFINITE;
      }
      scores[r * ld + t] = (float)acc;
    }
    if (bytes_read) {
#pragma omp atomic
      bytes_read[r] += counted;
    }
  }
  return rc;
}

/* ------------------------------------------------------------------------ */
/* Top-k                                                                    */
/* ------------------------------------------------------------------------ */
/* Keep the min(k, len) tokens with the largest scores ([ZH] "K3.1 Pro 中的
 * 稀疏注意力": the top 2048 are kept).  Order: score descending, then token
 * index ascending, so a tie goes to the lower index (one consistent
 * tie-break, cf. [ZH] "通信：高效的跨 GPU 通信").  The kept indices are
 * written in ascending token order and the rest of the k slots get -1.
 * Method: one full sort of the row, no blocking or early exit. */
static int cmp_score_desc_idx_asc(const void *a, const void *b, void *ctx) {
  const float *s = (const float *)ctx;
  int32_t ia = *(const int32_t *)a, ib = *(const int32_t *)b;
  float sa = s[ia], sb = s[ib];
  if (sa > sb) return -1;
  if (sa < sb) return 1;
  return (ia > ib) - (ia < ib);
}

static int cmp_int_asc(const void *a, const void *b) {
  int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
  return (x > y) - (x < y);
}

int or_topk(const float *scores, int64_t ld, const int32_t *row_len, int64_t n_rows, int64_t k, int32_t *idx,
            int64_t idx_ld) {
  if (!scores || !row_len || !idx || k < 0 || idx_ld < k) return OR_ERR_ARG;
  int rc = OR_OK;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < n_rows; ++r) {
    int64_t len = row_len[r];
    int32_t *out = idx + r * idx_ld;
    if (len < 0 || len > ld) {
#pragma omp atomic write
      rc = OR_ERR_ARG;
      continue;
    }
    const float *s = scores + r * ld;
    int bad = 0;
    for (int64_t t = 0; t < len; ++t)
      if (!isfinite(s[t])) bad = 1;
    if (bad) {
#pragma omp atomic write
      rc = OR_ERR_NONFINITE;
      continue;
    }
    int32_t *order = (int32_t *)malloc(sizeof(int32_t) * (size_t)(len > 0 ? len : 1));
    for (int64_t t = 0; t < len; ++t) order[t] = (int32_t)t;
    qsort_r(order, (size_t)len, sizeof(int32_t), cmp_score_desc_idx_asc, (void *)s);
    int64_t keep = k < len ? k : len;
    qsort(order, (size_t)keep, sizeof(int32_t), cmp_int_asc);
    for (int64_t i = 0; i < k; ++i) out[i] = i < keep ? order[i] : -1;
    free(order);
  }
  return rc;
}

/* ------------------------------------------------------------------------ */
/* Exact top-k merge across decode-context-parallel shards (one process)    */
/* ------------------------------------------------------------------------ */
/* [ZH] section "长上下文：带稀疏 indexer 的 decode 上下文并行": under decode
 * context parallelism shard r of W holds every W-th token (token t lives on
 * shard t mod W), and the global top-2048 must be merged across shards before
 * attention.  Section "流量减少 10× 的精确 top-k 合并": each shard picks its
 * best 1.5 * 2048 / W candidates straight from BF16 scores and packs each with
 * its score into 32 bits; every shard selects the same global top-2048 from the
 * gathered candidates; a shard that may hold more of the top-2048 than it sent
 * is detected and resends its full local top-k for that row.
 * Readings taken here:
 *   - the order is the BF16 value of the score (fp32 rounded to nearest, ties
 *     to even) descending, then token index ascending (the tie rule of or_topk);
 *   - c = ceil(1.5 k / W) candidates per shard; a shard holding at most c
 *     tokens sends them all;
 *   - detection uses only what the gathered candidates show: shard s is flagged
 *     when it holds more than c tokens and its c-th (last sent) candidate is
 *     among the min(k, len) first of the candidate union.  Otherwise every
 *     token it kept back ranks below that candidate, hence below the union's
 *     k-th, hence (the union being a subset of the row) below the true k-th;
 *   - a flagged shard resends its first min(k, held) tokens, and the output is
 *     the min(k, len) first of the second union, ascending, -1 padded.
 * The steps are carried out literally, each with a full sort. */
static double bf16_round(double x) {
  /* 8 significant bits, round to nearest, ties to even (normal range; the
   * BF16 subnormal range below 2^-126 keeps fewer bits and is not covered) */
  if (x == 0.0 || !isfinite(x)) return x;
  int e;
  double m = frexp(x, &e); /* |m| in [0.5, 1) */
  return ldexp(nearbyint(ldexp(m, 8)), e - 8);
}

double or_bf16_round(float x) { return bf16_round((double)x); }

static int cmp_dval_desc_idx_asc(const void *a, const void *b, void *ctx) {
  const double *v = (const double *)ctx;
  int32_t ia = *(const int32_t *)a, ib = *(const int32_t *)b;
  if (v[ia] > v[ib]) return -1;
  if (v[ia] < v[ib]) return 1;
  return (ia > ib) - (ia < ib);
}

/* The row's tokens on shard sh, first `take` of them in the order: the shard's
 * candidate list.  Appends to list[*n] and returns the number appended. */
static int64_t dcp_shard_list(const double *v, int64_t len, int64_t W, int64_t sh, int64_t take, int32_t *tmp,
                              int32_t *list, int64_t *n) {
  int64_t held = 0;
  for (int64_t t = sh; t < len; t += W) tmp[held++] = (int32_t)t;
  qsort_r(tmp, (size_t)held, sizeof(int32_t), cmp_dval_desc_idx_asc, (void *)v);
  const int64_t m = take < held ? take : held;
  for (int64_t i = 0; i < m; ++i) list[(*n)++] = tmp[i];
  return m;
}

int or_dcp_topk(const float *scores, int64_t ld, const int32_t *row_len, int64_t n_rows, int64_t k, int64_t n_shards,
                int32_t *idx, int64_t idx_ld, uint32_t *resend) {
  if (!scores || !row_len || !idx || !resend || k < 1 || idx_ld < k || n_shards < 1 || n_shards > 32)
    return OR_ERR_ARG;
  const int64_t W = n_shards;
  const int64_t c = (3 * k + 2 * W - 1) / (2 * W); /* ceil(1.5 k / W) */
  int rc = OR_OK;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < n_rows; ++r) {
    int64_t len = row_len[r];
    int32_t *out = idx + r * idx_ld;
    resend[r] = 0;
    if (len < 0 || len > ld) {
#pragma omp atomic write
      rc = OR_ERR_ARG;
      continue;
    }
    const float *s = scores + r * ld;
    const size_t cap = (size_t)(len > 0 ? len : 1);
    double *v = (double *)malloc(sizeof(double) * cap);
    int32_t *tmp = (int32_t *)malloc(sizeof(int32_t) * cap);
    int32_t *uni = (int32_t *)malloc(sizeof(int32_t) * cap);
    int32_t *last = (int32_t *)malloc(sizeof(int32_t) * (size_t)W); /* each shard's last sent token */
    int64_t *held = (int64_t *)malloc(sizeof(int64_t) * (size_t)W);
    char *kept = (char *)calloc(cap, 1);
    int bad = 0;
    for (int64_t t = 0; t < len; ++t) {
      if (!isfinite(s[t])) bad = 1;
      v[t] = bf16_round((double)s[t]);
    }
    if (bad) {
#pragma omp atomic write
      rc = OR_ERR_NONFINITE;
      len = 0;
    }
    const int64_t keep = k < len ? k : len;
    /* (1) every shard sends its first c tokens; the union is sorted in the order */
    int64_t n = 0;
    for (int64_t sh = 0; sh < W; ++sh) {
      held[sh] = sh < len ? (len - 1 - sh) / W + 1 : 0;
      const int64_t m = dcp_shard_list(v, len, W, sh, c, tmp, uni, &n);
      last[sh] = m > 0 ? uni[n - 1] : -1;
    }
    qsort_r(uni, (size_t)n, sizeof(int32_t), cmp_dval_desc_idx_asc, (void *)v);
    /* (2) flags: a shard that kept tokens back and whose last sent token is among
     * the union's keep first */
    for (int64_t p = 0; p < keep; ++p) kept[uni[p]] = 1;
    for (int64_t sh = 0; sh < W; ++sh)
      if (held[sh] > c && kept[last[sh]]) resend[r] |= 1u << sh;
    /* (3) the flagged shards resend their first k tokens; the second union decides */
    if (resend[r]) {
      n = 0;
      for (int64_t sh = 0; sh < W; ++sh)
        dcp_shard_list(v, len, W, sh, ((resend[r] >> sh) & 1u) ? k : c, tmp, uni, &n);
      qsort_r(uni, (size_t)n, sizeof(int32_t), cmp_dval_desc_idx_asc, (void *)v);
    }
    qsort(uni, (size_t)keep, sizeof(int32_t), cmp_int_asc);
    for (int64_t i = 0; i < k; ++i) out[i] = i < keep ? uni[i] : -1;
    free(v);
    free(tmp);
    free(uni);
    free(last);
    free(held);
    free(kept);
  }
  return rc;
}

/* ------------------------------------------------------------------------ */
/* Sparse MLA over a given index set                                        */
/* ------------------------------------------------------------------------ */
/* Exact attention of every query head over the listed tokens' latents
 * ([ZH] "K3.1 Pro 中的稀疏注意力", figure 1: each query head attends exactly
 * to the kept tokens' latents).  Keys are all 576 latent dims, values the
 * first 512 (the no-rope part).  For row r, head h and the set I of
 * non-negative entries of idx[r] (each entry one term):
 *   z_t = sm_scale * sum_{d<576} q[r][h][d] * kv_t[d]        (kv includes kv_scale)
 *   lse = log(sum_t exp(z_t))          natural log, computed as m + log(sum exp(z-m))
 *   o[c] = sum_t exp(z_t - lse) * kv_t[c]                     c < 512
 * An empty set gives o = 0 and lse = -inf.  Entries >= the request's
 * context length make the call fail with OR_ERR_RANGE.
 * out is [n_q][H][512] double, lse [n_q][H] double. */
int or_sparse_mla(const or_layout *L, int64_t layer, const uint8_t *pool, int64_t pool_rows,
                  const int32_t *bt, int64_t bt_ld, const int32_t *n_pages, const int32_t *ctx_len,
                  int64_t n_req, const int32_t *idx, int64_t idx_ld, int64_t k, const void *q, int64_t q_fmt,
                  const float *q_scale, const int32_t *q_req, int64_t n_q, int64_t H, double sm_scale,
                  double kv_scale, double *out, double *lse, int64_t *bytes_read) {
  if (!L || !pool || !bt || !n_pages || !ctx_len || !idx || !q || !q_req || !out || !lse) return OR_ERR_ARG;
  if ((q_fmt == 1 && !q_scale) || q_fmt < 0 || q_fmt > 1) return OR_ERR_ARG;
  int rc = OR_OK;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < n_q; ++r) {
    int64_t b = q_req[r];
    if (b < 0 || b >= n_req) {
#pragma omp atomic write
      rc = OR_ERR_ARG;
      continue;
    }
    double *kv = (double *)malloc(sizeof(double) * 576 * (size_t)(k > 0 ? k : 1));
    double *z = (double *)malloc(sizeof(double) * (size_t)(k > 0 ? k : 1));
    int64_t n = 0, bad = 0, counted = 0;
    for (int64_t i = 0; i < k; ++i) {
      int64_t t = idx[r * idx_ld + i], row;
      if (t < 0) continue;
      if (t >= ctx_len[b] || token_row(L, bt, bt_ld, n_pages, pool_rows, b, t, &row) != OR_OK) {
        bad = 1;
        continue;
      }
      or_latent_decode(L->lat_fmt, lat_row_ptr(L, pool, layer, row, t), kv_scale, kv + 576 * n);
      counted += L->lat_bytes;
      ++n;
    }
    if (bytes_read) bytes_read[r] = counted;
    if (bad) {
#pragma omp atomic write
      rc = OR_ERR_RANGE;
    }
    for (int64_t h = 0; h < H; ++h) {
      double *o = out + (r * H + h) * 512;
      if (n == 0) {
        for (int c = 0; c < 512; ++c) o[c] = 0.0;
        lse[r * H + h] = -INFINITY;
        continue;
      }
      double qv[576], m = -INFINITY;
      for (int64_t d = 0; d < 576; ++d) qv[d] = q_elem(q, q_fmt, q_scale, H, 576, r, h, d);
      for (int64_t i = 0; i < n; ++i) {
        double dot = 0.0;
        for (int64_t d = 0; d < 576; ++d) dot += qv[d] * kv[576 * i + d];
        z[i] = sm_scale * dot;
        if (z[i] > m) m = z[i];
      }
      double s = 0.0;
      for (int64_t i = 0; i < n; ++i) s += exp(z[i] - m);
      double l = m + log(s);
      lse[r * H + h] = l;
      for (int c = 0; c < 512; ++c) o[c] = 0.0;
      for (int64_t i = 0; i < n; ++i) {
        double p = exp(z[i] - l);
        for (int c = 0; c < 512; ++c) o[c] += p * kv[576 * i + c];
      }
    }
    free(kv);
    free(z);
  }
  return rc;
}
