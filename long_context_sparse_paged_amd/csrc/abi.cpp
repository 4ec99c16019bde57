// abi.cpp -- the C entry points declared in include/dsa.h.
// Every argument is checked here, on the host, before anything is enqueued.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "dsa_device.hpp"
#include "dsa_kernels.hpp"

using namespace dsa;

namespace {

// Token splits of the decode attention: fixed, so a request's result does not
// depend on the batch it is in.
constexpr int32_t kDecodeTokensPerSplit = 128;
constexpr int32_t kMaxHeads = 128;
constexpr int32_t kMaxGridY = 65535;

bool aligned(const void *p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) & (n - 1)) == 0; }

int64_t round_up_256(int64_t x) { return (x + 255) / 256 * 256; }

dsa_status check_layout(const dsa_layout *L) {
  if (!L) return DSA_ERR_NULL_ARG;
  dsa_layout ref;
  const dsa_status s = dsa_layout_make(L->page_size, L->n_layers, L->key_fmt, L->lat_fmt, L->extra_row_bytes, &ref);
  if (s != DSA_OK) return s;
  if (ref.key_bytes != L->key_bytes || ref.lat_bytes != L->lat_bytes || ref.lat_page_bytes != L->lat_page_bytes ||
      ref.key_page_bytes != L->key_page_bytes || ref.layer_stride != L->layer_stride || ref.row_stride != L->row_stride)
    return DSA_ERR_BAD_SHAPE;
  if (L->page_size != kPage) return DSA_ERR_UNSUPPORTED;
  return DSA_OK;
}

dsa_status launched(hipError_t e) { return e == hipSuccess ? DSA_OK : DSA_ERR_HIP; }

// The FP8 prefill GEMM writes the candidate lists itself when every row fits the tile lists
// and the page table covers ld (else the top-k samples and collects from the scores).
bool prefill_tile_mode(int64_t ld, int64_t off_ld) { return ld <= kTileModeMaxLd && off_ld * kPage >= ld; }

// Workspace of dsa_prefill_select: 256-B aligned parts, in this order.
struct PrefillCarve {
  int64_t qb, qc, sw, qlin, urow, bound, mpage, mreq, topk, cnt, list, pos, total;
};
PrefillCarve prefill_carve(int32_t n_q, int64_t ld, int32_t n_req, int64_t off_ld) {
  PrefillCarve c{};
  int64_t o = 0;
  auto take = [&](int64_t bytes) {
    const int64_t at = o;
    o += round_up_256(bytes);
    return at;
  };
  c.qb = take((int64_t)n_q * kIdxHeads * kIdxDim * 2);
  c.qc = take((int64_t)n_q * kIdxHeads * kIdxDim);
  c.sw = take((int64_t)((n_q + 31) / 32) * kIdxHeads * 32 * 4);
  c.qlin = take((int64_t)n_q * 2 * kIdxDim * 2);
  c.urow = take((int64_t)n_q * 16 * 4);
  c.bound = take((int64_t)n_q * 4);
  c.mpage = take((int64_t)n_req * off_ld * 16 * 4);
  c.mreq = take((int64_t)n_req * 16 * 4);
  c.topk = take((int64_t)(prefill_tile_mode(ld, off_ld) ? topk_tile_workspace_bytes(n_q, ld)
                                                       : topk_workspace_bytes(n_q, ld)));
  c.cnt = take((int64_t)n_q * 8);
  c.list = take((int64_t)n_q * kBandListCap * 8);
  c.pos = take((int64_t)n_q * kBandCap * 8);
  c.total = o;
  return c;
}

hipStream_t stream_of(dsa_stream_t s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace

extern "C" {

const char *dsa_status_str(dsa_status s) {
  switch (s) {
    case DSA_OK: return "ok";
    case DSA_ERR_NULL_ARG: return "a required pointer is NULL";
    case DSA_ERR_BAD_SHAPE: return "invalid size, count or leading dimension";
    case DSA_ERR_MISALIGNED: return "pointer lacks the required alignment";
    case DSA_ERR_UNSUPPORTED: return "format, head count or size not supported";
    case DSA_ERR_WORKSPACE_TOO_SMALL: return "workspace smaller than the *_workspace_size answer";
    case DSA_ERR_HIP: return "HIP launch failed";
    case DSA_ERR_SCRATCH_LIMIT: return "the call needs more scratch than the library's static scratch array holds";
    default: return "unknown status";
  }
}

const char *dsa_version(void) { return "dsa-gfx950 0.1"; }

dsa_status dsa_layout_make(int32_t page_size, int32_t n_layers, int32_t key_fmt, int32_t lat_fmt,
                           int64_t extra_row_bytes, dsa_layout *out) {
  if (!out) return DSA_ERR_NULL_ARG;
  if (page_size <= 0 || n_layers <= 0 || extra_row_bytes < 0) return DSA_ERR_BAD_SHAPE;
  if ((key_fmt != DSA_KEY_FP8_E4M3_SCALED && key_fmt != DSA_KEY_MXFP4) ||
      (lat_fmt != DSA_LAT_FP8_E4M3 && lat_fmt != DSA_LAT_NVFP4))
    return DSA_ERR_UNSUPPORTED;
  dsa_layout L;
  memset(&L, 0, sizeof L);
  L.page_size = page_size;
  L.n_layers = n_layers;
  L.key_fmt = key_fmt;
  L.lat_fmt = lat_fmt;
  L.key_bytes = key_fmt == DSA_KEY_FP8_E4M3_SCALED ? 132 : 68;
  L.lat_bytes = lat_fmt == DSA_LAT_FP8_E4M3 ? 576 : 352;
  L.lat_page_bytes = (int64_t)page_size * L.lat_bytes;
  L.key_page_bytes = (int64_t)page_size * L.key_bytes;
  L.layer_stride = round_up_256(L.lat_page_bytes + L.key_page_bytes);
  L.extra_row_bytes = extra_row_bytes;
  L.row_stride = round_up_256((int64_t)n_layers * L.layer_stride + extra_row_bytes);
  *out = L;
  return DSA_OK;
}

dsa_status dsa_resolve_pages(const dsa_layout *layout, int32_t layer, const int32_t *block_table, int64_t bt_ld,
                             const int32_t *n_pages, int32_t n_req, int32_t max_pages, int64_t pool_rows,
                             int64_t *lat_off, int64_t *key_off, int64_t off_ld, int32_t *err_flag,
                             dsa_stream_t stream) {
  dsa_status st = check_layout(layout);
  if (st != DSA_OK) return st;
  if (!block_table || !n_pages || !lat_off || !key_off) return DSA_ERR_NULL_ARG;
  if (n_req < 0 || max_pages < 0 || pool_rows < 0 || bt_ld < max_pages || off_ld < max_pages || layer < 0 ||
      layer >= layout->n_layers)
    return DSA_ERR_BAD_SHAPE;
  if (n_req > kMaxGridY) return DSA_ERR_UNSUPPORTED;
  if (!aligned(block_table, 4) || !aligned(n_pages, 4) || !aligned(lat_off, 8) || !aligned(key_off, 8) ||
      !aligned(err_flag, 4))
    return DSA_ERR_MISALIGNED;
  ResolveArgs a{};
  a.bt = block_table;
  a.bt_ld = bt_ld;
  a.n_pages = n_pages;
  a.n_req = n_req;
  a.max_pages = max_pages;
  a.pool_rows = pool_rows;
  a.row_stride = layout->row_stride;
  a.layer_off = (int64_t)layer * layout->layer_stride;
  a.lat_page_bytes = layout->lat_page_bytes;
  a.lat_off = lat_off;
  a.key_off = key_off;
  a.off_ld = off_ld;
  a.err = err_flag;
  return launched(launch_resolve(a, stream_of(stream)));
}

dsa_status dsa_indexer_score(const dsa_layout *layout, const uint8_t *pool, int64_t pool_bytes,
                             const int64_t *key_off, int64_t off_ld, int32_t n_req, const void *q, int32_t q_fmt,
                             const float *q_scale, const float *w, const int32_t *q_req, const int32_t *row_len,
                             int32_t n_q, float *scores, int64_t ld, void *workspace, size_t workspace_bytes,
                             int32_t *err_flag, dsa_stream_t stream) {
  dsa_status st = check_layout(layout);
  if (st != DSA_OK) return st;
  if (q_fmt != DSA_Q_BF16 && q_fmt != DSA_Q_FP8_E4M3 && q_fmt != DSA_Q_MXFP4) return DSA_ERR_UNSUPPORTED;
  if (q_fmt == DSA_Q_MXFP4 && layout->key_fmt != DSA_KEY_MXFP4) return DSA_ERR_UNSUPPORTED;
  if (n_q < 0 || n_req < 0 || ld < 0 || off_ld < 1 || pool_bytes < 0) return DSA_ERR_BAD_SHAPE;
  if (n_q == 0) return DSA_OK;
  if (!pool || !key_off || !q || !w || !q_req || !row_len || !scores) return DSA_ERR_NULL_ARG;
  if (q_fmt == DSA_Q_FP8_E4M3 && !q_scale) return DSA_ERR_NULL_ARG;
  if (!aligned(pool, 16) || !aligned(q, 16) || !aligned(key_off, 8) || !aligned(w, 4) || !aligned(q_req, 4) ||
      !aligned(row_len, 4) || !aligned(scores, 4) || !aligned(q_scale, 4) || !aligned(err_flag, 4))
    return DSA_ERR_MISALIGNED;
  ScoreArgs a{};
  a.pool = pool;
  a.pool_bytes = pool_bytes;
  a.key_off = key_off;
  a.off_ld = off_ld;
  a.n_req = n_req;
  a.q = q;
  a.q_scale = q_scale;
  a.w = w;
  a.q_req = q_req;
  a.row_len = row_len;
  a.n_q = n_q;
  a.scores = scores;
  a.ld = ld;
  a.err = err_flag;
  a.key_fmt = layout->key_fmt;
  a.q_fmt = q_fmt;
  a.ws = nullptr;
  if (q_fmt != DSA_Q_FP8_E4M3) {
    if (n_q > 4096) return DSA_ERR_UNSUPPORTED;
    return launched(launch_indexer_scan(a, stream_of(stream)));
  }
  if (layout->key_fmt != DSA_KEY_FP8_E4M3_SCALED) return DSA_ERR_UNSUPPORTED;  // FP8 queries need FP8 keys
  if (workspace_bytes < indexer_gemm_workspace_bytes(n_q)) return DSA_ERR_WORKSPACE_TOO_SMALL;
  if (!workspace) return DSA_ERR_NULL_ARG;
  if (!aligned(workspace, 256)) return DSA_ERR_MISALIGNED;
  a.ws = workspace;
  return launched(launch_indexer_gemm(a, stream_of(stream)));
}

dsa_status dsa_indexer_score_verify(const dsa_layout *layout, const uint8_t *pool, int64_t pool_bytes,
                                    const int64_t *key_off, int64_t off_ld, int32_t n_req, int32_t rows_per_req,
                                    const uint16_t *q, const float *w, const int32_t *row_len, float *scores,
                                    int64_t ld, int32_t *err_flag, dsa_stream_t stream) {
  dsa_status st = check_layout(layout);
  if (st != DSA_OK) return st;
  if (n_req < 0 || ld < 0 || off_ld < 1 || pool_bytes < 0 || rows_per_req < 1) return DSA_ERR_BAD_SHAPE;
  if (rows_per_req > kVerifyMaxRows || n_req > kVerifyMaxReq) return DSA_ERR_UNSUPPORTED;
  if (n_req == 0) return DSA_OK;
  if (!pool || !key_off || !q || !w || !row_len || !scores) return DSA_ERR_NULL_ARG;
  if (!aligned(pool, 16) || !aligned(q, 16) || !aligned(key_off, 8) || !aligned(w, 4) || !aligned(row_len, 4) ||
      !aligned(scores, 4) || !aligned(err_flag, 4))
    return DSA_ERR_MISALIGNED;
  VerifyArgs a{};
  a.pool = pool;
  a.pool_bytes = pool_bytes;
  a.key_off = key_off;
  a.off_ld = off_ld;
  a.n_req = n_req;
  a.m = rows_per_req;
  a.q = q;
  a.w = w;
  a.row_len = row_len;
  a.scores = scores;
  a.ld = ld;
  a.err = err_flag;
  a.key_fmt = layout->key_fmt;
  return launched(launch_indexer_verify(a, stream_of(stream)));
}

dsa_status dsa_indexer_score_workspace_size(int32_t n_q, int32_t q_fmt, size_t *bytes) {
  if (!bytes) return DSA_ERR_NULL_ARG;
  if (n_q < 0) return DSA_ERR_BAD_SHAPE;
  if (q_fmt != DSA_Q_BF16 && q_fmt != DSA_Q_FP8_E4M3 && q_fmt != DSA_Q_MXFP4) return DSA_ERR_UNSUPPORTED;
  *bytes = q_fmt == DSA_Q_FP8_E4M3 ? indexer_gemm_workspace_bytes(n_q) : 0;
  return DSA_OK;
}

dsa_status dsa_prefill_select_workspace_size(int32_t n_q, int64_t ld, int32_t n_req, int64_t off_ld, int32_t k,
                                             size_t *bytes) {
  if (!bytes) return DSA_ERR_NULL_ARG;
  if (n_q < 0 || ld < 0 || n_req < 0 || off_ld < 1 || k < 1) return DSA_ERR_BAD_SHAPE;
  if (k > kMaxTopK || ld > (int64_t)1024 * kSlice) return DSA_ERR_UNSUPPORTED;
  *bytes = (size_t)prefill_carve(n_q, ld, n_req, off_ld).total;
  return DSA_OK;
}

}  // extern "C"

namespace {

// Checks shared by the prefill-select calls; on success *c is the workspace carve.
dsa_status prefill_common(const dsa_layout *layout, const uint8_t *pool, int64_t pool_bytes, const int64_t *key_off,
                          int64_t off_ld, int32_t n_req, const int32_t *q_req, const int32_t *row_len, int32_t n_q,
                          int32_t k, const float *scores, int64_t ld, void *workspace, size_t workspace_bytes,
                          const int32_t *err_flag, PrefillCarve *c) {
  dsa_status st = check_layout(layout);
  if (st != DSA_OK) return st;
  size_t need;
  st = dsa_prefill_select_workspace_size(n_q, ld, n_req, off_ld, k, &need);
  if (st != DSA_OK) return st;
  if (pool_bytes < 0) return DSA_ERR_BAD_SHAPE;
  if (layout->key_fmt != DSA_KEY_FP8_E4M3_SCALED) return DSA_ERR_UNSUPPORTED;
  if (n_q == 0) return DSA_OK;
  if (n_q > kMaxGridY || n_req > kMaxGridY) return DSA_ERR_UNSUPPORTED;
  if ((int64_t)32 * ld * 4 > 0x7FFFFFFF) return DSA_ERR_UNSUPPORTED;  // the GEMM's 32-bit store offsets
  if (!pool || !key_off || !q_req || !row_len || !scores || !workspace) return DSA_ERR_NULL_ARG;
  if (!aligned(pool, 16) || !aligned(key_off, 8) || !aligned(q_req, 4) || !aligned(row_len, 4) ||
      !aligned(scores, 16) || !aligned(workspace, 256) || !aligned(err_flag, 4))
    return DSA_ERR_MISALIGNED;
  if (workspace_bytes < need) return DSA_ERR_WORKSPACE_TOO_SMALL;
  *c = prefill_carve(n_q, ld, n_req, off_ld);
  return DSA_OK;
}

PrefillWs prefill_ws(void *workspace, const PrefillCarve &c) {
  uint8_t *base = static_cast<uint8_t *>(workspace);
  PrefillWs pw{};
  pw.qb = reinterpret_cast<uint16_t *>(base + c.qb);
  pw.qc = base + c.qc;
  pw.sw = reinterpret_cast<float *>(base + c.sw);
  pw.qlin = reinterpret_cast<uint16_t *>(base + c.qlin);
  pw.urow = reinterpret_cast<float *>(base + c.urow);
  pw.bound = reinterpret_cast<float *>(base + c.bound);
  pw.mpage = reinterpret_cast<float *>(base + c.mpage);
  pw.mreq = reinterpret_cast<float *>(base + c.mreq);
  return pw;
}

TopkArgs prefill_topk_args(const int32_t *row_len, int32_t n_q, int32_t k, float *scores, int64_t ld, int32_t *idx,
                           int64_t idx_ld, int64_t off_ld, void *workspace, const PrefillCarve &c, int32_t *err_flag) {
  uint8_t *base = static_cast<uint8_t *>(workspace);
  BandWs band{};
  band.e = reinterpret_cast<float *>(base + c.bound);
  band.cnt = reinterpret_cast<int32_t *>(base + c.cnt);
  band.list = reinterpret_cast<uint2 *>(base + c.list);
  band.pos = reinterpret_cast<uint2 *>(base + c.pos);
  TopkArgs t{};
  t.scores = scores;
  t.ld = ld;
  t.row_len = row_len;
  t.n_rows = n_q;
  t.k = k;
  t.idx = idx;
  t.idx_ld = idx_ld;
  t.ws = base + c.topk;
  t.err = err_flag;
  t.band = band;
  t.tile_mode = prefill_tile_mode(ld, off_ld) ? 1 : 0;
  return t;
}

// The score half in two parts: prepare (the pre-pass, the key bound and, in tile mode, the
// sampled tiles and the thresholds) and the full GEMM.
struct PrefillScoreCall {
  ScoreArgs a;
  PrefillWs pw;
  TopkArgs t;
  int32_t max_pages;
  bool tile;
};

PrefillScoreCall prefill_score_call(const dsa_layout *layout, const uint8_t *pool, int64_t pool_bytes,
                                    const int64_t *key_off, int64_t off_ld, int32_t n_req, const uint8_t *q,
                                    const float *q_scale, const float *w, const int32_t *q_req,
                                    const int32_t *row_len, int32_t n_q, int32_t k, float *scores, int64_t ld,
                                    float *bound, void *workspace, const PrefillCarve &c, int32_t *err_flag) {
  PrefillScoreCall p{};
  ScoreArgs &a = p.a;
  a.pool = pool;
  a.pool_bytes = pool_bytes;
  a.key_off = key_off;
  a.off_ld = off_ld;
  a.n_req = n_req;
  a.q = q;
  a.q_scale = q_scale;
  a.w = w;
  a.q_req = q_req;
  a.row_len = row_len;
  a.n_q = n_q;
  a.scores = scores;
  a.ld = ld;
  a.err = err_flag;
  a.key_fmt = layout->key_fmt;
  a.q_fmt = DSA_Q_FP8_E4M3;
  p.pw = prefill_ws(workspace, c);
  p.pw.bound_out = bound;
  const int64_t pages_ld = (ld + kPage - 1) / kPage;  // pages a row of ld tokens spans (<= 131072)
  p.max_pages = (int32_t)(off_ld < pages_ld ? off_ld : pages_ld);
  p.tile = prefill_tile_mode(ld, off_ld);
  p.t = prefill_topk_args(row_len, n_q, k, scores, ld, nullptr, k, off_ld, workspace, c, err_flag);
  if (p.tile) p.pw.tiles = tile_lists(p.t.ws, n_q, ld, k);
  return p;
}

hipError_t prefill_prepare(const PrefillScoreCall &p, const int32_t *ctx_len, hipStream_t hs) {
  hipError_t e = launch_fp8_prepass(p.a, p.pw, ctx_len, p.max_pages, hs);
  if (e != hipSuccess || !p.tile) return e;
  e = launch_fp8_gemm(p.a, p.pw, ctx_len, 1, hs);
  if (e != hipSuccess) return e;
  return launch_topk_tile_est(p.t, hs);
}

hipError_t prefill_gemm(const PrefillScoreCall &p, const int32_t *ctx_len, hipStream_t hs) {
  return launch_fp8_gemm(p.a, p.pw, ctx_len, p.tile ? 2 : 0, hs);
}

hipError_t prefill_topk(const uint8_t *pool, int64_t pool_bytes, const int64_t *key_off, int64_t off_ld, int32_t n_req,
                        const int32_t *q_req, const int32_t *row_len, int32_t n_q, int32_t k, float *scores,
                        int64_t ld, int32_t *idx, int64_t idx_ld, void *workspace, const PrefillCarve &c,
                        int32_t *err_flag, hipStream_t hs) {
  const PrefillWs pw = prefill_ws(workspace, c);
  const TopkArgs t = prefill_topk_args(row_len, n_q, k, scores, ld, idx, idx_ld, off_ld, workspace, c, err_flag);
  const BandWs band = t.band;
  hipError_t e = launch_topk(t, hs);
  if (e != hipSuccess) return e;
  RescoreArgs rs{};
  rs.pool = pool;
  rs.pool_bytes = pool_bytes;
  rs.key_off = key_off;
  rs.off_ld = off_ld;
  rs.n_req = n_req;
  rs.q_req = q_req;
  rs.row_len = row_len;
  rs.n_q = n_q;
  rs.qb = pw.qb;
  rs.sw = pw.sw;
  rs.band = band;
  rs.scores = scores;
  rs.ld = ld;
  rs.err = err_flag;
  e = launch_band_rescore(rs, hs);
  if (e != hipSuccess) return e;
  return launch_topk_band_select(t, hs);
}

}  // namespace

extern "C" {

namespace {
enum class ScorePart { kAll, kPrepare, kGemm };

dsa_status prefill_score_entry(ScorePart part, const dsa_layout *layout, const uint8_t *pool, int64_t pool_bytes,
                               const int64_t *key_off, int64_t off_ld, int32_t n_req, const int32_t *ctx_len,
                               const uint8_t *q, const float *q_scale, const float *w, const int32_t *q_req,
                               const int32_t *row_len, int32_t n_q, int32_t k, float *scores, int64_t ld,
                               float *bound, void *workspace, size_t workspace_bytes, int32_t *err_flag,
                               dsa_stream_t stream) {
  PrefillCarve c{};
  const dsa_status st = prefill_common(layout, pool, pool_bytes, key_off, off_ld, n_req, q_req, row_len, n_q, k,
                                       scores, ld, workspace, workspace_bytes, err_flag, &c);
  if (st != DSA_OK || n_q == 0) return st;
  if (!ctx_len || !q || !q_scale || !w) return DSA_ERR_NULL_ARG;
  if (!aligned(q, 16) || !aligned(ctx_len, 4) || !aligned(q_scale, 4) || !aligned(w, 4) || !aligned(bound, 4))
    return DSA_ERR_MISALIGNED;
  const PrefillScoreCall p = prefill_score_call(layout, pool, pool_bytes, key_off, off_ld, n_req, q, q_scale, w, q_req,
                                                row_len, n_q, k, scores, ld, bound, workspace, c, err_flag);
  const hipStream_t hs = stream_of(stream);
  if (part != ScorePart::kGemm && prefill_prepare(p, ctx_len, hs) != hipSuccess) return DSA_ERR_HIP;
  if (part != ScorePart::kPrepare && prefill_gemm(p, ctx_len, hs) != hipSuccess) return DSA_ERR_HIP;
  return DSA_OK;
}
}  // namespace

dsa_status dsa_prefill_score_fp8(const dsa_layout *layout, const uint8_t *pool, int64_t pool_bytes,
                                 const int64_t *key_off, int64_t off_ld, int32_t n_req, const int32_t *ctx_len,
                                 const uint8_t *q, const float *q_scale, const float *w, const int32_t *q_req,
                                 const int32_t *row_len, int32_t n_q, int32_t k, float *scores, int64_t ld,
                                 float *bound, void *workspace, size_t workspace_bytes, int32_t *err_flag,
                                 dsa_stream_t stream) {
  return prefill_score_entry(ScorePart::kAll, layout, pool, pool_bytes, key_off, off_ld, n_req, ctx_len, q, q_scale,
                             w, q_req, row_len, n_q, k, scores, ld, bound, workspace, workspace_bytes, err_flag,
                             stream);
}

dsa_status dsa_prefill_prepare_fp8(const dsa_layout *layout, const uint8_t *pool, int64_t pool_bytes,
                                   const int64_t *key_off, int64_t off_ld, int32_t n_req, const int32_t *ctx_len,
                                   const uint8_t *q, const float *q_scale, const float *w, const int32_t *q_req,
                                   const int32_t *row_len, int32_t n_q, int32_t k, float *scores, int64_t ld,
                                   float *bound, void *workspace, size_t workspace_bytes, int32_t *err_flag,
                                   dsa_stream_t stream) {
  return prefill_score_entry(ScorePart::kPrepare, layout, pool, pool_bytes, key_off, off_ld, n_req, ctx_len, q,
                             q_scale, w, q_req, row_len, n_q, k, scores, ld, bound, workspace, workspace_bytes,
                             err_flag, stream);
}

dsa_status dsa_prefill_gemm_fp8(const dsa_layout *layout, const uint8_t *pool, int64_t pool_bytes,
                                const int64_t *key_off, int64_t off_ld, int32_t n_req, const int32_t *ctx_len,
                                const uint8_t *q, const float *q_scale, const float *w, const int32_t *q_req,
                                const int32_t *row_len, int32_t n_q, int32_t k, float *scores, int64_t ld,
                                float *bound, void *workspace, size_t workspace_bytes, int32_t *err_flag,
                                dsa_stream_t stream) {
  return prefill_score_entry(ScorePart::kGemm, layout, pool, pool_bytes, key_off, off_ld, n_req, ctx_len, q, q_scale,
                             w, q_req, row_len, n_q, k, scores, ld, bound, workspace, workspace_bytes, err_flag,
                             stream);
}

dsa_status dsa_prefill_topk_band(const dsa_layout *layout, const uint8_t *pool, int64_t pool_bytes,
                                 const int64_t *key_off, int64_t off_ld, int32_t n_req, const int32_t *q_req,
                                 const int32_t *row_len, int32_t n_q, int32_t k, float *scores, int64_t ld,
                                 int32_t *idx, int64_t idx_ld, void *workspace, size_t workspace_bytes,
                                 int32_t *err_flag, dsa_stream_t stream) {
  PrefillCarve c{};
  const dsa_status st = prefill_common(layout, pool, pool_bytes, key_off, off_ld, n_req, q_req, row_len, n_q, k,
                                       scores, ld, workspace, workspace_bytes, err_flag, &c);
  if (st != DSA_OK) return st;
  if (idx_ld < k) return DSA_ERR_BAD_SHAPE;
  if (n_q == 0) return DSA_OK;
  if (!idx) return DSA_ERR_NULL_ARG;
  if (!aligned(idx, 4)) return DSA_ERR_MISALIGNED;
  return launched(prefill_topk(pool, pool_bytes, key_off, off_ld, n_req, q_req, row_len, n_q, k, scores, ld, idx,
                               idx_ld, workspace, c, err_flag, stream_of(stream)));
}

dsa_status dsa_prefill_select(const dsa_layout *layout, const uint8_t *pool, int64_t pool_bytes,
                              const int64_t *key_off, int64_t off_ld, int32_t n_req, const int32_t *ctx_len,
                              const uint8_t *q, const float *q_scale, const float *w, const int32_t *q_req,
                              const int32_t *row_len, int32_t n_q, int32_t k, float *scores, int64_t ld,
                              int32_t *idx, int64_t idx_ld, float *bound, void *workspace, size_t workspace_bytes,
                              int32_t *err_flag, dsa_stream_t stream) {
  PrefillCarve c{};
  const dsa_status st = prefill_common(layout, pool, pool_bytes, key_off, off_ld, n_req, q_req, row_len, n_q, k,
                                       scores, ld, workspace, workspace_bytes, err_flag, &c);
  if (st != DSA_OK) return st;
  if (idx_ld < k) return DSA_ERR_BAD_SHAPE;
  if (n_q == 0) return DSA_OK;
  if (!ctx_len || !q || !q_scale || !w || !idx) return DSA_ERR_NULL_ARG;
  if (!aligned(q, 16) || !aligned(ctx_len, 4) || !aligned(q_scale, 4) || !aligned(w, 4) || !aligned(bound, 4) ||
      !aligned(idx, 4))
    return DSA_ERR_MISALIGNED;
  const hipStream_t hs = stream_of(stream);
  const PrefillScoreCall p = prefill_score_call(layout, pool, pool_bytes, key_off, off_ld, n_req, q, q_scale, w, q_req,
                                                row_len, n_q, k, scores, ld, bound, workspace, c, err_flag);
  if (prefill_prepare(p, ctx_len, hs) != hipSuccess || prefill_gemm(p, ctx_len, hs) != hipSuccess)
    return DSA_ERR_HIP;
  return launched(prefill_topk(pool, pool_bytes, key_off, off_ld, n_req, q_req, row_len, n_q, k, scores, ld, idx,
                               idx_ld, workspace, c, err_flag, hs));
}

dsa_status dsa_topk_workspace_size(int32_t n_rows, int64_t ld, int32_t k, size_t *bytes) {
  if (!bytes) return DSA_ERR_NULL_ARG;
  if (n_rows < 0 || ld < 0 || k < 1) return DSA_ERR_BAD_SHAPE;
  if (k > kMaxTopK || ld > (int64_t)1024 * kSlice) return DSA_ERR_UNSUPPORTED;
  *bytes = topk_workspace_bytes(n_rows, ld);
  return DSA_OK;
}

dsa_status dsa_topk(const float *scores, int64_t ld, const int32_t *row_len, int32_t n_rows, int32_t k, int32_t *idx,
                    int64_t idx_ld, void *workspace, size_t workspace_bytes, int32_t *err_flag,
                    dsa_stream_t stream) {
  size_t need;
  dsa_status st = dsa_topk_workspace_size(n_rows, ld, k, &need);
  if (st != DSA_OK) return st;
  if (idx_ld < k) return DSA_ERR_BAD_SHAPE;
  if (n_rows == 0) return DSA_OK;
  if (!scores || !row_len || !idx || !workspace) return DSA_ERR_NULL_ARG;
  if (n_rows > kMaxGridY) return DSA_ERR_UNSUPPORTED;
  if (!aligned(scores, 4) || !aligned(row_len, 4) || !aligned(idx, 4) || !aligned(workspace, 16) ||
      !aligned(err_flag, 4))
    return DSA_ERR_MISALIGNED;
  if (workspace_bytes < need) return DSA_ERR_WORKSPACE_TOO_SMALL;
  TopkArgs a{};
  a.scores = scores;
  a.ld = ld;
  a.row_len = row_len;
  a.n_rows = n_rows;
  a.k = k;
  a.idx = idx;
  a.idx_ld = idx_ld;
  a.ws = workspace;
  a.err = err_flag;
  return launched(launch_topk(a, stream_of(stream)));
}

dsa_status dsa_dcp_topk_workspace_size(int32_t n_rows, int32_t k, int32_t n_shards, size_t *bytes) {
  if (!bytes) return DSA_ERR_NULL_ARG;
  if (n_rows < 0 || k < 1 || n_shards < 1) return DSA_ERR_BAD_SHAPE;
  if (k > kDcpMaxK || n_shards > kDcpMaxShards) return DSA_ERR_UNSUPPORTED;
  *bytes = dcp_workspace_bytes(n_rows, k, n_shards);
  return DSA_OK;
}

dsa_status dsa_dcp_topk(const float *scores, int64_t ld, const int32_t *row_len, int32_t n_rows, int32_t k,
                        int32_t n_shards, int32_t *idx, int64_t idx_ld, uint32_t *resend_mask, void *workspace,
                        size_t workspace_bytes, int32_t *err_flag, dsa_stream_t stream) {
  size_t need;
  dsa_status st = dsa_dcp_topk_workspace_size(n_rows, k, n_shards, &need);
  if (st != DSA_OK) return st;
  if (ld < 0 || idx_ld < k) return DSA_ERR_BAD_SHAPE;
  if (ld > (int64_t)65536 * n_shards) return DSA_ERR_UNSUPPORTED;
  if (n_rows == 0) return DSA_OK;
  if (!scores || !row_len || !idx || !workspace) return DSA_ERR_NULL_ARG;
  if (n_rows > kMaxGridY) return DSA_ERR_UNSUPPORTED;
  if (!aligned(scores, 4) || !aligned(row_len, 4) || !aligned(idx, 4) || !aligned(resend_mask, 4) ||
      !aligned(workspace, 16) || !aligned(err_flag, 4))
    return DSA_ERR_MISALIGNED;
  if (workspace_bytes < need) return DSA_ERR_WORKSPACE_TOO_SMALL;
  DcpArgs a{};
  a.scores = scores;
  a.ld = ld;
  a.row_len = row_len;
  a.n_rows = n_rows;
  a.k = k;
  a.n_shards = n_shards;
  a.idx = idx;
  a.idx_ld = idx_ld;
  a.resend_mask = resend_mask;
  a.ws = workspace;
  a.err = err_flag;
  return launched(launch_dcp_topk(a, stream_of(stream)));
}

static dsa_status mla_common(const dsa_layout *layout, const uint8_t *pool, int64_t pool_bytes,
                             const int64_t *lat_off, int64_t off_ld, int32_t n_req, const int32_t *ctx_len,
                             const int32_t *idx, int64_t idx_ld, int32_t k, const void *q, int32_t q_fmt,
                             const float *q_scale, const int32_t *q_req, int32_t n_q, int32_t n_heads,
                             float sm_scale, float kv_scale, uint16_t *out, float *lse, void *workspace,
                             size_t workspace_bytes, int32_t *err_flag, dsa_stream_t stream, int32_t tps) {
  dsa_status st = check_layout(layout);
  if (st != DSA_OK) return st;
  if (q_fmt != DSA_Q_BF16 && q_fmt != DSA_Q_FP8_E4M3) return DSA_ERR_UNSUPPORTED;
  if (n_q < 0 || n_req < 0 || k < 0 || idx_ld < k || off_ld < 1 || pool_bytes < 0 || n_heads < 1)
    return DSA_ERR_BAD_SHAPE;
  if (n_heads > kMaxHeads || n_q > kMaxGridY) return DSA_ERR_UNSUPPORTED;
  if (k > 64 * tps) return DSA_ERR_UNSUPPORTED;  // at most 64 token splits per row
  if (n_q == 0) return DSA_OK;
  if (pool_bytes < layout->lat_page_bytes) return DSA_ERR_BAD_SHAPE;  // smaller than one page
  if (!pool || !lat_off || !ctx_len || !idx || !q || !out || !lse) return DSA_ERR_NULL_ARG;
  if (q_fmt == DSA_Q_FP8_E4M3 && !q_scale) return DSA_ERR_NULL_ARG;
  if (!aligned(pool, 16) || !aligned(q, 16) || !aligned(lat_off, 8) || !aligned(ctx_len, 4) || !aligned(idx, 4) ||
      !aligned(out, 8) || !aligned(lse, 4) || !aligned(q_scale, 4) || !aligned(q_req, 4) || !aligned(err_flag, 4) ||
      !aligned(workspace, 16))
    return DSA_ERR_MISALIGNED;
  const size_t need = mla_workspace_bytes(n_q, n_heads, k, tps);
  if (need > 0 && !workspace) return DSA_ERR_NULL_ARG;
  if (workspace_bytes < need) return DSA_ERR_WORKSPACE_TOO_SMALL;
  MlaArgs a{};
  a.pool = pool;
  a.pool_bytes = pool_bytes;
  a.lat_off = lat_off;
  a.off_ld = off_ld;
  a.n_req = n_req;
  a.ctx_len = ctx_len;
  a.idx = idx;
  a.idx_ld = idx_ld;
  a.k = k;
  a.q = q;
  a.q_scale = q_scale;
  a.q_req = q_req;
  a.n_q = n_q;
  a.n_heads = n_heads;
  a.sm_scale = sm_scale;
  a.kv_scale = kv_scale;
  a.out = out;
  a.lse = lse;
  a.err = err_flag;
  a.lat_fmt = layout->lat_fmt;
  a.q_fmt = q_fmt;
  a.ws = workspace;
  a.tokens_per_split = tps;
  return launched(launch_mla(a, stream_of(stream)));
}

// Prefill: one split per row while k <= 2048 (whole 64-token subtiles).  Rows with at most
// 16 heads (one head tile, e.g. the verify rows of speculative decoding) take short splits:
// one workgroup per row would walk its whole set alone.  The split size depends only on k
// and the head count, so a row's result never depends on the batch it is in.
static int32_t prefill_tokens_per_split(int32_t k, int32_t n_heads) {
  if (n_heads <= 16) return 256;
  const int32_t t = k <= 64 ? 64 : (k + 63) / 64 * 64;
  return t > 2048 ? 2048 : t;
}

dsa_status dsa_sparse_mla_decode_workspace_size(int32_t n_req, int32_t n_heads, int32_t k, size_t *bytes) {
  if (!bytes) return DSA_ERR_NULL_ARG;
  if (n_req < 0 || n_heads < 1 || k < 0) return DSA_ERR_BAD_SHAPE;
  *bytes = mla_workspace_bytes(n_req, n_heads, k, kDecodeTokensPerSplit);
  return DSA_OK;
}

dsa_status dsa_sparse_mla_decode(const dsa_layout *layout, const uint8_t *pool, int64_t pool_bytes,
                                 const int64_t *lat_off, int64_t off_ld, const int32_t *ctx_len, const int32_t *idx,
                                 int64_t idx_ld, int32_t k, const uint16_t *q, int32_t n_req, int32_t n_heads,
                                 float sm_scale, float kv_scale, uint16_t *out, float *lse, void *workspace,
                                 size_t workspace_bytes, int32_t *err_flag, dsa_stream_t stream) {
  return mla_common(layout, pool, pool_bytes, lat_off, off_ld, n_req, ctx_len, idx, idx_ld, k, q, DSA_Q_BF16, nullptr,
                    nullptr, n_req, n_heads, sm_scale, kv_scale, out, lse, workspace, workspace_bytes, err_flag,
                    stream, kDecodeTokensPerSplit);
}

dsa_status dsa_sparse_mla_prefill_workspace_size(int32_t n_q, int32_t n_heads, int32_t k, size_t *bytes) {
  if (!bytes) return DSA_ERR_NULL_ARG;
  if (n_q < 0 || n_heads < 1 || k < 0) return DSA_ERR_BAD_SHAPE;
  *bytes = mla_workspace_bytes(n_q, n_heads, k, prefill_tokens_per_split(k, n_heads));
  return DSA_OK;
}

dsa_status dsa_sparse_mla_prefill(const dsa_layout *layout, const uint8_t *pool, int64_t pool_bytes,
                                  const int64_t *lat_off, int64_t off_ld, int32_t n_req, const int32_t *ctx_len,
                                  const int32_t *idx, int64_t idx_ld, int32_t k, const void *q, int32_t q_fmt,
                                  const float *q_scale, const int32_t *q_req, int32_t n_q, int32_t n_heads,
                                  float sm_scale, float kv_scale, uint16_t *out, float *lse, void *workspace,
                                  size_t workspace_bytes, int32_t *err_flag, dsa_stream_t stream) {
  if (n_q > 0 && !q_req) return DSA_ERR_NULL_ARG;
  return mla_common(layout, pool, pool_bytes, lat_off, off_ld, n_req, ctx_len, idx, idx_ld, k, q, q_fmt, q_scale,
                    q_req, n_q, n_heads, sm_scale, kv_scale, out, lse, workspace, workspace_bytes, err_flag, stream,
                    prefill_tokens_per_split(k, n_heads));
}

// ---- fused score -> select (decode) ----
dsa_status dsa_indexer_select_workspace_size(int32_t n_q, int64_t ld, size_t *bytes) {
  if (!bytes) return DSA_ERR_NULL_ARG;
  if (n_q < 0 || ld < 0) return DSA_ERR_BAD_SHAPE;
  if (ld > (int64_t)1024 * kSlice) return DSA_ERR_UNSUPPORTED;
  *bytes = topk_workspace_bytes(n_q, ld);
  return DSA_OK;
}

// Checks shared by the fused calls (block table, rows, scores).
static dsa_status fused_common(const dsa_layout *layout, int64_t pool_bytes, const int32_t *block_table, int64_t bt_ld,
                               int32_t n_req, const int32_t *q_req, const int32_t *row_len, int32_t n_q,
                               const float *scores, int64_t ld, int32_t *err_flag) {
  dsa_status st = check_layout(layout);
  if (st != DSA_OK) return st;
  if (n_q < 0 || n_req < 0 || ld < 0 || bt_ld < 1 || pool_bytes < 0) return DSA_ERR_BAD_SHAPE;
  if (n_q > 4096 || ld > (int64_t)1024 * kSlice) return DSA_ERR_UNSUPPORTED;
  if (n_q == 0) return DSA_OK;
  if (!block_table || !q_req || !row_len || !scores) return DSA_ERR_NULL_ARG;
  if (!aligned(block_table, 4) || !aligned(q_req, 4) || !aligned(row_len, 4) || !aligned(scores, 4) ||
      !aligned(err_flag, 4))
    return DSA_ERR_MISALIGNED;
  return DSA_OK;
}

static dsa_status score_pages_check(const dsa_layout *layout, int32_t layer, const uint8_t *pool, const void *q,
                                    int32_t q_fmt, const float *w) {
  if (layer < 0 || layer >= layout->n_layers) return DSA_ERR_BAD_SHAPE;
  if (q_fmt != DSA_Q_BF16 && q_fmt != DSA_Q_MXFP4) return DSA_ERR_UNSUPPORTED;
  if (q_fmt == DSA_Q_MXFP4 && layout->key_fmt != DSA_KEY_MXFP4) return DSA_ERR_UNSUPPORTED;
  if (!pool || !q || !w) return DSA_ERR_NULL_ARG;
  if (!aligned(pool, 16) || !aligned(q, 16) || !aligned(w, 4)) return DSA_ERR_MISALIGNED;
  return DSA_OK;
}

static dsa_status topk_pages_check(const dsa_layout *layout, int64_t pool_bytes, int32_t n_q, int32_t k, int64_t ld,
                                   const void *workspace, size_t workspace_bytes, const int32_t *idx,
                                   const int32_t *phys, int64_t idx_ld) {
  if (k < 1 || idx_ld < k) return DSA_ERR_BAD_SHAPE;
  if (k > kMaxTopK || n_q > kMaxGridY) return DSA_ERR_UNSUPPORTED;
  if (phys && pool_bytes / layout->row_stride > (int64_t)(INT32_MAX / kPage)) return DSA_ERR_UNSUPPORTED;
  if (!idx || !workspace) return DSA_ERR_NULL_ARG;
  if (!aligned(idx, 4) || !aligned(phys, 4) || !aligned(workspace, 16)) return DSA_ERR_MISALIGNED;
  if (workspace_bytes < topk_workspace_bytes(n_q, ld)) return DSA_ERR_WORKSPACE_TOO_SMALL;
  return DSA_OK;
}

static dsa_status launch_score_pages(const dsa_layout *layout, int32_t layer, const uint8_t *pool,
                                     int64_t pool_bytes, const int32_t *block_table, int64_t bt_ld, int32_t n_req,
                                     const void *q, int32_t q_fmt, const float *w, const int32_t *q_req,
                                     const int32_t *row_len, int32_t n_q, float *scores, int64_t ld,
                                     int32_t *err_flag, dsa_stream_t stream) {
  ScoreArgs a{};
  a.pool = pool;
  a.pool_bytes = pool_bytes;
  a.key_off = nullptr;
  a.off_ld = bt_ld;
  a.n_req = n_req;
  a.q = q;
  a.w = w;
  a.q_req = q_req;
  a.row_len = row_len;
  a.n_q = n_q;
  a.scores = scores;
  a.ld = ld;
  a.err = err_flag;
  a.key_fmt = layout->key_fmt;
  a.q_fmt = q_fmt;
  a.bt = block_table;
  a.bt_ld = bt_ld;
  a.pool_rows = pool_bytes / layout->row_stride;
  a.row_stride = layout->row_stride;
  a.key_base = (int64_t)layer * layout->layer_stride + layout->lat_page_bytes;
  return launched(launch_indexer_scan(a, stream_of(stream)));
}

static dsa_status launch_topk_pages(const dsa_layout *layout, int64_t pool_bytes, const int32_t *block_table,
                                    int64_t bt_ld, int32_t n_req, const int32_t *q_req, const float *scores,
                                    int64_t ld, const int32_t *row_len, int32_t n_q, int32_t k, void *workspace,
                                    int32_t *idx, int32_t *phys, int64_t idx_ld, int32_t *err_flag,
                                    dsa_stream_t stream) {
  TopkArgs a{};
  a.scores = scores;
  a.ld = ld;
  a.row_len = row_len;
  a.n_rows = n_q;
  a.k = k;
  a.idx = idx;
  a.idx_ld = idx_ld;
  a.ws = workspace;
  a.err = err_flag;
  a.phys = phys;
  a.q_req = q_req;
  a.n_req = n_req;
  a.bt = block_table;
  a.bt_ld = bt_ld;
  a.pool_rows = pool_bytes / layout->row_stride;
  return launched(launch_topk(a, stream_of(stream)));
}

dsa_status dsa_indexer_score_pages(const dsa_layout *layout, int32_t layer, const uint8_t *pool, int64_t pool_bytes,
                                   const int32_t *block_table, int64_t bt_ld, int32_t n_req, const void *q,
                                   int32_t q_fmt, const float *w, const int32_t *q_req, const int32_t *row_len, int32_t n_q,
                                   float *scores, int64_t ld, int32_t *err_flag, dsa_stream_t stream) {
  dsa_status st = fused_common(layout, pool_bytes, block_table, bt_ld, n_req, q_req, row_len, n_q, scores, ld,
                               err_flag);
  if (st != DSA_OK || n_q == 0) return st;
  st = score_pages_check(layout, layer, pool, q, q_fmt, w);
  if (st != DSA_OK) return st;
  return launch_score_pages(layout, layer, pool, pool_bytes, block_table, bt_ld, n_req, q, q_fmt, w, q_req, row_len,
                            n_q, scores, ld, err_flag, stream);
}

dsa_status dsa_topk_pages(const dsa_layout *layout, int64_t pool_bytes, const int32_t *block_table, int64_t bt_ld,
                          int32_t n_req, const int32_t *q_req, const float *scores, int64_t ld,
                          const int32_t *row_len, int32_t n_q, int32_t k, void *workspace, size_t workspace_bytes,
                          int32_t *idx, int32_t *phys, int64_t idx_ld, int32_t *err_flag, dsa_stream_t stream) {
  dsa_status st = fused_common(layout, pool_bytes, block_table, bt_ld, n_req, q_req, row_len, n_q, scores, ld,
                               err_flag);
  if (st != DSA_OK) return st;
  if (k < 1 || idx_ld < k) return DSA_ERR_BAD_SHAPE;
  if (n_q == 0) return k > kMaxTopK ? DSA_ERR_UNSUPPORTED : DSA_OK;
  st = topk_pages_check(layout, pool_bytes, n_q, k, ld, workspace, workspace_bytes, idx, phys, idx_ld);
  if (st != DSA_OK) return st;
  return launch_topk_pages(layout, pool_bytes, block_table, bt_ld, n_req, q_req, scores, ld, row_len, n_q, k,
                           workspace, idx, phys, idx_ld, err_flag, stream);
}

dsa_status dsa_indexer_select(const dsa_layout *layout, int32_t layer, const uint8_t *pool, int64_t pool_bytes,
                              const int32_t *block_table, int64_t bt_ld, int32_t n_req, const void *q, int32_t q_fmt,
                              const float *w, const int32_t *q_req, const int32_t *row_len, int32_t n_q, int32_t k,
                              float *scores, int64_t ld, int32_t *idx, int32_t *phys, int64_t idx_ld,
                              void *workspace, size_t workspace_bytes, int32_t *err_flag, dsa_stream_t stream) {
  // every argument of both halves is checked before the first launch
  dsa_status st = fused_common(layout, pool_bytes, block_table, bt_ld, n_req, q_req, row_len, n_q, scores, ld,
                               err_flag);
  if (st != DSA_OK) return st;
  if (k < 1 || idx_ld < k) return DSA_ERR_BAD_SHAPE;
  if (layer < 0 || layer >= layout->n_layers) return DSA_ERR_BAD_SHAPE;
  if (n_q == 0) return k > kMaxTopK ? DSA_ERR_UNSUPPORTED : DSA_OK;
  st = score_pages_check(layout, layer, pool, q, q_fmt, w);
  if (st == DSA_OK) st = topk_pages_check(layout, pool_bytes, n_q, k, ld, workspace, workspace_bytes, idx, phys, idx_ld);
  if (st != DSA_OK) return st;
  st = launch_score_pages(layout, layer, pool, pool_bytes, block_table, bt_ld, n_req, q, q_fmt, w, q_req, row_len,
                          n_q, scores, ld, err_flag, stream);
  if (st != DSA_OK) return st;
  return launch_topk_pages(layout, pool_bytes, block_table, bt_ld, n_req, q_req, scores, ld, row_len, n_q, k,
                           workspace, idx, phys, idx_ld, err_flag, stream);
}

dsa_status dsa_sparse_mla_decode_phys(const dsa_layout *layout, int32_t layer, const uint8_t *pool, int64_t pool_bytes,
                                      const int32_t *phys, int64_t idx_ld, int32_t k, const uint16_t *q,
                                      int32_t n_req, int32_t n_heads, float sm_scale, float kv_scale, uint16_t *out,
                                      float *lse, void *workspace, size_t workspace_bytes, int32_t *err_flag,
                                      dsa_stream_t stream) {
  dsa_status st = check_layout(layout);
  if (st != DSA_OK) return st;
  if (layer < 0 || layer >= layout->n_layers) return DSA_ERR_BAD_SHAPE;
  if (n_req < 0 || k < 0 || idx_ld < k || pool_bytes < 0 || n_heads < 1) return DSA_ERR_BAD_SHAPE;
  if (n_heads > kMaxHeads || n_req > kMaxGridY || k > 64 * kDecodeTokensPerSplit) return DSA_ERR_UNSUPPORTED;
  if (n_req == 0) return DSA_OK;
  if (!pool || !phys || !q || !out || !lse) return DSA_ERR_NULL_ARG;
  if (!aligned(pool, 16) || !aligned(q, 16) || !aligned(phys, 4) || !aligned(out, 8) || !aligned(lse, 4) ||
      !aligned(err_flag, 4) || !aligned(workspace, 16))
    return DSA_ERR_MISALIGNED;
  const size_t need = mla_workspace_bytes(n_req, n_heads, k, kDecodeTokensPerSplit);
  if (need > 0 && !workspace) return DSA_ERR_NULL_ARG;
  if (workspace_bytes < need) return DSA_ERR_WORKSPACE_TOO_SMALL;
  MlaArgs a{};
  a.pool = pool;
  a.pool_bytes = pool_bytes;
  a.n_req = n_req;
  a.idx = phys;
  a.idx_ld = idx_ld;
  a.k = k;
  a.q = q;
  a.n_q = n_req;
  a.n_heads = n_heads;
  a.sm_scale = sm_scale;
  a.kv_scale = kv_scale;
  a.out = out;
  a.lse = lse;
  a.err = err_flag;
  a.lat_fmt = layout->lat_fmt;
  a.q_fmt = DSA_Q_BF16;
  a.ws = workspace;
  a.tokens_per_split = kDecodeTokensPerSplit;
  a.phys = 1;
  a.row_stride = layout->row_stride;
  a.layer_off = (int64_t)layer * layout->layer_stride;
  a.pool_rows = pool_bytes / layout->row_stride;
  return launched(launch_mla(a, stream_of(stream)));
}

// ---- decode attention without a caller workspace ----
// The split partials live in one file-scope device array per GPU.  Host code must not pass
// the array's name to a kernel (on the host it is only a stand-in symbol): its device address
// is looked up once per device with hipGetSymbolAddress, with that device current, and only
// that address is used.  Calls on one GPU share the array, so calls that overlap on a GPU race;
// nothing in it needs clearing (every partial slot a call reads is written by that call).
static __device__ __align__(256) uint8_t scratch[DSA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address (looked up on its first use), or nullptr on a HIP error.
void *scratch_of_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}
}  // namespace

dsa_status dsa_sparse_mla_decode_noalloc(const dsa_layout *layout, const uint8_t *pool, int64_t pool_bytes,
                                         const int64_t *lat_off, int64_t off_ld, const int32_t *ctx_len,
                                         const int32_t *idx, int64_t idx_ld, int32_t k, const uint16_t *q,
                                         int32_t n_req, int32_t n_heads, float sm_scale, float kv_scale,
                                         uint16_t *out, float *lse, int32_t *err_flag, dsa_stream_t stream) {
  if (n_req < 0 || n_heads < 1 || k < 0) return DSA_ERR_BAD_SHAPE;
  const size_t need = mla_workspace_bytes(n_req, n_heads, k, kDecodeTokensPerSplit);
  if (need > (size_t)DSA_NOALLOC_SCRATCH_BYTES) return DSA_ERR_SCRATCH_LIMIT;
  void *ws = nullptr;
  if (need > 0 && n_req > 0) {
    ws = scratch_of_current_device();
    if (!ws) return DSA_ERR_HIP;
  }
  return mla_common(layout, pool, pool_bytes, lat_off, off_ld, n_req, ctx_len, idx, idx_ld, k, q, DSA_Q_BF16, nullptr,
                    nullptr, n_req, n_heads, sm_scale, kv_scale, out, lse, ws, need, err_flag, stream,
                    kDecodeTokensPerSplit);
}

}  // extern "C"
