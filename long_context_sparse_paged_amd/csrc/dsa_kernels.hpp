// dsa_kernels.hpp -- internal launcher interface between the C ABI (abi.cpp) and the kernels.
// Arguments arrive here already validated on the host.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "dsa.h"

namespace dsa {

struct ResolveArgs {
  const int32_t *bt;
  int64_t bt_ld;
  const int32_t *n_pages;
  int32_t n_req, max_pages;
  int64_t pool_rows;
  int64_t row_stride, layer_off, lat_page_bytes;  // layer_off = layer * layer_stride
  int64_t *lat_off, *key_off;
  int64_t off_ld;
  int32_t *err;
};
hipError_t launch_resolve(const ResolveArgs &a, hipStream_t s);

struct ScoreArgs {
  const uint8_t *pool;
  int64_t pool_bytes;
  const int64_t *key_off;
  int64_t off_ld;
  int32_t n_req;
  const void *q;         // [n_q][32][128] bf16 or e4m3
  const float *q_scale;  // [n_q][32] (FP8 queries)
  const float *w;        // [n_q][32]
  const int32_t *q_req, *row_len;
  int32_t n_q;
  float *scores;
  int64_t ld;
  int32_t *err;
  int32_t key_fmt;
  int32_t q_fmt;  // DSA_Q_BF16 or DSA_Q_MXFP4 (scan); DSA_Q_FP8_E4M3 (GEMM)
  void *ws;  // e4m3 queries: indexer_gemm_workspace_bytes(n_q) bytes, 256-B aligned
  // Block-table mode (bt != NULL; the page resolve fused into the scan): the key page of
  // (request b, page p) is at bt[b * bt_ld + p] * row_stride + key_base, with bt_ld in place
  // of off_ld; a block id outside [0, pool_rows) flags DSA_DEVERR_BLOCK_RANGE.
  const int32_t *bt;
  int64_t bt_ld, pool_rows, row_stride, key_base;
};
hipError_t launch_indexer_scan(const ScoreArgs &a, hipStream_t s);  // bf16 queries
hipError_t launch_indexer_gemm(const ScoreArgs &a, hipStream_t s);  // e4m3 queries
size_t indexer_gemm_workspace_bytes(int32_t n_q);

// Candidates straight from the FP8 prefill GEMM (rows of at most kTileModeMaxLd tokens): the
// GEMM appends each row's scores at or above its threshold to one list per 256-token tile, in
// token order; the threshold comes from kSampleTiles tiles per 32-row block scored first.
constexpr int kTileTokens = 256;
constexpr int kTileCap = 32;
constexpr int kTileModeMaxLd = 1024 * kTileTokens;
constexpr int kSampleTiles = 16;
// Sampled tile i < kSampleTiles of a row block whose longest row (row_len clamped to
// [0, ld]) is lmax; -1 if the block has fewer tiles than that.
__host__ __device__ inline int sample_tile(int i, int64_t lmax) {
  const int nt = (int)((lmax + kTileTokens - 1) / kTileTokens);
  if (nt <= kSampleTiles) return i < nt ? i : -1;
  return (int)(((int64_t)(2 * i + 1) * nt) / (2 * kSampleTiles));
}
size_t topk_tile_workspace_bytes(int32_t n_rows, int64_t ld);
struct TileLists {      // the GEMM's view of the top-k workspace in tile mode
  uint32_t *est;        // [n_rows] threshold keys (written by the tile-est kernel)
  uint32_t *cnt;        // [n_rows][n_tiles]
  uint2 *cand;          // [n_rows][n_tiles][kTileCap]
  int32_t n_tiles, k;   // n_tiles = ceil(ld / 256); k of the top-k
};
TileLists tile_lists(void *ws, int32_t n_rows, int64_t ld, int32_t k);

// Prefill indexer on FP8 MFMA (indexer_gemm_fp8.hip): its inputs for the exact rescoring and
// the error bound, carved from the caller's workspace.
//
// Every score the FP8 GEMM writes is within E_r = delta sum_g U_rg M_bg of the bf16 GEMM's
// score for the same inputs (g over the 16 groups of 8 consecutive dims, U_rg =
// sum_j s_j max_{d in g} |q~_jd|, M_bg = max_t |ks_t| max_{d in g} |k_td|); delta covers how the
// FP8 MFMA truncates products inside each group of 8 (in the |x| half of the split ReLU), the
// bf16 parts of the linear half and every fp32 rounding, with a margin.
constexpr float kFp8GroupDelta = 0x1.6p-11f;
struct PrefillWs {
  uint16_t *qb;  // [n_q][32][128] bf16 sign-folded queries q~ (exact)
  uint8_t *qc;   // [n_q][32][128] e4m3 codes of q~
  float *sw;     // [ceil(n_q / 32)][32][32] s_j = w_j |qs_j|, [row block][head][row]
  uint16_t *qlin;  // [n_q][2][128] bf16: sum_j s_j q~_j as hi + lo parts
  float *urow;   // [n_q][16] U_rg
  float *mpage;  // [n_req][off_ld][16] max over each key page's tokens of |ks_t| max_{d in g} |k_td|
  float *mreq;   // [n_req][16] M_bg: the same over the request's pages
  float *bound;      // [n_q] E_r
  float *bound_out;  // [n_q] a copy of E_r for the caller (may be NULL)
  TileLists tiles;   // tile mode: the candidate lists the GEMM appends to (tiles.cand NULL: off)
};
// The FP8 prefill indexer: the pre-pass and key bound, then the GEMM -- mode 0 every tile,
// mode 1 the sampled tiles only, mode 2 every tile with the candidate lists (tile mode:
// mode 1, then launch_topk_tile_est, then mode 2).
hipError_t launch_fp8_prepass(const ScoreArgs &a, const PrefillWs &ws, const int32_t *ctx_len, int32_t max_pages,
                              hipStream_t s);
hipError_t launch_fp8_gemm(const ScoreArgs &a, const PrefillWs &ws, const int32_t *ctx_len, int mode, hipStream_t s);

// Speculative-verify decode: m rows per request share each key page read.
constexpr int kVerifyMaxRows = 8;
constexpr int kVerifyMaxReq = 1024;
struct VerifyArgs {
  const uint8_t *pool;
  int64_t pool_bytes;
  const int64_t *key_off;
  int64_t off_ld;
  int32_t n_req, m;      // rows r = b*m + i belong to request b
  const uint16_t *q;     // bf16 [n_req*m][32][128]
  const float *w;        // [n_req*m][32]
  const int32_t *row_len;
  float *scores;
  int64_t ld;
  int32_t *err;
  int32_t key_fmt;
};
hipError_t launch_indexer_verify(const VerifyArgs &a, hipStream_t s);

// Top-k: slices of kSlice scores, candidates per slice <= kSliceCap, rows of up to
// kShortRow scores are selected wholly in LDS.
constexpr int kSlice = 8192;
constexpr int kSliceCap = 1024;  // about 6x the candidates a slice of random scores holds at k = 2048
constexpr int kShortRow = 12288;
constexpr int kMaxTopK = 4096;
size_t topk_workspace_bytes(int32_t n_rows, int64_t ld);

// Band mode of the top-k: scores known only to within E_r of the exact ones.  A first pass
// finds the k-th largest approximate score T^ and lists, in token order, the tokens that are
// surely kept (score > T^ + 2 E_r: key all ones) and the band [T^ - 2 E_r, T^ + 2 E_r]; the band
// tokens are rescored exactly (band_rescore, in indexer_gemm.hip next to the GEMM whose
// arithmetic it repeats) and a second pass selects from the list.  A band longer than
// kBandCap makes the rescoring rewrite the whole score row exactly instead, and the second
// pass select from it.
constexpr int kBandCap = 4096;
constexpr int kBandListCap = kMaxTopK + kBandCap;
struct BandWs {
  const float *e;  // [n_rows] E_r; NULL: not band mode
  int32_t *cnt;    // [n_rows][2]: list length (-1: the first pass kept the whole row), band size
  uint2 *list;     // [n_rows][kBandListCap]: (key, token) in token order
  uint2 *pos;      // [n_rows][kBandCap]: (list position, token) of each band token
};


struct TopkArgs {
  const float *scores;
  int64_t ld;
  const int32_t *row_len;
  int32_t n_rows, k;
  int32_t *idx;
  int64_t idx_ld;
  void *ws;
  int32_t *err;
  // Physical rows (phys != NULL): phys[r][i] = bt[q_req[r] * bt_ld + t / 64] * 64 + t % 64 for
  // the kept token t = idx[r][i], -1 where idx is -1 or the block id is outside [0, pool_rows)
  // (which flags DSA_DEVERR_BLOCK_RANGE).
  int32_t *phys;
  const int32_t *q_req;  // request of each row, in [0, n_req) (else DSA_DEVERR_REQUEST)
  int32_t n_req;
  const int32_t *bt;     // [n_req][bt_ld]; a row longer than 64 bt_ld flags DSA_DEVERR_ROW_LEN
  int64_t bt_ld, pool_rows;
  BandWs band;           // band mode (band.e != NULL; no physical rows)
  int32_t tile_mode;     // band mode with the lists written by the FP8 GEMM (ld <= kTileModeMaxLd)
};
hipError_t launch_topk(const TopkArgs &a, hipStream_t s);            // band mode: the first pass
hipError_t launch_topk_tile_est(const TopkArgs &a, hipStream_t s);   // tile mode: thresholds from the sampled tiles
hipError_t launch_topk_band_select(const TopkArgs &a, hipStream_t s);  // band mode: the second pass

struct RescoreArgs {
  const uint8_t *pool;
  int64_t pool_bytes;
  const int64_t *key_off;
  int64_t off_ld;
  int32_t n_req;
  const int32_t *q_req, *row_len;
  int32_t n_q;
  const uint16_t *qb;  // PrefillWs::qb
  const float *sw;     // PrefillWs::sw
  BandWs band;
  float *scores;       // rows whose band overflowed are rewritten here
  int64_t ld;
  int32_t *err;
};
hipError_t launch_band_rescore(const RescoreArgs &a, hipStream_t s);

struct MlaArgs {
  const uint8_t *pool;
  int64_t pool_bytes;
  const int64_t *lat_off;
  int64_t off_ld;
  int32_t n_req;
  const int32_t *ctx_len;
  const int32_t *idx;
  int64_t idx_ld;
  int32_t k;
  const void *q;  // [n_q][H][576] bf16 or e4m3
  const float *q_scale;
  const int32_t *q_req;  // NULL: row r is request r
  int32_t n_q, n_heads;
  float sm_scale, kv_scale;
  uint16_t *out;
  float *lse;
  int32_t *err;
  int32_t lat_fmt, q_fmt;
  void *ws;
  int32_t tokens_per_split;  // multiple of 64, <= 2048; nsplit = ceil(k / tokens_per_split)
  // Physical-row mode (phys != 0, decode kernel only): idx holds pool_row * 64 + slot, and a
  // latent sits at pool_row * row_stride + layer_off + slot * lat_bytes; lat_off and ctx_len
  // are unused.  A pool row outside [0, pool_rows) flags DSA_DEVERR_BLOCK_RANGE.
  int32_t phys;
  int64_t row_stride, layer_off, pool_rows;
};
size_t mla_workspace_bytes(int32_t n_q, int32_t n_heads, int32_t k, int32_t tokens_per_split);
hipError_t launch_mla(const MlaArgs &a, hipStream_t s);

// Exact top-k merge across emulated decode-context-parallel shards.
constexpr int kDcpMaxShards = 8;
constexpr int kDcpMaxK = 2048;
struct DcpArgs {
  const float *scores;
  int64_t ld;
  const int32_t *row_len;
  int32_t n_rows, k, n_shards;
  int32_t *idx;
  int64_t idx_ld;
  uint32_t *resend_mask;  // may be NULL
  void *ws;
  int32_t *err;
};
int32_t dcp_candidates(int32_t k, int32_t n_shards);  // ceil(1.5 k / n_shards)
size_t dcp_workspace_bytes(int32_t n_rows, int32_t k, int32_t n_shards);
hipError_t launch_dcp_topk(const DcpArgs &a, hipStream_t s);

}  // namespace dsa
