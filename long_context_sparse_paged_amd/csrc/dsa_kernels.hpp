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
};
hipError_t launch_topk(const TopkArgs &a, hipStream_t s);

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
