// indexer_gemm.hip -- prefill indexer: (query rows) x (cached tokens) on bf16 MFMA, FP8 queries.
//
// Page "vLLM 为 Kimi K3.1 Pro 提供 Day-0 支持":
//  * section "预填充：按 token 而非按头分片注意力": in prefill every query token scores
//    every earlier token, a cost quadratic in length;
//  * section "预填充：上下文并行稀疏注意力": each row is scored against the full
//    context and the top-k is selected directly;
//  * section "低延迟解码：融合的 DSA 解码路径": the indexer query is quantised to FP8
//    with its scale folded into the head weights.
// Row r at position p scores tokens t <= p (row_len = p + 1):
//   score[r][t] = sum_j w[r][j] * ReLU(qs[r][j] * ks[t] * (qcode[r][j] . kcode[t]))
//
// Precision: gfx950's FP8 MFMA (v_mfma_*_f8f6f4 and the older fp8 ops) computes every
// single e4m3 x e4m3 product exactly but rounds inside its multi-product sums -- measured
// up to 1e-5 of sum|p| on indexer-shaped data, enough to move tokens across the top-k
// threshold by more than the 1e-5 tie window.  bf16 MFMA on the same values (e4m3 -> bf16
// is exact) accumulates in fp32 to ~1e-8.  So both operands are decoded to bf16 and the
// contraction runs on v_mfma_f32_32x32x16_bf16.
//
// Workgroup tile: 32 query rows x 256 tokens (4 pages); wave w owns page w (64 tokens,
// two 32-token MFMA columns).  The key fragments are decoded once per tile and stay in
// registers for all 32 heads.  The 32 rows' query codes are decoded into LDS two heads at
// a time (double buffered, sign of a negative qs folded in) and shared by the 4 waves.
// Per head and 32x32 sub-tile: 8 MFMAs (K = 128), then in the accumulator layout
//   acc += (w * |qs|) * sel(x),  sel = max(x,0) (ks >= 0) or min(x,0) (ks < 0);
// the store multiplies by ks.  Lane (column n, half h) at K-step s holds dims
// [64h + 8s, 64h + 8s + 8) of both operands (any dim order works if both agree).
// Grid order is row-block-major, so a row block's 128 KB of query codes stays in L2
// while its token tiles stream past.  Rows of one tile that belong to different
// requests are handled one request at a time with masked stores.
#include <math.h>

#include "dsa_device.hpp"
#include "dsa_kernels.hpp"

namespace dsa {

namespace {

constexpr int kGRows = 32;
constexpr int kGWaves = 4;
constexpr int kGTokWG = kGWaves * kPage;   // 256
constexpr int kKB = 132;                   // FP8 key row
constexpr int kKPB = kPage * kKB;          // 8448
constexpr int kChunks = kKPB / 16;         // 528
constexpr int kQLd = kIdxDim + 8;          // bf16 per LDS query row (pad against bank conflicts)

__global__ __launch_bounds__(256, 2) void indexer_gemm_kernel(const ScoreArgs a, const int n_tok_tiles) {
  __shared__ __align__(16) uint8_t s_page[kGWaves][kKPB];
  __shared__ __align__(16) uint16_t s_q[2][2][kGRows][kQLd];  // [buffer][head of the pair][row][dim]
  __shared__ __align__(16) float s_w[kIdxHeads][kGRows];  // w * |qs|, [head][row]
  __shared__ uint32_t s_neg[kIdxHeads];                   // rows with qs < 0, per head
  __shared__ int s_req[kGRows], s_len[kGRows];

  const int tile = blockIdx.x % n_tok_tiles;
  const int row0 = (blockIdx.x / n_tok_tiles) * kGRows;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int n = lane & 31, h = lane >> 5;
  const int64_t max_tok = a.ld < a.off_ld * kPage ? a.ld : a.off_ld * kPage;
  const bool report = tile == 0;

  if (tid < kIdxHeads) s_neg[tid] = 0;
  if (tid < kGRows) {
    const int r = row0 + tid;
    int req = -1, len = 0;
    if (r < a.n_q) {
      const int b = a.q_req[r];
      len = a.row_len[r];
      uint32_t e = 0;
      if (b < 0 || b >= a.n_req) e |= DSA_DEVERR_REQUEST; else req = b;
      if (len < 0 || len > max_tok) {
        e |= DSA_DEVERR_ROW_LEN;
        len = len < 0 ? 0 : (int)max_tok;
      }
      if (e && report) flag_error(a.err, e);
    }
    s_req[tid] = req;
    s_len[tid] = req >= 0 ? len : 0;
  }
  __syncthreads();
  for (int i = tid; i < kIdxHeads * kGRows; i += 256) {
    const int j = i / kGRows, m = i % kGRows, r = row0 + m;
    float v = 0.0f;
    if (r < a.n_q) {
      const float qs = a.q_scale[(int64_t)r * kIdxHeads + j];
      v = a.w[(int64_t)r * kIdxHeads + j] * fabsf(qs);
      if (qs < 0.0f) atomicOr(&s_neg[j], 1u << m);
    }
    s_w[j][m] = v;
  }
  __syncthreads();

  uint32_t todo = 0;
  for (int m = 0; m < kGRows; ++m)
    if (s_req[m] >= 0) todo |= 1u << m;
  const uint8_t *qbase = static_cast<const uint8_t *>(a.q);
  // this thread's share of a head tile: row qm, codes [16 qc, 16 qc + 16)
  const int qm = tid >> 3, qc = tid & 7;
  const bool q_ok = row0 + qm < a.n_q;
  const uint8_t *qsrc = qbase + ((int64_t)(row0 + qm) * kIdxHeads) * kIdxDim + 16 * qc;

  while (todo) {
    const int b = s_req[__ffs(todo) - 1];
    uint32_t rows = 0;
    int lmax = 0;
    for (int m = 0; m < kGRows; ++m)
      if (s_req[m] == b) {
        rows |= 1u << m;
        lmax = max(lmax, s_len[m]);
      }
    todo &= ~rows;
    if (tile * kGTokWG >= lmax) continue;  // uniform: the tile lies past every row's length

    // (1) this wave's key page -> LDS
    const int wtok0 = tile * kGTokWG + wid * kPage;
    bool page_ok = false;
    if (wtok0 < lmax) {
      const int64_t off = a.key_off[(int64_t)b * a.off_ld + wtok0 / kPage];
      if (off < 0 || off + kKPB > a.pool_bytes || (off & 15)) {
        if (lane == 0) flag_error(a.err, DSA_DEVERR_PAGE_OFFSET);
      } else {
        page_ok = true;
        const uint8_t *src = a.pool + off;
        for (int c = lane; c < kChunks; c += 64)
          *reinterpret_cast<u32x4_t *>(s_page[wid] + 16 * c) = *reinterpret_cast<const u32x4_t *>(src + 16 * c);
      }
    }
    // (2) head 0's query tile -> LDS as bf16
    auto stage_q = [&](int j, u32x4_t raw, int buf, int hh) {
      const bf16x8_t lo = e4m3x8_bf16(raw[0], raw[1]), hi = e4m3x8_bf16(raw[2], raw[3]);
      u32x4_t x0 = __builtin_bit_cast(u32x4_t, lo), x1 = __builtin_bit_cast(u32x4_t, hi);
      if ((s_neg[j] >> qm) & 1u) {
        x0 ^= 0x80008000u;
        x1 ^= 0x80008000u;
      }
      *reinterpret_cast<u32x4_t *>(&s_q[buf][hh][qm][16 * qc]) = x0;
      *reinterpret_cast<u32x4_t *>(&s_q[buf][hh][qm][16 * qc + 8]) = x1;
    };
    u32x4_t qraw0 = q_ok ? *reinterpret_cast<const u32x4_t *>(qsrc) : u32x4_t{};
    u32x4_t qraw1 = q_ok ? *reinterpret_cast<const u32x4_t *>(qsrc + kIdxDim) : u32x4_t{};
    stage_q(0, qraw0, 0, 0);
    stage_q(1, qraw1, 0, 1);
    __syncthreads();

    // (3) key fragments, decoded once, resident for all heads
    bf16x8_t bf[2][8];
    float ks[2], lo[2], hi[2];
    f32x16_t acc[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const uint8_t *kr = s_page[wid] + (32 * c + n) * kKB;
#pragma unroll
      for (int s = 0; s < 8; ++s)
        bf[c][s] = e4m3x8_bf16(*reinterpret_cast<const uint32_t *>(kr + 64 * h + 8 * s),
                               *reinterpret_cast<const uint32_t *>(kr + 64 * h + 8 * s + 4));
      ks[c] = *reinterpret_cast<const float *>(kr + 128);
      lo[c] = ks[c] < 0.0f ? -INFINITY : 0.0f;
      hi[c] = ks[c] < 0.0f ? 0.0f : INFINITY;
      acc[c] = f32x16_t{};
    }

    // (4) heads, two per barrier: the pair's query tiles are staged together
    for (int j0 = 0; j0 < kIdxHeads; j0 += 2) {
      const int buf = (j0 >> 1) & 1;
      if (j0 + 2 < kIdxHeads && q_ok) {
        qraw0 = *reinterpret_cast<const u32x4_t *>(qsrc + (j0 + 2) * kIdxDim);
        qraw1 = *reinterpret_cast<const u32x4_t *>(qsrc + (j0 + 3) * kIdxDim);
      }
      if (page_ok) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int j = j0 + hh;
          bf16x8_t af[8];
#pragma unroll
          for (int s = 0; s < 8; ++s) af[s] = *reinterpret_cast<const bf16x8_t *>(&s_q[buf][hh][n][64 * h + 8 * s]);
          float wv[16];
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const f32x4_t t4 = *reinterpret_cast<const f32x4_t *>(&s_w[j][8 * q4 + 4 * h]);
#pragma unroll
            for (int i = 0; i < 4; ++i) wv[4 * q4 + i] = t4[i];
          }
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            f32x16_t x = {};
#pragma unroll
            for (int s = 0; s < 8; ++s) x = mfma_32x32x16_bf16(af[s], bf[c][s], x);
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[c][i] = fmaf(wv[i], __builtin_amdgcn_fmed3f(x[i], lo[c], hi[c]), acc[c][i]);
          }
        }
      }
      if (j0 + 2 < kIdxHeads) {
        stage_q(j0 + 2, q_ok ? qraw0 : u32x4_t{}, buf ^ 1, 0);
        stage_q(j0 + 3, q_ok ? qraw1 : u32x4_t{}, buf ^ 1, 1);
      }
      __syncthreads();
    }

    // (5) store: acc[c][i] is row 8*(i/4) + 4h + i%4, token wtok0 + 32c + n
    if (page_ok) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int t = wtok0 + 32 * c + n;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int m = 8 * (i >> 2) + 4 * h + (i & 3);
          if (((rows >> m) & 1u) && t < s_len[m]) a.scores[(int64_t)(row0 + m) * a.ld + t] = ks[c] * acc[c][i];
        }
      }
    }
    __syncthreads();  // s_page / s_q are refilled for the next request of this tile
  }
}

}  // namespace

hipError_t launch_indexer_gemm(const ScoreArgs &a, hipStream_t s) {
  if (a.n_q == 0) return hipSuccess;
  if (a.key_fmt != 0) return hipErrorInvalidValue;
  const int64_t max_tok = a.ld < a.off_ld * kPage ? a.ld : a.off_ld * kPage;
  const int64_t n_tok_tiles = (max_tok + kGTokWG - 1) / kGTokWG;
  const int64_t n_row_blocks = (a.n_q + kGRows - 1) / kGRows;
  const int64_t grid = n_tok_tiles * n_row_blocks;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(indexer_gemm_kernel, dim3((unsigned)grid), dim3(256), 0, s, a, (int)n_tok_tiles);
  return hipGetLastError();
}

}  // namespace dsa
