// indexer_scan.hip -- decode indexer: stream every key page of each query row's request
// and score its 64 tokens with bf16 MFMA.
//
// Page "vLLM 为 Kimi K3.1 Pro 提供 Day-0 支持":
//  * section "K3.1 Pro 中的稀疏注意力": one 132-byte FP8 key per token (128 values
//    and a scale); 32 light heads score every earlier token for each query; decode
//    still scans the whole context, which makes this scan the bandwidth-bound part;
//  * section "量化：原生 MXFP4 索引器": 68-byte MXFP4 keys, fp32 accumulation and a
//    weighted reduction across heads;
//  * section "低延迟解码：融合的 DSA 解码路径": the scorer is key-balanced, i.e. work
//    is split by keys, not by request.
// Score of token t for query row r (the DeepSeek-V3.2 indexer form the first
// section points to): sum_j w[r][j] * ReLU(q[r][j] . k_t * scale_t).
//
// Work split: the pages of all rows form one list ("units"); each workgroup takes
// an equal contiguous share, so short and long requests cost the same per key.
// Per page a wave
//   1. loads the 64 keys (8448 or 4352 contiguous bytes) with coalesced 16-B loads
//      (prefetched one page ahead) and parks them in its LDS slot,
//   2. reads, per lane, the 64 key bytes that an MFMA B fragment needs, converts
//      them in registers to bf16 (exact for e4m3 and for e2m1 x E8M0),
//   3. runs 8 v_mfma_f32_32x32x16_bf16 per 32 tokens: D[head][token] =
//      q[32 heads][128] x k[128][32 tokens], fp32 accumulation,
//   4. epilogue in the accumulator layout: lane (token n, half h) holds 16 heads;
//      sum_j w_j * ReLU(x_j), one cross-half add, times the token's scale.
// The dot product's dims may be visited in any order as long as q and k agree: lane
// (n, h) at K-step s takes dims [64h + 8s, 64h + 8s + 8), which makes both the
// query fragment and the key fragment contiguous runs of bytes.
#include "dsa_device.hpp"
#include "dsa_kernels.hpp"

namespace dsa {

namespace {

constexpr int kScanWaves = 4;
constexpr int kScanMaxRows = 4096;

template <int KEY_FMT>
struct KeyRow {
  static constexpr int kBytes = KEY_FMT == 0 ? 132 : 68;
  static constexpr int kPageBytes = kPage * kBytes;               // 8448 / 4352
  static constexpr int kChunks = kPageBytes / 16;                 // 528 / 272
  static constexpr int kLoadsPerLane = (kChunks + 63) / 64;       // 9 / 5
};

// Clamped length of row r (0 for an invalid request); flags bad rows once (block 0).
__device__ __forceinline__ int row_length(const ScoreArgs &a, int r, int64_t max_tok, bool report) {
  int len = a.row_len[r];
  const int b = a.q_req[r];
  uint32_t e = 0;
  if (b < 0 || b >= a.n_req) {
    e |= DSA_DEVERR_REQUEST;
    len = 0;
  }
  if (len < 0 || len > max_tok) {
    e |= DSA_DEVERR_ROW_LEN;
    len = len < 0 ? 0 : (int)max_tok;
  }
  if (e && report) flag_error(a.err, e);
  return len;
}

template <int KEY_FMT>
__global__ __launch_bounds__(256) void indexer_scan_kernel(const ScoreArgs a) {
  using KR = KeyRow<KEY_FMT>;
  __shared__ __align__(16) uint8_t s_page[kScanWaves][KR::kPageBytes];
  __shared__ int s_tmp[4];
  extern __shared__ int s_start[];  // [n_q + 1]: first unit of each row

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int n_q = a.n_q;
  const int64_t max_tok = a.ld < a.off_ld * kPage ? a.ld : a.off_ld * kPage;

  // 1) prefix of page counts over rows (each thread a contiguous run of rows)
  const int per = (n_q + 255) / 256;
  const int r0 = min(n_q, tid * per), r1 = min(n_q, r0 + per);
  int mine = 0;
  for (int r = r0; r < r1; ++r) mine += (row_length(a, r, max_tok, blockIdx.x == 0) + kPage - 1) / kPage;
  int total;
  int run = block_scan_incl_256(mine, s_tmp, total) - mine;
  for (int r = r0; r < r1; ++r) {
    s_start[r] = run;
    run += (row_length(a, r, max_tok, false) + kPage - 1) / kPage;
  }
  if (tid == 0) s_start[n_q] = total;
  __syncthreads();

  // 2) this workgroup's share of units; its waves take every kScanWaves-th unit in lockstep
  const int u_beg = (int)((int64_t)total * blockIdx.x / gridDim.x);
  const int u_end = (int)((int64_t)total * (blockIdx.x + 1) / gridDim.x);
  const int n_iter = (u_end - u_beg + kScanWaves - 1) / kScanWaves;
  if (n_iter == 0) return;  // uniform across the workgroup

  int u = u_beg + wid;
  int r = 0;
  if (u < u_end) {  // largest r < n_q with s_start[r] <= u
    int lo = 0, hi = n_q;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_start[mid] <= u) lo = mid; else hi = mid;
    }
    r = lo;
  }

  u32x4_t buf[KR::kLoadsPerLane];
  auto page_of = [&](int uu, int rr, const uint8_t *&src) -> bool {
    const int p = uu - s_start[rr];
    const int64_t off = a.key_off[(int64_t)a.q_req[rr] * a.off_ld + p];
    if (off < 0 || off + KR::kPageBytes > a.pool_bytes || (off & 15)) {
      if (lane == 0) flag_error(a.err, DSA_DEVERR_PAGE_OFFSET);
      return false;
    }
    src = a.pool + off;
    return true;
  };
  auto issue_loads = [&](const uint8_t *src) {
#pragma unroll
    for (int i = 0; i < KR::kLoadsPerLane; ++i) {
      const int c = lane + 64 * i;
      if (c < KR::kChunks) buf[i] = *reinterpret_cast<const u32x4_t *>(src + 16 * c);
    }
  };

  bool have = false;
  if (u < u_end) {
    const uint8_t *src;
    have = page_of(u, r, src);
    if (have) issue_loads(src);
  }

  int cur_row = -1, cur_len = 0;
  bf16x8_t qf[8];
  float wv[16];
  const int n = lane & 31, h = lane >> 5;
  uint8_t *slot = s_page[wid];

  for (int it = 0; it < n_iter; ++it) {
    if (have) {
#pragma unroll
      for (int i = 0; i < KR::kLoadsPerLane; ++i) {
        const int c = lane + 64 * i;
        if (c < KR::kChunks) *reinterpret_cast<u32x4_t *>(slot + 16 * c) = buf[i];
      }
    }
    const int cu = u, cr = r;
    const bool chave = have;
    // prefetch the wave's next page while this one is scored
    u += kScanWaves;
    have = false;
    if (u < u_end) {
      while (u >= s_start[r + 1]) ++r;
      const uint8_t *src;
      have = page_of(u, r, src);
      if (have) issue_loads(src);
    }
    __syncthreads();

    if (chave) {
      if (cr != cur_row) {
        cur_row = cr;
        cur_len = row_length(a, cr, max_tok, false);
        const uint16_t *qr = reinterpret_cast<const uint16_t *>(a.q) + ((int64_t)cr * kIdxHeads + n) * kIdxDim;
#pragma unroll
        for (int s = 0; s < 8; ++s) qf[s] = *reinterpret_cast<const bf16x8_t *>(qr + 64 * h + 8 * s);
#pragma unroll
        for (int i = 0; i < 16; ++i) wv[i] = a.w[(int64_t)cr * kIdxHeads + 8 * (i >> 2) + 4 * h + (i & 3)];
      }
      const int p = cu - s_start[cr];
      const int rem = cur_len - p * kPage;  // valid tokens in this page, >= 1
      float *out = a.scores + (int64_t)cr * a.ld + (int64_t)p * kPage;
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        if (32 * c2 >= rem) break;
        const int tt = 32 * c2 + n;
        const uint8_t *row = slot + tt * KR::kBytes;
        f32x16_t acc = {};
        float scale = 1.0f;
        if constexpr (KEY_FMT == 0) {
#pragma unroll
          for (int s = 0; s < 8; ++s) {
            const uint32_t d0 = *reinterpret_cast<const uint32_t *>(row + 64 * h + 8 * s);
            const uint32_t d1 = *reinterpret_cast<const uint32_t *>(row + 64 * h + 8 * s + 4);
            acc = mfma_32x32x16_bf16(qf[s], e4m3x8_bf16(d0, d1), acc);
          }
          scale = *reinterpret_cast<const float *>(row + 128);
        } else {
          const uint32_t sc4 = *reinterpret_cast<const uint32_t *>(row + 64);
#pragma unroll
          for (int s = 0; s < 8; ++s) {
            const uint32_t dw = *reinterpret_cast<const uint32_t *>(row + 32 * h + 4 * s);
            const float p2 = e8m0_pow2(sc4 >> (8 * (2 * h + (s >> 2))));
            acc = mfma_32x32x16_bf16(qf[s], e2m1x8_bf16(dw, p2), acc);
          }
        }
        // ReLU(x * scale) = scale * max(x, 0) for scale >= 0, scale * min(x, 0) otherwise
        const bool neg = scale < 0.0f;
        float sum = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float x = acc[i];
          sum = fmaf(wv[i], neg ? fminf(x, 0.0f) : fmaxf(x, 0.0f), sum);
        }
        const float score = sum_halves(sum) * scale;
        if (h == 0 && tt < rem) out[tt] = score;
      }
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_indexer_scan(const ScoreArgs &a, hipStream_t s) {
  if (a.n_q == 0) return hipSuccess;
  if (a.n_q > kScanMaxRows) return hipErrorInvalidValue;
  const int64_t max_tok = a.ld < a.off_ld * kPage ? a.ld : a.off_ld * kPage;
  const int64_t max_units = (int64_t)a.n_q * ((max_tok + kPage - 1) / kPage);
  int64_t grid = (max_units + 7) / 8;
  if (grid > 2048) grid = 2048;
  if (grid < 1) grid = 1;
  const size_t dyn = sizeof(int) * (size_t)(a.n_q + 1);
  if (a.key_fmt == 0)
    hipLaunchKernelGGL(indexer_scan_kernel<0>, dim3((unsigned)grid), dim3(256), dyn, s, a);
  else
    hipLaunchKernelGGL(indexer_scan_kernel<1>, dim3((unsigned)grid), dim3(256), dyn, s, a);
  return hipGetLastError();
}

}  // namespace dsa
