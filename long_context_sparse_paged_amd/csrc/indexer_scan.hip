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
//
// Native FP4 scoring (QF4, MXFP4 keys with MXFP4 queries; section "量化：原生 MXFP4 索引器":
// scoring on native FP4 matrix instructions with fp32 accumulation, and section "低延迟解码：
// 融合的 DSA 解码路径": the indexer query is quantised to FP8 or MXFP4 upstream): no decode at
// all -- per 32 tokens two v_mfma_scale_f32_32x32x64_f8f6f4 with both operands in e2m1 and
// their E8M0 block scales.  Lane (n, h) at K-step s holds dims [64s + 32h, 64s + 32h + 32) --
// exactly one 32-element MX block, i.e. 16 bytes of the row and one scale byte.  Every
// e2m1 x e2m1 product is exact, and within a block the products share one power of two.
//
// Block-table mode (BT) serves the fused score -> select path (section "低延迟解码：融合的 DSA
// 解码路径": a key-balanced scorer, then an exact top-k that emits physical rows): page
// addresses come straight from the block table (pool row * row stride + the layer's key-page
// offset), so no separate resolve launch precedes the scan.
#include <math.h>

#include <type_traits>

#include "dsa_device.hpp"
#include "dsa_kernels.hpp"

namespace dsa {

namespace {

// f(integral_constant<int, i>) for i = 0 .. N-1, unrolled (register arrays stay statically indexed)
template <int I, int N, class F>
__device__ __forceinline__ void static_for_impl(F &f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for_impl<I + 1, N>(f);
  }
}
template <int N, class F>
__device__ __forceinline__ void static_for(F f) {
  static_for_impl<0, N>(f);
}

constexpr int kScanWaves = 4;
constexpr int kScanMaxRows = 4096;
constexpr int kScoreBufUnits = 32;  // pages of scores a wave holds in LDS before writing them out

template <int KEY_FMT>
struct KeyRow {
  static constexpr int kBytes = KEY_FMT == 0 ? 132 : 68;
  static constexpr int kPageBytes = kPage * kBytes;               // 8448 / 4352
  static constexpr int kChunks = kPageBytes / 16;                 // 528 / 272
  static constexpr int kLoadsPerLane = (kChunks + 63) / 64;       // 9 / 5
  static constexpr int kFullLoads = kChunks / 64;                 // 8 / 4 (then 16 lanes of a tail)
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

template <int KEY_FMT, bool BT, bool QF4>
__global__ __launch_bounds__(256, 2) void indexer_scan_kernel(const ScoreArgs a) {
  using KR = KeyRow<KEY_FMT>;
  __shared__ __align__(16) uint8_t s_page[kScanWaves][KR::kPageBytes];
  __shared__ __align__(16) float s_sc[kScanWaves][kScoreBufUnits][kPage];
  __shared__ int s_tmp[4];
  extern __shared__ int s_start[];  // [n_q + 1]: first unit of each row

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int n_q = a.n_q;
  const int64_t pages_ld = BT ? a.bt_ld : a.off_ld;
  const int64_t max_tok = a.ld < pages_ld * kPage ? a.ld : pages_ld * kPage;

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

  // each wave: an equal contiguous share of all units; no block barriers from here on
  const int64_t nw = (int64_t)gridDim.x * kScanWaves, gw = (int64_t)blockIdx.x * kScanWaves + wid;
  // values below are wave-uniform; readfirstlane lets the compiler keep them (and the
  // control flow that depends on them) in scalar registers
  const int total_u = __builtin_amdgcn_readfirstlane(total);
  const int u_beg = (int)((int64_t)total_u * gw / nw), u_end = (int)((int64_t)total_u * (gw + 1) / nw);
  if (u_beg >= u_end) return;
  int r = 0;
  {
    int lo = 0, hi = n_q;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (__builtin_amdgcn_readfirstlane(s_start[mid]) <= u_beg) lo = mid; else hi = mid;
    }
    r = lo;
  }
  // Page offsets of the wave's units, 64 at a time: lane i looks up unit ob + i once, and the
  // loop reads its unit's offset with v_readlane.  So the steady-state loop issues no
  // dependent memory read that would make the compiler wait on vmcnt -- and with it on the
  // page prefetches in flight.
  int ob = -1;
  int64_t lane_off = -1;
  auto fill_offsets = [&](int first) __attribute__((always_inline)) {
    ob = first;
    const int uu = first + lane;
    lane_off = -1;
    if (uu < u_end) {
      int lo = 0, hi = n_q;  // row of unit uu: largest row with s_start[row] <= uu
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_start[mid] <= uu) lo = mid; else hi = mid;
      }
      if constexpr (BT) {
        const int blk = a.bt[(int64_t)a.q_req[lo] * a.bt_ld + (uu - s_start[lo])];
        if (blk < 0 || blk >= a.pool_rows)
          flag_error(a.err, DSA_DEVERR_BLOCK_RANGE);
        else
          lane_off = (int64_t)blk * a.row_stride + a.key_base;
      } else {
        lane_off = a.key_off[(int64_t)a.q_req[lo] * a.off_ld + (uu - s_start[lo])];
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // drain on this rare path (see the query reload below)
  };
  // Source of unit uu's page.  An invalid page is flagged and replaced by the pool's first page
  // (in bounds: pool_bytes >= one page is checked above) so that every prefetch issues the same
  // number of loads -- the compiler's wait counting then stays exact across loop iterations.
  auto src_of = [&](int uu, bool &ok) -> const uint8_t * {
    if (uu - ob >= 64 || ob < 0) fill_offsets(uu);
    const int li = __builtin_amdgcn_readfirstlane(uu - ob);
    const uint32_t olo = __builtin_amdgcn_readlane((uint32_t)(uint64_t)lane_off, li);
    const uint32_t ohi = __builtin_amdgcn_readlane((uint32_t)((uint64_t)lane_off >> 32), li);
    const int64_t off = (int64_t)(((uint64_t)ohi << 32) | olo);
    ok = !(off < 0 || off + KR::kPageBytes > a.pool_bytes || (off & 15));
    if (!ok) {
      // (block-table mode: a bad block id was flagged when its offset was formed)
      if (lane == 0 && !(BT && off < 0)) flag_error(a.err, DSA_DEVERR_PAGE_OFFSET);
      return a.pool;
    }
    return a.pool + off;
  };
  auto row_of = [&](int uu, int rr) {  // advance rr to unit uu's row (LDS reads only)
    while (uu >= __builtin_amdgcn_readfirstlane(s_start[rr + 1])) ++rr;
    return rr;
  };
  // pages in flight per wave (four in flight measured no faster for the short MXFP4 pages:
  // their random 4352-B reads, not the bytes in flight, set the pace)
  constexpr int NBUF = 2;
  u32x4_t bufs[NBUF][KR::kLoadsPerLane];
  // keys are read once per step: nontemporal loads keep them from displacing cached data
  constexpr int kTail = KR::kChunks - 64 * KR::kFullLoads;  // 16-B chunks in the partial last load
  auto load = [&](u32x4_t (&buf)[KR::kLoadsPerLane], const uint8_t *src) {
    const u32x4_t *p = reinterpret_cast<const u32x4_t *>(src);
#pragma unroll
    for (int i = 0; i < KR::kFullLoads; ++i) buf[i] = __builtin_nontemporal_load(p + lane + 64 * i);
    if constexpr (kTail > 0)  // every lane loads (lanes >= kTail re-read an in-page chunk)
      buf[KR::kFullLoads] = __builtin_nontemporal_load(p + 64 * KR::kFullLoads + (lane < kTail ? lane : 0));
  };
  uint8_t *slot = s_page[wid];
  auto park = [&](const u32x4_t (&buf)[KR::kLoadsPerLane]) {
    u32x4_t *q = reinterpret_cast<u32x4_t *>(slot) + lane;
#pragma unroll
    for (int i = 0; i < KR::kFullLoads; ++i) q[64 * i] = buf[i];
    if constexpr (kTail > 0)
      if (lane < kTail) q[64 * KR::kFullLoads] = buf[KR::kFullLoads];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  // Score write-back.  Scores written as the keys stream in interleave small writes with the
  // read stream and cost HBM efficiency; instead each wave keeps up to kScoreBufUnits pages of
  // scores in LDS and writes them out together (at the end of its range for most workloads).
  int nb = 0, buf_lo = 0, buf_hi = 0, buf_rem = 0;
  const bool vec_out = (reinterpret_cast<uintptr_t>(a.scores) & 15) == 0 && (a.ld & 3) == 0;
  auto lds_sync = [&]() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  auto flush = [&]() __attribute__((always_inline)) {
    lds_sync();
    for (int k = 0; k < nb; k += 4) {  // four pages (16 lanes x 4 scores each) per pass
      const int q = k + (lane >> 4), j = 4 * (lane & 15);
      const int64_t dst = (int64_t)(((uint64_t)(uint32_t)__shfl(buf_hi, q, 64) << 32) | (uint32_t)__shfl(buf_lo, q, 64));
      const int rq = __shfl(buf_rem, q, 64);
      if (q < nb && j < rq) {
        const f32x4_t s4 = *reinterpret_cast<const f32x4_t *>(&s_sc[wid][q][j]);
        float *o = a.scores + dst + j;
        if (vec_out && j + 4 <= rq) {
          *reinterpret_cast<f32x4_t *>(o) = s4;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (j + e < rq) o[e] = s4[e];
        }
      }
    }
    lds_sync();
    nb = 0;
  };

  int cur_row = -1, cur_len = 0;
  static_assert(!QF4 || KEY_FMT == 1, "FP4 queries go with MXFP4 keys");
  bf16x8_t qf[8];
  i32x8_t qa[2];     // QF4: the query's e2m1 block of each K-step (low four dwords)
  uint32_t qsc[2];   // QF4: its E8M0 scale (low byte)
  float wv[16];
  const int n = lane & 31, h = lane >> 5;
  auto compute = [&](int uu, int rr) __attribute__((always_inline)) {
    if (rr != cur_row) {
      cur_row = rr;
      cur_len = __builtin_amdgcn_readfirstlane(row_length(a, rr, max_tok, false));
      const uint16_t *qr = reinterpret_cast<const uint16_t *>(a.q) + ((int64_t)rr * kIdxHeads + n) * kIdxDim;
      if constexpr (QF4) {
        // query row of head n: 68 bytes in the key format (64 B of e2m1 pairs, 4 E8M0 scales)
        const uint8_t *q4 = static_cast<const uint8_t *>(a.q) + ((int64_t)rr * kIdxHeads + n) * 68;
        const uint32_t s4 = *reinterpret_cast<const uint32_t *>(q4 + 64);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const uint32_t *qw = reinterpret_cast<const uint32_t *>(q4 + 16 * (2 * s + h));
          qa[s] = i32x8_t{(int)qw[0], (int)qw[1], (int)qw[2], (int)qw[3], 0, 0, 0, 0};
          qsc[s] = s4 >> (8 * (2 * s + h));
        }
      } else {
#pragma unroll
        for (int s = 0; s < 8; ++s) qf[s] = *reinterpret_cast<const bf16x8_t *>(qr + 64 * h + 8 * s);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) wv[i] = a.w[(int64_t)rr * kIdxHeads + 8 * (i >> 2) + 4 * h + (i & 3)];
      // Drain here, on this rare path: loads still outstanding where it rejoins the common path
      // would make the compiler put a vmcnt wait -- counting the page prefetches -- before
      // every page's first MFMA.  (gfx9 s_waitcnt encoding: vmcnt 0, expcnt 7, lgkmcnt 15.)
      __builtin_amdgcn_s_waitcnt(0x0F70);
    }
    const int p = uu - __builtin_amdgcn_readfirstlane(s_start[rr]);
    const int rem = cur_len - p * kPage;
    // score of token 32 c2 + n; both half-waves end up holding the same value
    auto block = [&](int c2) {
      const uint8_t *row = slot + (32 * c2 + n) * KR::kBytes;
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
      } else if constexpr (QF4) {
        const uint32_t sc4 = *reinterpret_cast<const uint32_t *>(row + 64);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          // 16 B of block 2s + h (68-B rows: dword reads)
          const uint32_t *kw = reinterpret_cast<const uint32_t *>(row + 16 * (2 * s + h));
          const i32x8_t kb = {(int)kw[0], (int)kw[1], (int)kw[2], (int)kw[3], 0, 0, 0, 0};
          acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa[s], kb, acc, 4, 4, 0, qsc[s], 0,
                                                                sc4 >> (8 * (2 * s + h)));
        }
      } else {
        const uint32_t sc4 = *reinterpret_cast<const uint32_t *>(row + 64);
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const uint32_t dw = *reinterpret_cast<const uint32_t *>(row + 32 * h + 4 * s);
          const float p2 = e8m0_pow2(sc4 >> (8 * (2 * h + (s >> 2))));
          acc = mfma_32x32x16_bf16(qf[s], e2m1x8_bf16(dw, p2), acc);
        }
      }
      // ReLU(x * scale) = scale * med3(x, lo, hi): (lo, hi) = (0, inf) for scale >= 0, (-inf, 0) otherwise
      const float lo = scale < 0.0f ? -INFINITY : 0.0f, hi = scale < 0.0f ? 0.0f : INFINITY;
      float sum = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) sum = fmaf(wv[i], __builtin_amdgcn_fmed3f(acc[i], lo, hi), sum);
      return sum_halves(sum) * scale;
    };
    // scores go to the wave's LDS buffer; lane nb keeps the page's destination and length
    float *sb = s_sc[wid][nb];
    if (rem >= kPage) {
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) sb[32 * c2 + n] = block(c2);  // both lanes of a token write the same value
    } else {
      for (int c2 = 0; c2 < 2 && 32 * c2 < rem; ++c2) sb[32 * c2 + n] = block(c2);
    }
    const int64_t dst = (int64_t)rr * a.ld + (int64_t)p * kPage;
    if (lane == nb) {
      buf_lo = (int)(uint32_t)(uint64_t)dst;
      buf_hi = (int)(uint32_t)((uint64_t)dst >> 32);
      buf_rem = min(rem, kPage);
    }
    if (++nb == kScoreBufUnits) flush();
  };

  // Software pipeline: NBUF pages in registers in flight while one more is scored from LDS.
  // The steady-state loop handles NBUF units per trip and always issues NBUF pages of loads.
  if (a.pool_bytes < KR::kPageBytes) {  // no page can be valid
    if (lane == 0) flag_error(a.err, DSA_DEVERR_PAGE_OFFSET);
    return;
  }
  int u = u_beg;
  int rl = row_of(u, r);
  bool okb[NBUF];
  int rowb[NBUF];
  // units u_beg .. u_beg + NBUF - 1; a wave with fewer units still issues every load (of the
  // pool's first page), so the number of loads in flight is the same on every path
  static_for<NBUF>([&](auto I) {
    constexpr int i = decltype(I)::value;
    okb[i] = false;
    rowb[i] = rl;
    const uint8_t *src = a.pool;
    if (u + i < u_end) {
      rl = row_of(u + i, rl);
      rowb[i] = rl;
      src = src_of(u + i, okb[i]);
    }
    load(bufs[i], src);
  });
  // unit u sits in buffer (u - u_beg) % NBUF: park it, refill the buffer with unit u + NBUF,
  // score unit u from LDS
  auto stage = [&](auto I, bool refill) __attribute__((always_inline)) {
    constexpr int i = decltype(I)::value;
    park(bufs[i]);
    const bool c = okb[i];
    const int cr = rowb[i];
    if (refill) {
      rl = row_of(u + NBUF, rl);
      rowb[i] = rl;
      load(bufs[i], src_of(u + NBUF, okb[i]));
    }
    if (c) compute(u, cr); else __builtin_amdgcn_s_waitcnt(0x0F70);
    ++u;
  };
  while (u + 2 * NBUF - 1 < u_end) static_for<NBUF>([&](auto I) { stage(I, true); });
  // the last units (fewer than 2 NBUF), starting again at buffer 0
  while (u < u_end)
    static_for<NBUF>([&](auto I) {
      if (u < u_end) stage(I, u + NBUF < u_end);
    });
  if (nb > 0) flush();
}

template <int KEY_FMT, bool QF4>
void launch_scan_t(const ScoreArgs &a, dim3 grid, size_t dyn, hipStream_t s) {
  if (a.bt != nullptr)
    hipLaunchKernelGGL((indexer_scan_kernel<KEY_FMT, true, QF4>), grid, dim3(256), dyn, s, a);
  else
    hipLaunchKernelGGL((indexer_scan_kernel<KEY_FMT, false, QF4>), grid, dim3(256), dyn, s, a);
}

}  // namespace

hipError_t launch_indexer_scan(const ScoreArgs &a, hipStream_t s) {
  if (a.n_q == 0) return hipSuccess;
  if (a.n_q > kScanMaxRows) return hipErrorInvalidValue;
  const int64_t pages_ld = a.bt != nullptr ? a.bt_ld : a.off_ld;
  const int64_t max_tok = a.ld < pages_ld * kPage ? a.ld : pages_ld * kPage;
  const int64_t max_units = (int64_t)a.n_q * ((max_tok + kPage - 1) / kPage);
  int64_t grid = (max_units + 15) / 16;
  if (grid > 512) grid = 512;
  if (grid < 1) grid = 1;
  const size_t dyn = sizeof(int) * (size_t)(a.n_q + 1);
  if (a.q_fmt == DSA_Q_MXFP4) {
    if (a.key_fmt != 1) return hipErrorInvalidValue;
    launch_scan_t<1, true>(a, dim3((unsigned)grid), dyn, s);
  } else if (a.key_fmt == 0) {
    launch_scan_t<0, false>(a, dim3((unsigned)grid), dyn, s);
  } else {
    launch_scan_t<1, false>(a, dim3((unsigned)grid), dyn, s);
  }
  return hipGetLastError();
}

}  // namespace dsa
