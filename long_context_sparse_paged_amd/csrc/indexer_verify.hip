// indexer_verify.hip -- decode indexer for speculative verification: the m query rows of a
// request (the last accepted token plus m-1 draft tokens) are scored from one read of each
// key page.
//
// Page "vLLM 为 Kimi K3.1 Pro 提供 Day-0 支持":
//  * section "量化：原生 MXFP4 索引器": during speculative verification the keys are reused
//    across query rows, so that they are not read again for every row;
//  * section "低延迟解码：融合的 DSA 解码路径": DSpark speculative decoding with 7 draft
//    tokens, i.e. 8 query rows per request;
//  * section "K3.1 Pro 中的稀疏注意力": the indexer score of one row (132-byte FP8 keys or
//    68-byte MXFP4 keys, 32 heads): sum_j w_j * ReLU(q_j . k_t * scale_t).
//
// Rows r = b*m + i (i < m) belong to request b; row r scores tokens t < row_len[r].
//
// Work split: a tile is NW consecutive pages (one per wave) of one request; the tiles of all
// requests form one list and each workgroup takes an equal contiguous share, so the scan
// stays key-balanced.  Wave w of the workgroup owns page w of each tile.  The request's m
// query rows (m x 8 KB bf16) and head weights sit in LDS, shared by the NW waves, and are
// restaged (between two barriers) only when the workgroup's tile moves to another request.
// Per page a wave
//   1. loads the 64 keys with coalesced nontemporal 16-B loads, one page ahead, and parks
//      them in its LDS slot,
//   2. decodes the B fragments of both 32-token blocks to bf16 once (exact),
//   3. for each row of the request (m is a compile-time count, so the rows unroll): 8 + 8
//      v_mfma_f32_32x32x16_bf16 with A fragments read from LDS at immediate offsets, then
//      the weighted ReLU head sum in the accumulator layout into a per-wave LDS buffer,
//   4. stores the previous page's m x 64 scores at the top of the next iteration, before the
//      next page load, so that waiting for a page never waits for score stores.
// The per-row arithmetic (operand order, accumulation order, epilogue) is the same as the
// one-row scan's, so a row's scores do not depend on which of the two kernels made them.
#include <math.h>

#include "dsa_device.hpp"
#include "dsa_kernels.hpp"

namespace dsa {

namespace {

template <int KEY_FMT>
struct VKeyRow {
  static constexpr int kBytes = KEY_FMT == 0 ? 132 : 68;
  static constexpr int kPageBytes = kPage * kBytes;          // 8448 / 4352
  static constexpr int kChunks = kPageBytes / 16;            // 528 / 272
  static constexpr int kLoadsPerLane = (kChunks + 63) / 64;  // 9 / 5
  static constexpr int kFullLoads = kChunks / 64;            // 8 / 4
};

// Clamped length of row r; flags a bad length (reported by block 0 only).
__device__ __forceinline__ int vrow_length(const VerifyArgs &a, int r, int64_t max_tok, bool report) {
  int len = a.row_len[r];
  if (len < 0 || len > max_tok) {
    if (report) flag_error(a.err, DSA_DEVERR_ROW_LEN);
    len = len < 0 ? 0 : (int)max_tok;
  }
  return len;
}

// NW waves per workgroup, one page each per tile; M rows per request (a compile-time
// count, so the row loop unrolls and each row's LDS reads take the row as an immediate offset).
template <int KEY_FMT, int M, int NW>
__global__ __launch_bounds__(64 * NW, 2) void indexer_verify_kernel(const VerifyArgs a) {
  using KR = VKeyRow<KEY_FMT>;
  constexpr int NT = 64 * NW;
  __shared__ __align__(16) uint8_t s_page[NW][KR::kPageBytes];
  // query rows of the current request: [row][head][16 chunks of 8 dims], chunk c of head j
  // stored at chunk position c ^ (j & 15) so that the A-fragment reads are conflict-free
  __shared__ __align__(16) uint16_t s_q[M][kIdxHeads][kIdxDim];
  __shared__ __align__(16) float s_w[M][kIdxHeads];
  __shared__ int s_len[M];
  __shared__ float s_out[NW][M][kPage];  // the wave's last page of scores, stored one iteration later
  __shared__ int s_tmp[NW];
  extern __shared__ int s_dyn[];  // [n_req + 1] first tile of each request, then [n_req] pages
  int *s_start = s_dyn, *s_pages = s_dyn + a.n_req + 1;

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int n_req = a.n_req;
  constexpr int m = M;
  const int64_t max_tok = a.ld < a.off_ld * kPage ? a.ld : a.off_ld * kPage;

  // tiles per request: ceil(pages / NW), pages from the request's longest row
  const int per = (n_req + NT - 1) / NT;
  const int r0 = min(n_req, tid * per), r1 = min(n_req, r0 + per);
  int mine = 0;
  for (int b = r0; b < r1; ++b) {
    int len = 0;
    for (int i = 0; i < m; ++i) len = max(len, vrow_length(a, b * m + i, max_tok, blockIdx.x == 0));
    const int pg = (len + kPage - 1) / kPage;
    s_pages[b] = pg;
    mine += (pg + NW - 1) / NW;
  }
  int total;
  int run = block_scan_incl<NT>(mine, s_tmp, total) - mine;
  for (int b = r0; b < r1; ++b) {
    s_start[b] = run;
    run += (s_pages[b] + NW - 1) / NW;
  }
  if (tid == 0) s_start[n_req] = total;
  __syncthreads();

  const int total_t = __builtin_amdgcn_readfirstlane(total);
  const int t_beg = (int)((int64_t)total_t * blockIdx.x / gridDim.x);
  const int t_end = (int)((int64_t)total_t * (blockIdx.x + 1) / gridDim.x);
  if (t_beg >= t_end) return;  // uniform over the workgroup
  if (a.pool_bytes < KR::kPageBytes) {  // no page can be valid
    if (tid == 0) flag_error(a.err, DSA_DEVERR_PAGE_OFFSET);
    return;
  }
  auto req_of = [&](int tt) {  // largest request with s_start[b] <= tt
    int lo = 0, hi = n_req;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_start[mid] <= tt) lo = mid; else hi = mid;
    }
    return lo;
  };

  // Page offsets of this wave's pages for the next 64 tiles, one per lane (read back with
  // v_readlane): -2 = the request has no page w in this tile (nothing to do, not an error).
  int ob = -1;
  int64_t lane_off = -2;
  auto fill_offsets = [&](int first) {
    ob = first;
    const int tt = first + lane;
    lane_off = -2;
    if (tt < t_end) {
      const int b = req_of(tt);
      const int p = NW * (tt - s_start[b]) + wid;
      if (p < s_pages[b]) lane_off = a.key_off[(int64_t)b * a.off_ld + p];
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // drain on this rare path (vmcnt 0)
  };
  // Source of this wave's page of tile tt; `has` = the page exists, `ok` = its offset is valid.
  // Without a valid page the wave loads the pool's first page (in bounds) so that every
  // iteration issues the same loads and the compiler's wait counts stay exact.
  auto src_of = [&](int tt, bool &has, bool &ok) -> const uint8_t * {
    if (tt - ob >= 64 || ob < 0) fill_offsets(tt);
    const int li = __builtin_amdgcn_readfirstlane(tt - ob);
    const uint32_t olo = __builtin_amdgcn_readlane((uint32_t)(uint64_t)lane_off, li);
    const uint32_t ohi = __builtin_amdgcn_readlane((uint32_t)((uint64_t)lane_off >> 32), li);
    const int64_t off = (int64_t)(((uint64_t)ohi << 32) | olo);
    has = off != -2;
    ok = has && !(off < 0 || off + KR::kPageBytes > a.pool_bytes || (off & 15));
    if (has && !ok) {
      if (lane == 0) flag_error(a.err, DSA_DEVERR_PAGE_OFFSET);
    }
    return ok ? a.pool + off : a.pool;
  };

  u32x4_t b0[KR::kLoadsPerLane];
  constexpr int kTail = KR::kChunks - 64 * KR::kFullLoads;
  auto load = [&](u32x4_t (&buf)[KR::kLoadsPerLane], const uint8_t *src) {
    const u32x4_t *p = reinterpret_cast<const u32x4_t *>(src);
#pragma unroll
    for (int i = 0; i < KR::kFullLoads; ++i) buf[i] = __builtin_nontemporal_load(p + lane + 64 * i);
    if constexpr (kTail > 0)
      buf[KR::kFullLoads] = __builtin_nontemporal_load(p + 64 * KR::kFullLoads + (lane < kTail ? lane : 0));
  };
  uint8_t *slot = s_page[wid];
  auto wave_sync = [&]() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  auto park = [&](const u32x4_t (&buf)[KR::kLoadsPerLane]) {
    wave_sync();  // the previous page's reads of the slot are done
    u32x4_t *q = reinterpret_cast<u32x4_t *>(slot) + lane;
#pragma unroll
    for (int i = 0; i < KR::kFullLoads; ++i) q[64 * i] = buf[i];
    if constexpr (kTail > 0)
      if (lane < kTail) q[64 * KR::kFullLoads] = buf[KR::kFullLoads];
    wave_sync();
  };

  // Stage request b's rows: all threads, between two barriers.
  int cur_b = -1;
  auto stage = [&](int b) {
    __syncthreads();  // every wave has finished with the previous request's rows
    const int nch = m * kIdxHeads * (kIdxDim / 8);
    const u32x4_t *qg = reinterpret_cast<const u32x4_t *>(a.q) + (int64_t)b * nch;
    for (int i = tid; i < nch; i += NT) {
      const int g = i >> 9, j = (i >> 4) & 31, c = i & 15;
      const u32x4_t v = qg[i];
      *reinterpret_cast<u32x4_t *>(&s_q[g][j][8 * (c ^ (j & 15))]) = v;
    }
    for (int i = tid; i < m * kIdxHeads; i += NT) s_w[i >> 5][i & 31] = a.w[(int64_t)b * m * kIdxHeads + i];
    if (tid < m) s_len[tid] = vrow_length(a, b * m + tid, max_tok, false);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // drain here, off the common path
    __syncthreads();
  };

  const int n = lane & 31, h = lane >> 5;
  const int tok = 32 * h + n;  // lane (n, h) handles token 32 h + n of a page
  // Scores of the last page, per row: the row's page base and valid count (wave-uniform).
  // They are stored at the top of the next iteration, before the next page load is issued,
  // so that the wait for a page never has to wait for stores issued after it.
  uint64_t pend_base[M];
  int pend_nv[M];
#pragma unroll
  for (int g = 0; g < M; ++g) {
    pend_base[g] = reinterpret_cast<uint64_t>(a.scores);
    pend_nv[g] = 0;
  }
  auto flush = [&]() {
#pragma unroll
    for (int g = 0; g < M; ++g) {
      const float v = s_out[wid][g][tok];
      const __amdgpu_buffer_rsrc_t ors =
          __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<float *>(pend_base[g]), 0, 4 * pend_nv[g], 0x00020000);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), ors, 4 * tok, 0, 0);
    }
  };
  auto compute = [&](int tt, int b, bool valid) {
    b = __builtin_amdgcn_readfirstlane(b);
    if (b != cur_b) {
      stage(b);
      cur_b = b;
    }
    // An invalid page (none for this wave in the tile, or a bad offset) is scored like any
    // other -- from the pool's first bytes -- and its stores get an empty range, so every
    // iteration issues the same memory operations and the wait for the next page counts
    // only the stores issued after it, not a drain of everything.
    // wave-uniform, so that the score stores' buffer descriptors live in scalar registers
    const int p = __builtin_amdgcn_readfirstlane(NW * (tt - s_start[b]) + wid);
    // B fragments of both 32-token blocks, decoded once for all rows
    bf16x8_t kf[2][8];
    float scale[2];
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      const uint8_t *row = slot + (32 * c2 + n) * KR::kBytes;
      if constexpr (KEY_FMT == 0) {
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const uint32_t d0 = *reinterpret_cast<const uint32_t *>(row + 64 * h + 8 * s);
          const uint32_t d1 = *reinterpret_cast<const uint32_t *>(row + 64 * h + 8 * s + 4);
          kf[c2][s] = e4m3x8_bf16(d0, d1);
        }
        scale[c2] = *reinterpret_cast<const float *>(row + 128);
      } else {
        const uint32_t sc4 = *reinterpret_cast<const uint32_t *>(row + 64);
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const uint32_t dw = *reinterpret_cast<const uint32_t *>(row + 32 * h + 4 * s);
          kf[c2][s] = e2m1x8_bf16(dw, e8m0_pow2(sc4 >> (8 * (2 * h + (s >> 2)))));
        }
        scale[c2] = 1.0f;
      }
    }
    float lo[2], hi[2];
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      lo[c2] = scale[c2] < 0.0f ? -INFINITY : 0.0f;
      hi[c2] = scale[c2] < 0.0f ? 0.0f : INFINITY;
    }
    // Rows one after another (unrolled: each row's A-fragment reads take the row as an
    // immediate LDS offset); the other wave on the SIMD fills one wave's epilogue time.  Every
    // row of the request runs its MFMAs; a row that does not reach this page stores nothing
    // (its buffer range is empty), so the row loop has no branch.
    auto load_a = [&](int g, bf16x8_t (&qa)[8]) {
      const uint16_t *qrow = &s_q[g][n][0];
#pragma unroll
      for (int s = 0; s < 8; ++s) qa[s] = *reinterpret_cast<const bf16x8_t *>(qrow + 8 * ((8 * h + s) ^ (n & 15)));
    };
    auto row = [&](int g, const bf16x8_t (&qa)[8]) {
      f32x16_t c0 = {}, c1 = {};
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        c0 = mfma_32x32x16_bf16(qa[s], kf[0][s], c0);
        c1 = mfma_32x32x16_bf16(qa[s], kf[1][s], c1);
      }
      const int rem = __builtin_amdgcn_readfirstlane(s_len[g]) - p * kPage;
      const float *wg = &s_w[g][4 * h];
      float sum0 = 0.0f, sum1 = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float wv = wg[8 * (i >> 2) + (i & 3)];
        sum0 = fmaf(wv, __builtin_amdgcn_fmed3f(c0[i], lo[0], hi[0]), sum0);
        sum1 = fmaf(wv, __builtin_amdgcn_fmed3f(c1[i], lo[1], hi[1]), sum1);
      }
      const float s0 = sum_halves(sum0) * scale[0], s1 = sum_halves(sum1) * scale[1];
      s_out[wid][g][tok] = h ? s1 : s0;
      // the page's part of the row as a buffer of max(0, min(rem, 64)) scores: the later
      // stores past it are dropped by the range check
      pend_nv[g] = __builtin_amdgcn_readfirstlane(!valid || rem < 0 ? 0 : (rem > kPage ? kPage : rem));
      const uint64_t base = reinterpret_cast<uint64_t>(a.scores + (int64_t)(b * m + g) * a.ld + (int64_t)p * kPage);
      pend_base[g] = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(base >> 32)) << 32) |
                     (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)base);
    };
#pragma unroll
    for (int g = 0; g < M; ++g) {
      bf16x8_t qa[8];
      load_a(g, qa);
      row(g, qa);
    }
  };

  // Pipeline: one page in flight in registers while the previous one is scored from LDS (the
  // kernel is bound by the matrix cores, not by HBM, once several rows share a page); every
  // iteration issues the same loads and stores, so the compiler's wait for a page is exact.
  int t = t_beg;
  int bl = req_of(t);
  auto adv = [&](int tt, int bb) {  // request of tile tt, walking forward from bb
    while (tt >= __builtin_amdgcn_readfirstlane(s_start[bb + 1])) ++bb;
    return bb;
  };
  bool has0, ok0;
  int rq0 = bl;
  load(b0, src_of(t, has0, ok0));
  for (; t < t_end; ++t) {
    park(b0);
    const bool v0 = ok0;
    const int c0 = rq0;
    // past the last tile the load reads the pool's first page (in bounds) and is not used
    const uint8_t *nsrc = a.pool;
    if (t + 1 < t_end) {
      bl = adv(t + 1, bl);
      rq0 = bl;
      nsrc = src_of(t + 1, has0, ok0);
    }
    flush();  // the previous page's scores (an empty range before the first page)
    load(b0, nsrc);
    compute(t, c0, v0);
  }
  flush();
}

// m <= 4: two 4-wave workgroups per CU; m <= 8: one 8-wave workgroup per CU (one copy of the
// query rows, up to 64 KB, for eight pages).  Either way two waves per SIMD.
template <int KEY_FMT, int M, int NW = (M <= 4 ? 4 : 8)>
hipError_t launch_verify_t(const VerifyArgs &a, hipStream_t s) {
  const int64_t max_tok = a.ld < a.off_ld * kPage ? a.ld : a.off_ld * kPage;
  const int64_t max_tiles = (int64_t)a.n_req * (((max_tok + kPage - 1) / kPage + NW - 1) / NW);
  int64_t grid = (max_tiles + 7) / 8;
  const int64_t cap = NW == 4 ? 512 : 256;
  if (grid > cap) grid = cap;
  if (grid < 1) grid = 1;
  const size_t dyn = sizeof(int) * (size_t)(2 * a.n_req + 1);
  hipLaunchKernelGGL((indexer_verify_kernel<KEY_FMT, M, NW>), dim3((unsigned)grid), dim3(64 * NW), dyn, s, a);
  return hipGetLastError();
}

template <int KEY_FMT>
hipError_t launch_verify_m(const VerifyArgs &a, hipStream_t s) {
  switch (a.m) {
    case 1: return launch_verify_t<KEY_FMT, 1>(a, s);
    case 2: return launch_verify_t<KEY_FMT, 2>(a, s);
    case 3: return launch_verify_t<KEY_FMT, 3>(a, s);
    case 4: return launch_verify_t<KEY_FMT, 4>(a, s);
    case 5: return launch_verify_t<KEY_FMT, 5>(a, s);
    case 6: return launch_verify_t<KEY_FMT, 6>(a, s);
    case 7: return launch_verify_t<KEY_FMT, 7>(a, s);
    default: return launch_verify_t<KEY_FMT, 8>(a, s);
  }
}

}  // namespace

hipError_t launch_indexer_verify(const VerifyArgs &a, hipStream_t s) {
  if (a.n_req == 0) return hipSuccess;
  if (a.m < 1 || a.m > kVerifyMaxRows || a.n_req > kVerifyMaxReq) return hipErrorInvalidValue;
  return a.key_fmt == 0 ? launch_verify_m<0>(a, s) : launch_verify_m<1>(a, s);
}

}  // namespace dsa
