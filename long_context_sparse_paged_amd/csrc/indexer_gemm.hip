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
// The ReLU is applied per head, exactly as in the decode scan.  With the sign of qs folded
// into the query (q~ = sign(qs) qcode), s_j = w_j |qs_j| and x_j = q~_j . kcode:
//   score = sum_j s_j ReLU(ks x_j) = ks sum_j s_j med3(x_j, lo, hi),
// (lo, hi) = (0, inf) for ks >= 0 and (-inf, 0) otherwise.  Every term is >= 0, so a row
// where no head is positive scores exactly +0 and a small score next to large per-head
// terms keeps fp32's relative precision (a split into a linear part and sum_j s_j |x_j|
// saves one VALU op per element but cancels in both cases).
//
// Pre-pass (indexer_qprep_kernel), one workgroup per row, into the caller's workspace:
//   qb[r][32][128] bf16: q~_j (exact);
//   sw[r/32][32][r%32] fp32: s_j, laid out as the GEMM's LDS weight tile.
//
// GEMM workgroup tile: 32 query rows x 256 tokens (4 pages); wave w owns page w (64
// tokens, two 32-token MFMA columns).  The key fragments are decoded once per tile and
// stay in registers for all 32 heads.  Query tiles move global -> LDS by direct LDS loads
// two heads at a time (double buffered, no VALU, 16-B chunks XOR-swizzled by row so the
// MFMA operand reads are conflict-free).  Per head pair: four 8-MFMA chains, each after
// the first interleaved with the accumulation of the one before it.  Lane (column n, half
// h) at K-step s holds dims [64h + 8s, 64h + 8s + 8) of both operands.  Grid order is
// row-block-major, so a row block's 288 KB of query tiles stays in L2 while its token
// tiles stream past.  Rows of one tile that belong to different requests are handled one
// request at a time with masked stores.
#include <math.h>

#include "dsa_device.hpp"
#include "dsa_kernels.hpp"

namespace dsa {

namespace {

constexpr int kGRows = 32;
constexpr int kGWaves = 4;
constexpr int kGTokWG = kGWaves * kPage;         // 256
constexpr int kKB = 132;                         // FP8 key row
constexpr int kKPB = kPage * kKB;                // 8448
constexpr int kChunks = kKPB / 16;               // 528
constexpr int kPer = (kChunks + 63) / 64;        // 9 16-byte chunks per lane, the last partial
constexpr int kPageLds = kPer * 1024;            // a wave's page region, padded to whole loads
constexpr int kQbHeads = kIdxHeads;              // 32
constexpr int kGroup = 4;                        // heads staged per barrier
constexpr int kGroups = kQbHeads / kGroup;       // 8
constexpr int kHeadTile = kGRows * kIdxDim;      // bf16 per staged head tile (8 KB)
static_assert(kGroup * kHeadTile * 2 <= kGWaves * kPageLds, "query buffer 1 fits in the page region");
constexpr int64_t kQbRow = (int64_t)kQbHeads * kIdxDim;  // bf16 per workspace row

// ---- pre-pass: sign-folded bf16 queries and weights for one row ----
__global__ __launch_bounds__(256) void indexer_qprep_kernel(const ScoreArgs a, uint16_t *qb, float *sw) {
  const int r = blockIdx.x, t = threadIdx.x, j = t >> 3, d0 = 16 * (t & 7);
  const float qs = a.q_scale[(int64_t)r * kIdxHeads + j];
  const float s = a.w[(int64_t)r * kIdxHeads + j] * fabsf(qs);
  const u32x4_t raw = *reinterpret_cast<const u32x4_t *>(static_cast<const uint8_t *>(a.q) +
                                                         ((int64_t)r * kIdxHeads + j) * kIdxDim + d0);
  u32x4_t x0 = __builtin_bit_cast(u32x4_t, e4m3x8_bf16(raw[0], raw[1]));
  u32x4_t x1 = __builtin_bit_cast(u32x4_t, e4m3x8_bf16(raw[2], raw[3]));
  if (qs < 0.0f) {
    x0 ^= 0x80008000u;
    x1 ^= 0x80008000u;
  }
  uint16_t *dst = qb + (int64_t)r * kQbRow + (int64_t)j * kIdxDim + d0;
  *reinterpret_cast<u32x4_t *>(dst) = x0;
  *reinterpret_cast<u32x4_t *>(dst + 8) = x1;
  if ((t & 7) == 0) sw[((int64_t)(r / kGRows) * kIdxHeads + j) * kGRows + r % kGRows] = s;
}

// ---- GEMM ----
__global__ __launch_bounds__(256, 2) void indexer_gemm_kernel(const ScoreArgs a, const int n_tok_tiles,
                                                              const uint16_t *qb, const float *sw) {
  // query tiles are double buffered four heads at a time; buffer 1 shares its LDS with the
  // key pages, which are read only once per tile (to decode the key fragments)
  __shared__ __align__(16) uint16_t s_q0[kGroup * kHeadTile];    // [head of the group][row][dim], swizzled
  __shared__ __align__(16) uint8_t s_pg[kGWaves * kPageLds];     // key pages, then query buffer 1
  __shared__ __align__(16) float s_w[kIdxHeads][kGRows];         // s_j, [head][row]
  __shared__ int s_len[kGRows];

  const int tile = blockIdx.x % n_tok_tiles;
  const int rb = blockIdx.x / n_tok_tiles, row0 = rb * kGRows;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int n = lane & 31, h = lane >> 5;
  const int64_t max_tok = a.ld < a.off_ld * kPage ? a.ld : a.off_ld * kPage;
  const bool report = tile == 0;

  typedef void __attribute__((address_space(1))) gvoid;
  typedef void __attribute__((address_space(3))) lvoid;
  auto qbuf = [&](int buf) -> uint16_t * { return buf ? reinterpret_cast<uint16_t *>(s_pg) : s_q0; };
  // the block's workspace rows as a buffer: rows past n_q are out of range and read as zero
  const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(qb + (int64_t)row0 * kQbRow), 0, (int)(min(kGRows, a.n_q - row0) * kQbRow * 2), 0x00020000);
  // query tiles of heads 4g .. 4g+3 -> buffer g & 1: wave w stages head 4g + w with eight
  // direct LDS loads of 4 rows; the lane for row m, LDS chunk c' fetches chunk c' ^ (m & 15)
  auto stage = [&](int g) {
    uint16_t *dst = qbuf(g & 1) + wid * kHeadTile;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int m = 4 * i + (lane >> 4);
      const int voff = 2 * (m * (int)kQbRow + wid * kIdxDim + 8 * ((lane & 15) ^ (m & 15)));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(qrs, (lvoid *)(dst + 4 * i * kIdxDim), 16, voff, 2 * kGroup * g * kIdxDim,
                                               0, 0);
    }
  };
  // the weight tile (4 KB, one 1-KB load per wave) and the first head pair go out before
  // anything is waited on
  __builtin_amdgcn_global_load_lds((const gvoid *)(sw + (int64_t)rb * kIdxHeads * kGRows + 256 * wid + 4 * lane),
                                   (lvoid *)&s_w[8 * wid][0], 16, 0, 0);
  stage(0);

  // rows of the block: lane m < 32 of every wave holds row m's request and length
  int my_req = -1, my_len = 0;
  if (lane < kGRows) {
    const int r = row0 + lane;
    if (r < a.n_q) {
      const int b = a.q_req[r];
      int len = a.row_len[r];
      uint32_t e = 0;
      if (b < 0 || b >= a.n_req) e |= DSA_DEVERR_REQUEST; else my_req = b;
      if (len < 0 || len > max_tok) {
        e |= DSA_DEVERR_ROW_LEN;
        len = len < 0 ? 0 : (int)max_tok;
      }
      if (e && report && wid == 0) flag_error(a.err, e);
      my_len = my_req >= 0 ? len : 0;
    }
    if (wid == 0) s_len[lane] = my_len;
  }
  uint32_t todo = (uint32_t)__ballot(lane < kGRows && my_req >= 0);
  bool first = true;

  while (todo) {
    const int b = __builtin_amdgcn_readlane(my_req, __ffs(todo) - 1);
    const bool mine = lane < kGRows && my_req == b;
    const uint32_t rows = (uint32_t)__ballot(mine);
    const int lmax = (int)wave_max_u32(mine ? (uint32_t)my_len : 0u);
    const int lmin = (int)wave_min_u32(mine ? (uint32_t)my_len : 0xFFFFFFFFu);
    todo &= ~rows;
    if (tile * kGTokWG >= lmax) continue;  // uniform: the tile lies past every row's length
    if (!first) stage(0);  // a second request in this tile restarts the head loop
    first = false;

    // (1) this wave's key page -> LDS, all nine chunk loads in flight at once
    const int wtok0 = tile * kGTokWG + wid * kPage;
    bool page_ok = false;
    if (wtok0 < lmax) {
      int64_t off = a.key_off[(int64_t)b * a.off_ld + wtok0 / kPage];
      // one page per wave: the offset is wave-uniform, so the descriptor lives in SGPRs
      off = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(off >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((int)off));
      if (off < 0 || off + kKPB > a.pool_bytes || (off & 15)) {
        if (lane == 0) flag_error(a.err, DSA_DEVERR_PAGE_OFFSET);
      } else {
        page_ok = true;
        // the descriptor's range (one page) zero-fills the tail of the last load, which
        // lands in the region's padding
        const __amdgpu_buffer_rsrc_t rsrc =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(a.pool + off), 0, kKPB, 0x00020000);
        u32x4_t pg[kPer];
#pragma unroll
        for (int i = 0; i < kPer; ++i) pg[i] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, 16 * lane + 1024 * i, 0, 0);
#pragma unroll
        for (int i = 0; i < kPer; ++i) *reinterpret_cast<u32x4_t *>(s_pg + wid * kPageLds + 16 * lane + 1024 * i) = pg[i];
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the direct LDS loads (weights, group 0) landed
    __syncthreads();

    // (2) key fragments, decoded once, resident for all heads
    bf16x8_t bf[2][8];
    float ks[2], lo[2], hi[2];
    f32x16_t acc[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const uint8_t *kr = s_pg + wid * kPageLds + (32 * c + n) * kKB;
#pragma unroll
      for (int s = 0; s < 8; ++s)
        bf[c][s] = e4m3x8_bf16(*reinterpret_cast<const uint32_t *>(kr + 64 * h + 8 * s),
                               *reinterpret_cast<const uint32_t *>(kr + 64 * h + 8 * s + 4));
      ks[c] = *reinterpret_cast<const float *>(kr + 128);
      lo[c] = ks[c] < 0.0f ? -INFINITY : 0.0f;
      hi[c] = ks[c] < 0.0f ? 0.0f : INFINITY;
      acc[c] = f32x16_t{};
    }

    __syncthreads();  // every wave has its key fragments: the page region becomes query buffer 1
    stage(1);

    bf16x8_t af[8];
    auto load_af = [&](int buf, int hh) {
      const uint16_t *row = qbuf(buf) + hh * kHeadTile + n * kIdxDim;
#pragma unroll
      for (int s = 0; s < 8; ++s) af[s] = *reinterpret_cast<const bf16x8_t *>(row + 8 * ((8 * h + s) ^ (n & 15)));
    };
    auto chain = [&](int c, f32x16_t x) {
#pragma unroll
      for (int s = 0; s < 8; ++s) x = mfma_32x32x16_bf16(af[s], bf[c][s], x);
      return x;
    };
    auto load_w = [&](float *wv, int j) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4_t t4 = *reinterpret_cast<const f32x4_t *>(&s_w[j][8 * q4 + 4 * h]);
#pragma unroll
        for (int i = 0; i < 4; ++i) wv[4 * q4 + i] = t4[i];
      }
    };
    auto accum = [&](int c, const f32x16_t &x, const float *wv) {
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[c][i] = fmaf(wv[i], __builtin_amdgcn_fmed3f(x[i], lo[c], hi[c]), acc[c][i]);
    };
    auto interleave = [] {
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // four VALU
      }
    };

    // (3) the 32 heads, four per barrier: acc accumulates s_j med3(x_j).  Chain i of a group
    // is (head i/2, column i%2); each chain after the first overlaps the accumulation of the
    // one before it.
    for (int g = 0; g < kGroups; ++g) {
      const int buf = g & 1;
      if (g > 0 && g + 1 < kGroups) stage(g + 1);
      if (page_ok) {
        // one set of weights: head hd's are read last by the accumulation that overlaps
        // chain 2hd+2, just before head hd+1's are loaded
        float wv[16];
        load_af(buf, 0);
        load_w(wv, kGroup * g);
        f32x16_t xp = chain(0, f32x16_t{});
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 1; i < 2 * kGroup; ++i) {
          const int hd = i >> 1, c = i & 1, cp = (i - 1) & 1;
          if (c == 0) load_af(buf, hd);
          if (c == 1 && hd > 0) load_w(wv, kGroup * g + hd);
          const f32x16_t xn = chain(c, f32x16_t{});
          accum(cp, xp, wv);
          interleave();
          __builtin_amdgcn_sched_barrier(0);
          xp = xn;
        }
        accum(1, xp, wv);
      }
      __builtin_amdgcn_s_waitcnt(0x0F70);  // the next group's tiles have landed in LDS
      __syncthreads();
    }

    // (4) store ks * acc: element i is row 8*(i/4) + 4h + i%4, token wtok0 + 32c + n.  The
    // stores are non-temporal, so that the scores streaming out do not evict from L2 the key
    // pages the next row blocks read again
    if (page_ok) {
      // row addresses are formed here, not hoisted out of the request loop where 16 of
      // them would hold 32 VGPRs through the head loop
      int64_t ld = a.ld;
      uint32_t rws = rows;
      int h4 = 4 * h;
      asm volatile("" : "+s"(ld), "+s"(rws), "+v"(h4));
      float *const out = a.scores + (int64_t)row0 * ld;
      // the block's score rows as a buffer (32 ld floats fit 32-bit offsets, checked at
      // launch): a lane offset for (row 4h, token t) plus a scalar offset per row step
      const __amdgpu_buffer_rsrc_t ors = __builtin_amdgcn_make_buffer_rsrc(out, 0, 0x7FFFFFFF, 0x00020000);
      const int ld32 = (int)ld;
      // the common case: every row of the block is this request's and the wave's 64 tokens
      // lie below every row's length, so no element needs a mask
      const bool whole = rws == 0xFFFFFFFFu && wtok0 + kPage <= lmin;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int t = wtok0 + 32 * c + n;
        if (whole) {
          const int voff = 4 * (h4 * ld32 + t);
#pragma unroll
          for (int i = 0; i < 16; ++i)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(ks[c] * acc[c][i]), ors, voff,
                                                  4 * (8 * (i >> 2) + (i & 3)) * ld32, 2 /* nt */);
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int m = 8 * (i >> 2) + h4 + (i & 3);
            if (((rws >> m) & 1u) && t < s_len[m]) __builtin_nontemporal_store(ks[c] * acc[c][i], &out[m * ld + t]);
          }
        }
      }
    }
    __syncthreads();  // s_page / s_q are refilled for the next request of this tile
  }
  // no direct LDS load may still be in flight when the workgroup's LDS is released: a tile
  // whose every request was skipped never waited for the prologue's loads
  if (first) __builtin_amdgcn_s_waitcnt(0x0F70);
}

// ---- exact rescoring of the band tokens of the FP8 prefill path ----
// The score of (row r, token t) exactly as indexer_gemm_kernel computes it: the same bf16
// operands, the same MFMA chain over the same K order (lane (column n, half h) at K-step s holds
// dims [64h + 8s, 64h + 8s + 8)), and the same fp32 epilogue, sequential over heads 0..31.  Here
// the MFMA's 32 rows are the 32 heads of row r and its 32 columns are 32 listed tokens; an
// element of the product depends only on its own row and column, so every x_j is the GEMM's
// bit for bit.  One wave per workgroup; grid (n_q, kRescoreY), tiles of 32 band tokens strided
// over y (every token of the row when the band overflowed).
constexpr int kRescoreY = 4;

__global__ __launch_bounds__(64) void band_rescore_kernel(const RescoreArgs a) {
  const int r = blockIdx.x, lane = threadIdx.x, n = lane & 31, h = lane >> 5;
  const int nl = a.band.cnt[2 * r], nb = a.band.cnt[2 * r + 1];
  if (nl < 0) return;  // the whole row was kept
  const int b = a.q_req[r];
  if (b < 0 || b >= a.n_req) return;  // flagged by the GEMM
  const int64_t max_tok = a.ld < a.off_ld * kPage ? a.ld : a.off_ld * kPage;
  const int len = (int)min((int64_t)max(a.row_len[r], 0), max_tok);
  const bool full = nb > kBandCap;
  const int ntok = full ? len : nb;
  const int tiles = (ntok + 31) / 32;
  if ((int)blockIdx.y >= tiles) return;

  // the row's 32 heads as the A operand: lane (head n, half h)
  const uint16_t *qrow = a.qb + (int64_t)r * kQbRow + n * kIdxDim + 64 * h;
  bf16x8_t af[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) af[s] = *reinterpret_cast<const bf16x8_t *>(qrow + 8 * s);
  const float *swr = a.sw + (int64_t)(r / kGRows) * kIdxHeads * kGRows + r % kGRows;  // s_j at swr[32 j]
  uint2 *list = a.band.list + (int64_t)r * kBandListCap;
  const uint2 *bpos = a.band.pos + (int64_t)r * kBandCap;
  const int64_t *koff = a.key_off + (int64_t)b * a.off_ld;
  const int lim = min(nl, kBandListCap);

  // two tiles per round (q and q + gridDim.y), their dependent loads interleaved: column n of
  // tile u is the token t[u] (list position p[u] in band mode)
  for (int q0 = blockIdx.y; q0 < tiles; q0 += 2 * gridDim.y) {
    int t[2], p[2];
    bool valid[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int bi = 32 * (q0 + u * (int)gridDim.y) + n;
      valid[u] = bi < ntok;
      t[u] = 0;
      p[u] = 0;
      if (valid[u]) {
        if (full) {
          t[u] = bi;
        } else {
          const uint2 e = bpos[bi];
          p[u] = (int)e.x;
          t[u] = (int)e.y;
          valid[u] = p[u] >= 0 && p[u] < lim;
        }
      }
      valid[u] = valid[u] && t[u] >= 0 && t[u] < len;
    }
    int64_t off[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) off[u] = valid[u] ? koff[t[u] >> 6] : -1;
    bf16x8_t bfr[2][8];
    float ks[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      valid[u] = valid[u] && off[u] >= 0 && off[u] + kKPB <= a.pool_bytes && (off[u] & 15) == 0;
      ks[u] = 0.0f;
      if (valid[u]) {
        const uint8_t *kr = a.pool + off[u] + (t[u] & (kPage - 1)) * kKB;
#pragma unroll
        for (int s = 0; s < 8; ++s)
          bfr[u][s] = e4m3x8_bf16(*reinterpret_cast<const uint32_t *>(kr + 64 * h + 8 * s),
                                  *reinterpret_cast<const uint32_t *>(kr + 64 * h + 8 * s + 4));
        ks[u] = *reinterpret_cast<const float *>(kr + 128);
      } else {
#pragma unroll
        for (int s = 0; s < 8; ++s) bfr[u][s] = bf16x8_t{};
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      f32x16_t x = f32x16_t{};
#pragma unroll
      for (int s = 0; s < 8; ++s) x = mfma_32x32x16_bf16(af[s], bfr[u][s], x);
      // element i of lane (n, h) is head 8 (i / 4) + 4h + i % 4: lanes n < 32 take the other half's
      float xo[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const auto sw2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x[i]), __float_as_uint(x[i]), false, false);
        xo[i] = __uint_as_float(sw2[1]);
      }
      if (h == 0 && valid[u]) {
        const float lo = ks[u] < 0.0f ? -INFINITY : 0.0f, hi = ks[u] < 0.0f ? 0.0f : INFINITY;
        float acc = 0.0f;
#pragma unroll
        for (int j = 0; j < kIdxHeads; ++j) {
          const int i = 4 * (j >> 3) + (j & 3);
          const float xj = (j & 4) ? xo[i] : x[i];
          acc = fmaf(swr[kGRows * j], __builtin_amdgcn_fmed3f(xj, lo, hi), acc);
        }
        const float sc = ks[u] * acc;
        if (full) a.scores[(int64_t)r * a.ld + t[u]] = sc;
        else list[p[u]].x = score_key(sc);
      }
    }
  }
}

}  // namespace

hipError_t launch_band_rescore(const RescoreArgs &a, hipStream_t s) {
  if (a.n_q == 0) return hipSuccess;
  if (a.band.e == nullptr) return hipErrorInvalidValue;
  hipLaunchKernelGGL(band_rescore_kernel, dim3(a.n_q, kRescoreY), dim3(64), 0, s, a);
  return hipGetLastError();
}

size_t indexer_gemm_workspace_bytes(int32_t n_q) {
  if (n_q <= 0) return 0;
  const int64_t qb = ((int64_t)n_q * kQbRow * 2 + 255) & ~int64_t(255);
  const int64_t sw = (int64_t)((n_q + kGRows - 1) / kGRows) * kIdxHeads * kGRows * 4;
  return (size_t)(qb + sw);
}

hipError_t launch_indexer_gemm(const ScoreArgs &a, hipStream_t s) {
  if (a.n_q == 0) return hipSuccess;
  if (a.key_fmt != 0 || a.ws == nullptr) return hipErrorInvalidValue;
  const int64_t max_tok = a.ld < a.off_ld * kPage ? a.ld : a.off_ld * kPage;
  const int64_t n_tok_tiles = (max_tok + kGTokWG - 1) / kGTokWG;
  const int64_t n_row_blocks = (a.n_q + kGRows - 1) / kGRows;
  const int64_t grid = n_tok_tiles * n_row_blocks;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  if ((int64_t)kGRows * a.ld * 4 > 0x7FFFFFFF) return hipErrorInvalidValue;  // 32-bit store offsets
  uint16_t *qb = static_cast<uint16_t *>(a.ws);
  float *sw = reinterpret_cast<float *>(static_cast<uint8_t *>(a.ws) +
                                        (((int64_t)a.n_q * kQbRow * 2 + 255) & ~int64_t(255)));
  hipLaunchKernelGGL(indexer_qprep_kernel, dim3(a.n_q), dim3(256), 0, s, a, qb, sw);
  if (grid == 0) return hipGetLastError();
  hipLaunchKernelGGL(indexer_gemm_kernel, dim3((unsigned)grid), dim3(256), 0, s, a, (int)n_tok_tiles, qb, sw);
  return hipGetLastError();
}

}  // namespace dsa
