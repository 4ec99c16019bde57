// indexer_gemm_fp8.hip -- prefill indexer on FP8 MFMA, with the bound an exact top-k needs.
//
// Page "vLLM 为 Kimi K3.1 Pro 提供 Day-0 支持":
//  * section "低延迟解码：融合的 DSA 解码路径": the indexer query is quantised to FP8 (its scale
//    folded into the head weights), so the scores are defined on e4m3 query and key codes;
//  * section "预填充：上下文并行稀疏注意力": each row is scored against the full context and
//    its top-k selected directly.
// The bf16 GEMM (indexer_gemm.hip) is exact to fp32 rounding.  This one feeds the raw e4m3
// codes of both operands to v_mfma_scale_f32_32x32x64_f8f6f4 (unit scales).  How that
// instruction sums, as measured on gfx950 (one large product against small ones placed at
// chosen dims, and both signs): the 64 products of one instruction form 8 groups of 8
// consecutive K; within a group every product is cut toward zero to a multiple of
// 2^(E - 13), E the exponent of the group's largest |product|; the group sums then add up
// (and onto the accumulator) at fp32 precision.  A product of two e4m3 values has at most 8
// significant bits, so the largest product of a group is exact and each of the other seven
// loses less than 2^(E - 13):
//   |x^ - x| < 7 * 2^-13 * sum_g max_{d in g} |q~_d k_d|  (+ fp32 rounding)
// for one head.
//
// The epilogue splits the ReLU: with s_j = w_j |qs_j| and sigma = sign(ks),
//   score = ks sum_j s_j ReLU-part(x_j) = |ks| / 2 * (sigma L + S),
//   L = sum_j s_j x_j = q_lin . k,   q_lin = sum_j s_j q~_j,   S = sum_j s_j |x_j|.
// L runs on bf16 MFMA with q_lin as two bf16 parts (hi + lo, 2^-18 relative) against the keys
// decoded from the fragments; it seeds the accumulators, and each head then costs one fma
// with |x| (an operand modifier) per element instead of a med3 and an fma.  Only S carries the
// FP8 truncation, so with |q~_d k_d| <= max_{g} |q~| * max_{g} |k|:
//   |s^ - s| <= delta * sum_g U_rg * A_tg,  U_rg = sum_j s_j max_{d in g} |q~_jd|,
//                                         A_tg = |ks_t| max_{d in g} |k_td|,
// and for the whole row E_r = delta * sum_g U_rg M_bg with M_bg = max_t A_tg over the
// request's tokens.  delta = 5.5 * 2^-13 covers half the 7 * 2^-13 above, the q_lin parts, the
// fp32 rounding of the group sums, of the accumulation (which starts at |L|) and of the bf16
// path's own sums, with a margin.  The top-k kernels in band mode use E_r to find the tokens
// whose order it could change and rescore those exactly.  (Exact zeros are not kept: a token no
// head scores positive comes out as a small residue, inside the bound.)
//
// Kernels:
//   indexer_qprep_fp8_kernel  one workgroup per row: the bf16 q~ (for exact rescoring), the
//                             e4m3 q~ codes, s_j as the GEMM's weight tile, q_lin and U_r;
//   key_bound_kernel          one wave per key page: the page's group maxima of A_tg;
//   key_bound_reduce_kernel   one workgroup per request: M_b over its pages;
//   indexer_gemm_fp8_kernel   the GEMM: 32 query rows x 256 tokens per workgroup, as the bf16
//                             kernel, with the key fragments kept as raw e4m3 bytes (no decode)
//                             and 2 MFMAs per (head, 32 tokens) instead of 8; tile 0 of each
//                             row block writes E_r.
// Lane (column n, half h) at K-step s holds dims [64s + 32h, 64s + 32h + 32) of both
// operands (the f8f6f4 32x32x64 operand layout: 32 one-byte elements per lane).
#include <math.h>

#include "dsa_device.hpp"
#include "dsa_kernels.hpp"

namespace dsa {

namespace {

constexpr int kGRows = 32;
// cache policy of the score stores: non-temporal (the nt bit), so that the scores streaming
// out do not evict from L2 the key pages the next row blocks read again
constexpr int kStoreNT = 2;
constexpr int kGWaves = 4;
constexpr int kGTokWG = kGWaves * kPage;   // 256
constexpr int kKB = 132;                   // FP8 key row
constexpr int kKPB = kPage * kKB;          // 8448
constexpr int kPer = (kKPB / 16 + 63) / 64;  // 9 16-byte chunks per lane, the last partial
constexpr int kPageLds = kPer * 1024;      // a wave's page region, padded to whole loads
constexpr int kGroup = 4;                  // heads staged per barrier
constexpr int kGroups = kIdxHeads / kGroup;  // 8
constexpr int kGroups8 = kIdxDim / 8;        // 16 K-groups of 8 dims (the FP8 MFMA's summation groups)
constexpr int kHeadTileB = kGRows * kIdxDim;  // bytes per staged e4m3 head tile (4 KB)
static_assert(kGroup * kHeadTileB <= kGWaves * kPageLds, "query buffer 1 fits in the page region");

// ---- pre-pass: one workgroup per row ----
// |bf16| maximum of the 8 values of a 16-byte group (as bits: non-negative, so integer order;
// a NaN orders above +inf)
__device__ __forceinline__ uint32_t absmax8_bits(u32x4_t v) {
  uint32_t m = 0u;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t a = v[i] & 0x7FFF7FFFu;
    m = max(m, max(a >> 16, a & 0xFFFFu));
  }
  return m << 16;
}

__global__ __launch_bounds__(256) void indexer_qprep_fp8_kernel(const ScoreArgs a, PrefillWs ws) {
  const int r = blockIdx.x, t = threadIdx.x, j = t >> 3, d0 = 16 * (t & 7);
  __shared__ float s_u[kIdxHeads][kGroups8 + 1];  // s_j max_{d in g} |q~_jd|, [head][group]
  __shared__ float s_lin[kIdxHeads][kIdxDim + 4];  // s_j q~_jd
  const float qs = a.q_scale[(int64_t)r * kIdxHeads + j];
  const float s = a.w[(int64_t)r * kIdxHeads + j] * fabsf(qs);
  u32x4_t raw = *reinterpret_cast<const u32x4_t *>(static_cast<const uint8_t *>(a.q) +
                                                   ((int64_t)r * kIdxHeads + j) * kIdxDim + d0);
  u32x4_t x0 = __builtin_bit_cast(u32x4_t, e4m3x8_bf16(raw[0], raw[1]));  // group 2 (t & 7)
  u32x4_t x1 = __builtin_bit_cast(u32x4_t, e4m3x8_bf16(raw[2], raw[3]));  // group 2 (t & 7) + 1
  s_u[j][2 * (t & 7)] = s * __uint_as_float(absmax8_bits(x0));
  s_u[j][2 * (t & 7) + 1] = s * __uint_as_float(absmax8_bits(x1));
  if (qs < 0.0f) {  // q~ = sign(qs) code: flip the sign bits (exact)
    x0 ^= 0x80008000u;
    x1 ^= 0x80008000u;
    raw ^= 0x80808080u;
  }
  uint16_t *dst = ws.qb + (int64_t)r * kIdxHeads * kIdxDim + (int64_t)j * kIdxDim + d0;
  *reinterpret_cast<u32x4_t *>(dst) = x0;
  *reinterpret_cast<u32x4_t *>(dst + 8) = x1;
  *reinterpret_cast<u32x4_t *>(ws.qc + ((int64_t)r * kIdxHeads + j) * kIdxDim + d0) = raw;
  if ((t & 7) == 0) ws.sw[((int64_t)(r / kGRows) * kIdxHeads + j) * kGRows + r % kGRows] = s;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    s_lin[j][d0 + 2 * i] = s * __uint_as_float(x0[i] << 16);
    s_lin[j][d0 + 2 * i + 1] = s * __uint_as_float(x0[i] & 0xFFFF0000u);
    s_lin[j][d0 + 8 + 2 * i] = s * __uint_as_float(x1[i] << 16);
    s_lin[j][d0 + 8 + 2 * i + 1] = s * __uint_as_float(x1[i] & 0xFFFF0000u);
  }
  __syncthreads();
  if (t < kGroups8) {
    float u = 0.0f;
    for (int i = 0; i < kIdxHeads; ++i) u += s_u[i][t];
    ws.urow[(int64_t)r * kGroups8 + t] = u;
  }
  if (t < kIdxDim) {  // q_lin[d] = sum_j s_j q~_jd as bf16 hi + lo
    float q = 0.0f;
    for (int i = 0; i < kIdxHeads; ++i) q += s_lin[i][t];
    const __bf16 hi = (__bf16)q;
    const __bf16 lo = (__bf16)(q - (float)hi);
    ws.qlin[(int64_t)r * 2 * kIdxDim + t] = __builtin_bit_cast(uint16_t, hi);
    ws.qlin[(int64_t)r * 2 * kIdxDim + kIdxDim + t] = __builtin_bit_cast(uint16_t, lo);
  }
}

// ---- key bound: A_tg = |ks_t| max_{d in g} |k_td|, its maximum per page, then per request ----
// Tokens at or past the request's length do not count: a page's unused slots may hold anything.
__global__ __launch_bounds__(256) void key_bound_kernel(const ScoreArgs a, PrefillWs ws, const int32_t *ctx_len,
                                                        int max_pages) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int b = blockIdx.y, p = blockIdx.x * 4 + wid;
  if (p >= max_pages) return;
  const int64_t off = a.key_off[(int64_t)b * a.off_ld + p];
  uint32_t gm[kGroups8];
#pragma unroll
  for (int g = 0; g < kGroups8; ++g) gm[g] = 0u;
  if ((int64_t)p * kPage + lane < ctx_len[b] && off >= 0 && off + kKPB <= a.pool_bytes && (off & 15) == 0) {
    const uint8_t *row = a.pool + off + lane * kKB;  // lane = token of the page
    const float ks = fabsf(*reinterpret_cast<const float *>(row + kIdxDim));
#pragma unroll
    for (int g = 0; g < kGroups8; ++g) {
      const uint32_t lo = *reinterpret_cast<const uint32_t *>(row + 8 * g);
      const uint32_t hi = *reinterpret_cast<const uint32_t *>(row + 8 * g + 4);
      const u32x4_t v = __builtin_bit_cast(u32x4_t, e4m3x8_bf16(lo, hi));
      const float m = ks * __uint_as_float(absmax8_bits(v));
      gm[g] = m <= 3.0e38f ? __float_as_uint(m) : 0x7F800000u;  // NaN or overflow: +inf
    }
  }
  float *out = ws.mpage + ((int64_t)b * a.off_ld + p) * kGroups8;
#pragma unroll
  for (int g = 0; g < kGroups8; ++g) {
    const uint32_t m = wave_max_u32(gm[g]);  // non-negative: integer order
    if (lane == g) out[g] = __uint_as_float(m);
  }
}

__global__ __launch_bounds__(256) void key_bound_reduce_kernel(const ScoreArgs a, PrefillWs ws, int max_pages) {
  __shared__ uint32_t s_m[4][kGroups8];
  const int b = blockIdx.x, lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  uint32_t m[kGroups8];
#pragma unroll
  for (int g = 0; g < kGroups8; ++g) m[g] = 0u;
  for (int p = threadIdx.x; p < max_pages; p += 256) {
    const float *src = ws.mpage + ((int64_t)b * a.off_ld + p) * kGroups8;
#pragma unroll
    for (int g = 0; g < kGroups8; ++g) m[g] = max(m[g], __float_as_uint(src[g]));
  }
#pragma unroll
  for (int g = 0; g < kGroups8; ++g) {
    const uint32_t x = wave_max_u32(m[g]);
    if (lane == g) s_m[wid][g] = x;
  }
  __syncthreads();
  if (threadIdx.x < kGroups8) {
    const int g = threadIdx.x;
    ws.mreq[(int64_t)b * kGroups8 + g] = __uint_as_float(max(max(s_m[0][g], s_m[1][g]), max(s_m[2][g], s_m[3][g])));
  }
}

// ---- GEMM ----
// MODE 0: every tile.  MODE 1: only the kSampleTiles sampled tiles of each row block (the
// scores the tile-est kernel draws thresholds from).  MODE 2: every tile, and each long row's
// scores at or above its threshold are appended, in token order, to the row's list for the
// tile (the lists the band top-k selects from instead of re-reading the scores).
template <int MODE>
__global__ __launch_bounds__(256, 2) void indexer_gemm_fp8_kernel(const ScoreArgs a, const int n_tok_tiles,
                                                                  PrefillWs ws, const int32_t *ctx_len) {
  // query tiles (e4m3 codes) are double buffered four heads at a time; buffer 1 shares its LDS
  // with the key pages, which are read only once per tile (to load the key fragments)
  __shared__ __align__(16) uint8_t s_q0[kGroup * kHeadTileB];   // [head of the group][row][128 B], swizzled
  __shared__ __align__(16) uint8_t s_pg[kGWaves * kPageLds];    // key pages, then query buffer 1, then scores
  __shared__ __align__(16) float s_w[kIdxHeads][kGRows];        // s_j, [head][row]
  __shared__ int s_len[kGRows];
  __shared__ float s_ef[kGRows];   // MODE 2: each row's threshold as a float
  __shared__ uint32_t s_emit;      // MODE 2: rows that keep lists
  __shared__ int s_pok[kGWaves];   // MODE 2: the wave's page was read

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int n = lane & 31, h = lane >> 5;
  const int64_t max_tok = a.ld < a.off_ld * kPage ? a.ld : a.off_ld * kPage;
  int tile, rb;
  if constexpr (MODE == 1) {
    rb = blockIdx.x / kSampleTiles;
    // the block's longest row, clamped to [0, ld] (the tile-est kernel computes the same)
    uint32_t lm = 0u;
    if (lane < kGRows && rb * kGRows + lane < a.n_q) {
      const int64_t l = a.row_len[rb * kGRows + lane];
      lm = (uint32_t)(l < 0 ? 0 : (l > a.ld ? a.ld : l));
    }
    lm = wave_max_u32(lm);
    tile = sample_tile(blockIdx.x % kSampleTiles, lm);
    if (tile < 0 || (int64_t)tile * kGTokWG >= max_tok) return;  // nothing in flight yet
  } else {
    tile = blockIdx.x % n_tok_tiles;
    rb = blockIdx.x / n_tok_tiles;
  }
  const int row0 = rb * kGRows;
  const bool report = MODE == 1 ? blockIdx.x % kSampleTiles == 0 : tile == 0;

  typedef void __attribute__((address_space(1))) gvoid;
  typedef void __attribute__((address_space(3))) lvoid;
  auto qbuf = [&](int buf) -> uint8_t * { return buf ? s_pg : s_q0; };
  // the block's code rows as a buffer: rows past n_q are out of range and read as zero
  const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc(
      ws.qc + (int64_t)row0 * kIdxHeads * kIdxDim, 0, (int)(min(kGRows, a.n_q - row0) * kIdxHeads * kIdxDim), 0x00020000);
  // head tiles 4g .. 4g+3 -> buffer g & 1: wave w stages head 4g + w with four direct LDS loads
  // of 8 rows; the lane for row m, LDS chunk c' fetches chunk c' ^ (m & 7)
  auto stage = [&](int g) {
    uint8_t *dst = qbuf(g & 1) + wid * kHeadTileB;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 8 * i + (lane >> 3);
      const int voff = m * kIdxHeads * kIdxDim + (kGroup * g + wid) * kIdxDim + 16 * ((lane & 7) ^ (m & 7));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(qrs, (lvoid *)(dst + 1024 * i), 16, voff, 0, 0, 0);
    }
  };
  __builtin_amdgcn_global_load_lds((const gvoid *)(ws.sw + (int64_t)rb * kIdxHeads * kGRows + 256 * wid + 4 * lane),
                                   (lvoid *)&s_w[8 * wid][0], 16, 0, 0);
  stage(0);

  int my_req = -1, my_len = 0;
  if (lane < kGRows) {
    const int r = row0 + lane;
    if (r < a.n_q) {
      const int b = a.q_req[r];
      int len = a.row_len[r];
      uint32_t e = 0;
      if (b < 0 || b >= a.n_req) e |= DSA_DEVERR_REQUEST; else my_req = b;
      // the key bound covers the request's first ctx_len tokens only
      const int64_t lim = my_req >= 0 && ctx_len[b] < max_tok ? ctx_len[b] : max_tok;
      if (len < 0 || len > lim) {
        e |= DSA_DEVERR_ROW_LEN;
        len = len < 0 ? 0 : (int)max(lim, (int64_t)0);
      }
      if (e && report && wid == 0) flag_error(a.err, e);
      my_len = my_req >= 0 ? len : 0;
      if (report && wid == 0) {  // E_r = delta sum_g U_rg M_bg
        float e = 0.0f;
        if (my_req >= 0) {
#pragma unroll
          for (int g = 0; g < kGroups8; ++g)
            e = fmaf(ws.urow[(int64_t)r * kGroups8 + g], ws.mreq[(int64_t)b * kGroups8 + g], e);
        }
        ws.bound[r] = kFp8GroupDelta * e;
        if (ws.bound_out) ws.bound_out[r] = kFp8GroupDelta * e;
      }
    }
    if (wid == 0) s_len[lane] = my_len;
  }
  if constexpr (MODE == 2) {
    // rows that keep lists: a valid request, longer than the top-k selects whole and than k
    const bool emit = lane < kGRows && my_req >= 0 && my_len > kShortRow && ws.tiles.k < my_len;
    const uint32_t em = (uint32_t)__ballot(emit);
    if (wid == 0 && lane < kGRows) {
      const int r = row0 + lane;
      if (emit) {
        const uint32_t est = ws.tiles.est[r];
        s_ef[lane] = est == 0u ? -INFINITY : key_score(est);
      }
      // an emitting row's count for this tile is written below unless the tile lies past it
      if (r < a.n_q && (!emit || (int64_t)tile * kGTokWG >= my_len))
        ws.tiles.cnt[(int64_t)r * ws.tiles.n_tiles + tile] = 0u;
      if (lane == 0) s_emit = em;
    }
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
    if (tile * kGTokWG >= lmax) continue;
    if (!first) stage(0);
    first = false;

    // the linear part's query operand, in flight with the page: lane (row n, half h) at
    // K-step s' holds dims 64 (s'/4) + 32h + 8 (s'%4) .. +8 of q_lin's hi and lo rows (rows past
    // n_q read as zero)
    bf16x8_t la[8][2];
    {
      const __amdgpu_buffer_rsrc_t lrs = __builtin_amdgcn_make_buffer_rsrc(
          ws.qlin + (int64_t)row0 * 2 * kIdxDim, 0, (int)(min(kGRows, a.n_q - row0) * 2 * kIdxDim * 2), 0x00020000);
#pragma unroll
      for (int sp = 0; sp < 8; ++sp) {
#pragma unroll
        for (int pc = 0; pc < 2; ++pc) {
          const int voff = 2 * ((n * 2 + pc) * kIdxDim + 64 * (sp >> 2) + 32 * h + 8 * (sp & 3));
          la[sp][pc] = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(lrs, voff, 0, 0));
        }
      }
    }

    // (1) this wave's key page -> LDS
    const int wtok0 = tile * kGTokWG + wid * kPage;
    bool page_ok = false;
    if (wtok0 < lmax) {
      int64_t off = a.key_off[(int64_t)b * a.off_ld + wtok0 / kPage];
      off = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(off >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((int)off));
      if (off < 0 || off + kKPB > a.pool_bytes || (off & 15)) {
        if (lane == 0) flag_error(a.err, DSA_DEVERR_PAGE_OFFSET);
      } else {
        page_ok = true;
        const __amdgpu_buffer_rsrc_t rsrc =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(a.pool + off), 0, kKPB, 0x00020000);
        u32x4_t pg[kPer];
#pragma unroll
        for (int i = 0; i < kPer; ++i) pg[i] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, 16 * lane + 1024 * i, 0, 0);
#pragma unroll
        for (int i = 0; i < kPer; ++i) *reinterpret_cast<u32x4_t *>(s_pg + wid * kPageLds + 16 * lane + 1024 * i) = pg[i];
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();

    // (2) key fragments: raw e4m3 bytes, resident for all heads
    i32x8_t kb[2][2];
    float ks[2];
    f32x16_t acc[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const uint8_t *kr = s_pg + wid * kPageLds + (32 * c + n) * kKB;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const uint32_t *w32 = reinterpret_cast<const uint32_t *>(kr + 64 * s + 32 * h);
#pragma unroll
        for (int i = 0; i < 8; ++i) kb[c][s][i] = (int)w32[i];
      }
      ks[c] = *reinterpret_cast<const float *>(kr + 128);
    }
    __syncthreads();  // every wave has its key fragments: the page region becomes query buffer 1
    stage(1);

    // (2b) the linear part L = q_lin . k on bf16 MFMA, the keys decoded from the fragments;
    // acc starts at sign(ks) L, so that after the heads acc = sign(ks) L + sum_j s_j |x_j| and
    // the score is |ks| / 2 * acc
    if (page_ok) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        f32x16_t l = f32x16_t{};
#pragma unroll
        for (int sp = 0; sp < 8; ++sp) {
          const bf16x8_t bk = e4m3x8_bf16((uint32_t)kb[c][sp >> 2][2 * (sp & 3)], (uint32_t)kb[c][sp >> 2][2 * (sp & 3) + 1]);
          l = mfma_32x32x16_bf16(la[sp][0], bk, l);
          l = mfma_32x32x16_bf16(la[sp][1], bk, l);
        }
        const float sg = ks[c] < 0.0f ? -1.0f : 1.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[c][i] = sg * l[i];
      }
    }

    i32x8_t qa[2][2];  // [head parity][K-step]
    auto load_qa = [&](i32x8_t(&q)[2], int buf, int hh) {
      const uint8_t *row = qbuf(buf) + hh * kHeadTileB + n * kIdxDim;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int c0 = 4 * s + 2 * h;  // source chunks c0, c0 + 1 of the row
        const u32x4_t lo4 = *reinterpret_cast<const u32x4_t *>(row + 16 * (c0 ^ (n & 7)));
        const u32x4_t hi4 = *reinterpret_cast<const u32x4_t *>(row + 16 * ((c0 + 1) ^ (n & 7)));
        q[s] = i32x8_t{(int)lo4[0], (int)lo4[1], (int)lo4[2], (int)lo4[3], (int)hi4[0], (int)hi4[1], (int)hi4[2], (int)hi4[3]};
      }
    };
    auto chain = [&](const i32x8_t(&q)[2], int c) {
      f32x16_t x = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(q[0], kb[c][0], f32x16_t{}, 0, 0, 0, 0x7f, 0, 0x7f);
      return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(q[1], kb[c][1], x, 0, 0, 0, 0x7f, 0, 0x7f);
    };
    auto load_w = [&](float *wv, int j) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4_t t4 = *reinterpret_cast<const f32x4_t *>(&s_w[j][8 * q4 + 4 * h]);
#pragma unroll
        for (int i = 0; i < 4; ++i) wv[4 * q4 + i] = t4[i];
      }
    };
    auto interleave = [] {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);   // eight VALU
      }
    };
    auto accum = [&](int c, const f32x16_t &x, const float *wv) {
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[c][i] = fmaf(wv[i], fabsf(x[i]), acc[c][i]);
    };

    // (3) the 32 heads as one software pipeline of 64 chains (head j, column c), four heads
    // per barrier: each chain overlaps the accumulation of the chain before it (also across
    // a barrier), and a head's query fragments and weights are read from LDS while the chains
    // of the head before it run
    float wv[2][16];  // [head parity]
    f32x16_t xp = f32x16_t{};
    for (int g = 0; g < kGroups; ++g) {
      const int buf = g & 1;
      if (g > 0 && g + 1 < kGroups) stage(g + 1);
      if (page_ok) {
        load_qa(qa[0], buf, 0);
#pragma unroll
        for (int i = 0; i < 2 * kGroup; ++i) {
          const int hd = i >> 1, c = i & 1;
          if (c == 0) {
            if (hd + 1 < kGroup) load_qa(qa[(hd + 1) & 1], buf, hd + 1);
            load_w(wv[hd & 1], kGroup * g + hd);
          }
          const f32x16_t xn = chain(qa[hd & 1], c);
          // the chain before: column c ^ 1 of head hd - 1 + c (head 3 of the last group at i = 0)
          if (g > 0 || i > 0) accum(c ^ 1, xp, wv[((i + 7) >> 1) & 1]);
          interleave();
          __builtin_amdgcn_sched_barrier(0);
          xp = xn;
        }
      }
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the next group's tiles have landed in LDS
      __syncthreads();
    }
    if (page_ok) accum(1, xp, wv[1]);

    // (4) store ks * acc: element i is row 8*(i/4) + 4h + i%4, token wtok0 + 32c + n
    if (page_ok) {
      int64_t ld = a.ld;
      uint32_t rws = rows;
      int h4 = 4 * h;
      asm volatile("" : "+s"(ld), "+s"(rws), "+v"(h4));
      float *const out = a.scores + (int64_t)row0 * ld;
      const __amdgpu_buffer_rsrc_t ors = __builtin_amdgcn_make_buffer_rsrc(out, 0, 0x7FFFFFFF, 0x00020000);
      const int ld32 = (int)ld;
      const bool whole = rws == 0xFFFFFFFFu && wtok0 + kPage <= lmin;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int t = wtok0 + 32 * c + n;
        const float hk = 0.5f * fabsf(ks[c]);
        if (whole) {
          const int voff = 4 * (h4 * ld32 + t);
#pragma unroll
          for (int i = 0; i < 16; ++i)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(hk * acc[c][i]), ors, voff,
                                                  4 * (8 * (i >> 2) + (i & 3)) * ld32, kStoreNT);
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int m = 8 * (i >> 2) + h4 + (i & 3);
            if (((rws >> m) & 1u) && t < s_len[m]) __builtin_nontemporal_store(hk * acc[c][i], &out[m * ld + t]);
          }
        }
      }
    }
    if constexpr (MODE == 2) {
      const uint32_t em = s_emit & rows;  // this request's rows that keep lists (uniform)
      if (em) {
        // (5) the tile's scores to LDS as [32 rows][256 tokens] (the page region is free once
        // the last head group's barrier has passed)
        float *sl = reinterpret_cast<float *>(s_pg);
        if (lane == 0) s_pok[wid] = page_ok ? 1 : 0;
        if (page_ok) {
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const float hk = 0.5f * fabsf(ks[c]);
#pragma unroll
            for (int i = 0; i < 16; ++i)
              sl[(8 * (i >> 2) + 4 * h + (i & 3)) * kGTokWG + kPage * wid + 32 * c + n] = hk * acc[c][i];
          }
        }
        __syncthreads();
        // (6) thread (row m, segment g) takes tokens 32g .. 32g + 31 of the tile: the ones at or
        // above the row's threshold, ranked through a scan over the row's eight segments
        const int m = tid >> 3, g = tid & 7;
        const int t0 = tile * kGTokWG + 32 * g;
        uint32_t mask = 0u;
        if (((em >> m) & 1u) && s_pok[g >> 1]) {
          const float ef = s_ef[m];
          const int lm = s_len[m];
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const f32x4_t v = *reinterpret_cast<const f32x4_t *>(&sl[m * kGTokWG + 32 * g + 4 * q]);
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (t0 + 4 * q + e < lm && !(v[e] < ef)) mask |= 1u << (4 * q + e);
          }
        }
        const int cnt = __popc(mask);
        int incl = cnt;
#pragma unroll
        for (int dd = 1; dd < 8; dd <<= 1) {
          const int o = __shfl_up(incl, dd, 8);
          if (g >= dd) incl += o;
        }
        const int total = __shfl(incl, 7, 8);
        if ((em >> m) & 1u) {
          const int r = row0 + m;
          uint2 *dst = ws.tiles.cand + ((int64_t)r * ws.tiles.n_tiles + tile) * kTileCap;
          int pos = incl - cnt;
          while (mask) {
            const int bpos = __ffs(mask) - 1;
            mask &= mask - 1u;
            if (pos < kTileCap) dst[pos] = make_uint2(score_key(sl[m * kGTokWG + 32 * g + bpos]), (uint32_t)(t0 + bpos));
            ++pos;
          }
          if (g == 7) ws.tiles.cnt[(int64_t)r * ws.tiles.n_tiles + tile] = (uint32_t)total;
        }
      }
    }
    __syncthreads();
  }
  if (first) __builtin_amdgcn_s_waitcnt(0x0F70);
}

}  // namespace

hipError_t launch_fp8_prepass(const ScoreArgs &a, const PrefillWs &ws, const int32_t *ctx_len, int32_t max_pages,
                              hipStream_t s) {
  if (a.n_q == 0) return hipSuccess;
  if (a.key_fmt != 0 || max_pages < 0 || max_pages > a.off_ld || a.n_req > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL(indexer_qprep_fp8_kernel, dim3(a.n_q), dim3(256), 0, s, a, ws);
  if (a.n_req > 0) {
    if (max_pages > 0)
      hipLaunchKernelGGL(key_bound_kernel, dim3((max_pages + 3) / 4, a.n_req), dim3(256), 0, s, a, ws, ctx_len,
                         max_pages);
    hipLaunchKernelGGL(key_bound_reduce_kernel, dim3(a.n_req), dim3(256), 0, s, a, ws, max_pages);
  }
  return hipGetLastError();
}

hipError_t launch_fp8_gemm(const ScoreArgs &a, const PrefillWs &ws, const int32_t *ctx_len, int mode, hipStream_t s) {
  if (a.n_q == 0) return hipSuccess;
  if (a.key_fmt != 0 || mode < 0 || mode > 2) return hipErrorInvalidValue;
  const int64_t max_tok = a.ld < a.off_ld * kPage ? a.ld : a.off_ld * kPage;
  const int64_t n_tok_tiles = (max_tok + kGTokWG - 1) / kGTokWG;
  const int64_t n_row_blocks = (a.n_q + kGRows - 1) / kGRows;
  if (n_tok_tiles * n_row_blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  if ((int64_t)kGRows * a.ld * 4 > 0x7FFFFFFF) return hipErrorInvalidValue;  // 32-bit store offsets
  // the lists have one entry per 256 tokens of ld: the page table must cover ld
  if (mode != 0 && (ws.tiles.cand == nullptr || n_tok_tiles != ws.tiles.n_tiles)) return hipErrorInvalidValue;
  if (n_tok_tiles == 0) return hipSuccess;
  if (mode == 0)
    hipLaunchKernelGGL(indexer_gemm_fp8_kernel<0>, dim3((unsigned)(n_row_blocks * n_tok_tiles)), dim3(256), 0, s, a,
                       (int)n_tok_tiles, ws, ctx_len);
  else if (mode == 1)
    hipLaunchKernelGGL(indexer_gemm_fp8_kernel<1>, dim3((unsigned)(n_row_blocks * kSampleTiles)), dim3(256), 0, s, a,
                       (int)n_tok_tiles, ws, ctx_len);
  else
    hipLaunchKernelGGL(indexer_gemm_fp8_kernel<2>, dim3((unsigned)(n_row_blocks * n_tok_tiles)), dim3(256), 0, s, a,
                       (int)n_tok_tiles, ws, ctx_len);
  return hipGetLastError();
}

}  // namespace dsa
