// mla.hip -- exact MLA attention over each query row's selected tokens (decode and prefill).
//
// Page "vLLM 为 Kimi K3.1 Pro 提供 Day-0 支持":
//  * section "K3.1 Pro 中的稀疏注意力" and figure 1: every query head attends exactly
//    to the kept tokens' latents; attention reads the full latent only for them;
//  * section "长上下文：带稀疏 indexer 的 decode 上下文并行": partial attention
//    outputs are merged by log-sum-exp -- used here to merge token splits;
//  * section "预填充：上下文并行稀疏注意力": a prefill workgroup handles one query
//    row over its local heads, reading the selected tokens straight from the cache.
// Keys are all 576 latent dims, values the first 512 (the no-rope part).
//
// One workgroup = (query row, token split, 16-head tile); 4 waves.  The split's token
// offsets are resolved once (index -> page -> pool offset).  Then, per 64-token subtile:
//   gather  the 64 latents (nontemporal 16-B loads, issued one subtile ahead into
//           registers) are decoded to bf16 -- exact for e4m3 and NVFP4 -- into one
//           token-major LDS tile Kt[64][576];
//   QK      wave w: S^T[16 tokens][16 heads] = Kt[16w..] . Q^T, 18 v_mfma_f32_16x16x32_bf16;
//   softmax online, per head, in log2 units; P is rounded to bf16 once and the same
//           rounded values feed both P.V and the row sum that normalises O; the LSE takes
//           a second row sum of the unrounded p (with few tokens the rounding of P would
//           not average out of the LSE);
//   PV      wave w: O^T[128 dims][16 heads] += V^T . P^T over the 64 tokens.  The V^T
//           operand (8 consecutive tokens of one dim per lane) is read from the same
//           token-major tile with ds_read_b64_tr_b16: in each 16-lane group, source lane
//           L points at row r0 + (L>>2), dims d0 + 4(L&3), and lane i receives rows
//           r0..r0+3 of dim d0 + i.  The S^T accumulator layout is already the B-operand
//           layout of P^T.
// kv_scale and the query's FP8 scale are applied in fp32 (logits and output), never
// folded into bf16 operands.  Token splits have a fixed size and are merged in a fixed
// order, so a row's result does not depend on the batch.
#include <math.h>

#include <type_traits>

#include "dsa_device.hpp"
#include "dsa_kernels.hpp"

namespace dsa {

namespace {

typedef __attribute__((ext_vector_type(4))) short i16x4_t;

constexpr int kSub = 64;     // tokens per subtile
constexpr int kKtLd = 592;   // bf16 per Kt row (576 + 16 pad: rows land 8 banks apart)
constexpr int kMaxTps = 2048;

struct MlaWs {
  float *o;    // [n_q][nsplit][H][512] unnormalised partial outputs
  float4 *ml;  // [n_q][nsplit][H] (running max in log2 units, sum of the bf16-rounded p, fp32 sum of p, 0)
};

__host__ __device__ inline int64_t a16(int64_t x) { return (x + 15) & ~int64_t(15); }

__host__ __device__ inline MlaWs mla_carve(void *ws, int32_t n_q, int32_t H, int nsplit) {
  MlaWs w;
  uint8_t *p = static_cast<uint8_t *>(ws);
  w.o = reinterpret_cast<float *>(p);
  p += a16(4 * (int64_t)n_q * nsplit * H * kVDim);
  w.ml = reinterpret_cast<float4 *>(p);
  return w;
}

// 16 raw bytes of a latent row chunk per gather item.
template <int LAT_FMT>
struct Gather {
  // FP8: 36 chunks of 16 B per token (16 dims each).  NVFP4: 16 chunks of 16 B of e2m1
  // (32 dims each, two 16-dim block scales) + 4 chunks of 16 B of rope e4m3 (16 dims each).
  static constexpr int kChunks = LAT_FMT == 0 ? 36 : 20;
  static constexpr int kItems = kSub * kChunks;          // 2304 / 1280
  static constexpr int kPerThread = kItems / 256;        // 9 / 5
  static_assert(kItems % 256 == 0, "gather items must tile the workgroup");
};

__device__ __forceinline__ i16x4_t tr16(const uint16_t *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t *)(const_cast<uint16_t *>(p)));
}

template <int LAT_FMT, int Q_FMT>
__global__ __launch_bounds__(256, 2) void mla_kernel(const MlaArgs a, const int nsplit, const int tps, MlaWs w) {
  using G = Gather<LAT_FMT>;
  constexpr int LB = LAT_FMT == 0 ? 576 : 352;
  constexpr int64_t LPB = (int64_t)kPage * LB;
  __shared__ __align__(16) uint16_t s_kt[kSub * kKtLd];
  __shared__ __align__(16) uint16_t s_p[4][64 * 4];
  __shared__ float s_red[3][4][16];
  extern __shared__ int64_t s_off[];  // [tps]: pool offset of each of the split's tokens

  const int ht = blockIdx.x, sp = blockIdx.y, r = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int hl = lane & 15, g = lane >> 4;
  const int H = a.n_heads;
  const int h = ht * 16 + hl;
  const bool hvalid = h < H;
  const int b = a.q_req ? a.q_req[r] : r;
  const bool rvalid = b >= 0 && b < a.n_req;
  if (!rvalid && tid == 0 && sp == 0 && ht == 0) flag_error(a.err, DSA_DEVERR_REQUEST);
  const int ctx = rvalid && !a.phys ? a.ctx_len[b] : 0;
  const int t_beg = sp * tps;
  const int n_tok = max(0, min(a.k, t_beg + tps) - t_beg);

  // Q^T fragments: lane (head hl, group g) holds q[h][32s + 8g .. +8] for s < 18.  Loaded
  // first, so that they travel together with the index and page-offset reads below.
  bf16x8_t qf[18];
  u32x2_t qc8[18];
  float qscale = 1.0f;
  if (hvalid) {
    if constexpr (Q_FMT == 0) {
      const uint16_t *qr = static_cast<const uint16_t *>(a.q) + ((int64_t)r * H + h) * kLatDim;
#pragma unroll
      for (int s = 0; s < 18; ++s) qf[s] = *reinterpret_cast<const bf16x8_t *>(qr + 32 * s + 8 * g);
    } else {
      const uint8_t *qr = static_cast<const uint8_t *>(a.q) + ((int64_t)r * H + h) * kLatDim;
#pragma unroll
      for (int s = 0; s < 18; ++s) qc8[s] = *reinterpret_cast<const u32x2_t *>(qr + 32 * s + 8 * g);
      qscale = a.q_scale[(int64_t)r * H + h];
    }
  } else {
#pragma unroll
    for (int s = 0; s < 18; ++s) {
      qf[s] = bf16x8_t{};
      qc8[s] = u32x2_t{};
    }
  }

  // (0) pool offsets of the split's tokens (-1: padding or invalid)
  for (int j = tid; j < n_tok; j += 256) {
    int64_t off = -1;
    if (rvalid && a.phys) {  // physical rows: the address needs no page-table read
      const int pr = a.idx[(int64_t)r * a.idx_ld + t_beg + j];
      if (pr >= 0) {
        const int64_t o = (int64_t)(pr >> 6) * a.row_stride + a.layer_off + (int64_t)(pr & 63) * LB;
        if ((pr >> 6) >= a.pool_rows || o + LB > a.pool_bytes)
          flag_error(a.err, DSA_DEVERR_BLOCK_RANGE);
        else
          off = o;
      }
    } else if (rvalid) {
      const int t = a.idx[(int64_t)r * a.idx_ld + t_beg + j];
      if (t >= 0) {
        const int pg = t >> 6;
        if (t >= ctx || pg >= a.off_ld) {
          flag_error(a.err, DSA_DEVERR_INDEX);
        } else {
          const int64_t po = a.lat_off[(int64_t)b * a.off_ld + pg];
          if (po < 0 || po + LPB > a.pool_bytes || (po & 15))
            flag_error(a.err, DSA_DEVERR_PAGE_OFFSET);
          else
            off = po + (int64_t)(t & 63) * LB;
        }
      }
    }
    s_off[j] = off;
  }

  if constexpr (Q_FMT == 1) {
#pragma unroll
    for (int s = 0; s < 18; ++s) qf[s] = e4m3x8_bf16(qc8[s][0], qc8[s][1]);
  }
  const float c2 = a.sm_scale * a.kv_scale * qscale * kLog2e;  // logits in log2 units
  __syncthreads();  // s_off ready; query loads drained before the gather pipeline starts
  __builtin_amdgcn_s_waitcnt(0x0F70);

  // (1) gather pipeline: raw 16-B chunks of the next subtile live in registers
  u32x4_t raw[G::kPerThread];
  uint32_t bsc[G::kPerThread];  // NVFP4: the chunk's two e4m3 block scales (bytes 0, 1)
  auto issue = [&](int t0) {
    // the tokens' pool offsets first (clamped reads, no branch: all LDS reads in flight
    // together), then the loads
    int64_t offs[G::kPerThread];
#pragma unroll
    for (int i = 0; i < G::kPerThread; ++i) {
      const int j = t0 + (tid + 256 * i) / G::kChunks;
      const int64_t o = s_off[min(j, n_tok - 1)];
      offs[i] = j < n_tok ? o : -1;
    }
#pragma unroll
    for (int i = 0; i < G::kPerThread; ++i) {
      const int item = tid + 256 * i;
      const int tok = item / G::kChunks, c = item - tok * G::kChunks;
      const int64_t off = offs[i];
      // every lane issues the load (an invalid token reads the pool's first bytes and is
      // zeroed on decode), so the number of loads in flight is the same on every path
      const uint8_t *base = a.pool + (off < 0 ? 0 : off);
      if constexpr (LAT_FMT == 0) {
        raw[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(base + 16 * c));
      } else {
        const int boff = c < 16 ? 16 * c : 288 + 16 * (c - 16);
        raw[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(base + boff));
        bsc[i] = *reinterpret_cast<const uint16_t *>(base + 256 + 2 * (c < 16 ? c : 0));
      }
    }
  };
  auto park = [&](int t0) {
#pragma unroll
    for (int i = 0; i < G::kPerThread; ++i) {
      const int item = tid + 256 * i;
      const int tok = item / G::kChunks, c = item - tok * G::kChunks;
      const int j = t0 + tok;
      const bool ok = j < n_tok && s_off[j] >= 0;
      uint16_t *dst = s_kt + tok * kKtLd;
      if constexpr (LAT_FMT == 0) {
        bf16x8_t lo = e4m3x8_bf16(raw[i][0], raw[i][1]), hi = e4m3x8_bf16(raw[i][2], raw[i][3]);
        if (!ok) lo = hi = bf16x8_t{};
        *reinterpret_cast<bf16x8_t *>(dst + 16 * c) = lo;
        *reinterpret_cast<bf16x8_t *>(dst + 16 * c + 8) = hi;
      } else if (c < 16) {  // 32 no-rope dims: e2m1 x block scale
        const float s0 = e4m3_f32(bsc[i] & 0xFFu), s1 = e4m3_f32((bsc[i] >> 8) & 0xFFu);
        bf16x8_t v0 = nvfp4x8_bf16(raw[i][0], s0), v1 = nvfp4x8_bf16(raw[i][1], s0);
        bf16x8_t v2 = nvfp4x8_bf16(raw[i][2], s1), v3 = nvfp4x8_bf16(raw[i][3], s1);
        if (!ok) v0 = v1 = v2 = v3 = bf16x8_t{};
        *reinterpret_cast<bf16x8_t *>(dst + 32 * c) = v0;
        *reinterpret_cast<bf16x8_t *>(dst + 32 * c + 8) = v1;
        *reinterpret_cast<bf16x8_t *>(dst + 32 * c + 16) = v2;
        *reinterpret_cast<bf16x8_t *>(dst + 32 * c + 24) = v3;
      } else {  // 16 rope dims, e4m3
        bf16x8_t lo = e4m3x8_bf16(raw[i][0], raw[i][1]), hi = e4m3x8_bf16(raw[i][2], raw[i][3]);
        if (!ok) lo = hi = bf16x8_t{};
        *reinterpret_cast<bf16x8_t *>(dst + 512 + 16 * (c - 16)) = lo;
        *reinterpret_cast<bf16x8_t *>(dst + 512 + 16 * (c - 16) + 8) = hi;
      }
    }
  };

  float m_run = -INFINITY, l_run = 0.0f, lf_run = 0.0f;
  f32x4_t o[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) o[dt] = f32x4_t{};

  if (n_tok > 0) issue(0);
  for (int t0 = 0; t0 < n_tok; t0 += kSub) {
    park(t0);
    __syncthreads();
    if (t0 + kSub < n_tok) issue(t0 + kSub);  // uniform; flies while this subtile is computed

    // (2) S^T = K Q^T, wave w: tokens 16w..16w+15
    f32x4_t acc = {};
    const uint16_t *krow = s_kt + (16 * wid + hl) * kKtLd + 8 * g;
#pragma unroll
    for (int s = 0; s < 18; ++s) acc = mfma_16x16x32_bf16(*reinterpret_cast<const bf16x8_t *>(krow + 32 * s), qf[s], acc);
    float z[4], mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = t0 + 16 * wid + 4 * g + i;
      z[i] = (j < n_tok && s_off[j] >= 0) ? acc[i] * c2 : -INFINITY;
      mx = fmaxf(mx, z[i]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    if (g == 0) s_red[0][wid][hl] = mx;
    __syncthreads();
    const float m_new =
        fmaxf(m_run, fmaxf(fmaxf(s_red[0][0][hl], s_red[0][1][hl]), fmaxf(s_red[0][2][hl], s_red[0][3][hl])));
    const float alpha = m_new == -INFINITY ? 1.0f : exp2f(m_run - m_new);
    float ps = 0.0f, pf = 0.0f;
    bf16x4_t pb;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = z[i] == -INFINITY ? 0.0f : exp2f(z[i] - m_new);
      pb[i] = (__bf16)p;
      ps += (float)pb[i];
      pf += p;
    }
    *reinterpret_cast<bf16x4_t *>(s_p[wid] + 4 * lane) = pb;
    ps += __shfl_xor(ps, 16, 64);
    ps += __shfl_xor(ps, 32, 64);
    pf += __shfl_xor(pf, 16, 64);
    pf += __shfl_xor(pf, 32, 64);
    if (g == 0) {
      s_red[1][wid][hl] = ps;
      s_red[2][wid][hl] = pf;
    }
    __syncthreads();
    l_run = l_run * alpha + ((s_red[1][0][hl] + s_red[1][1][hl]) + (s_red[1][2][hl] + s_red[1][3][hl]));
    lf_run = lf_run * alpha + ((s_red[2][0][hl] + s_red[2][1][hl]) + (s_red[2][2][hl] + s_red[2][3][hl]));
    m_run = m_new;

    // (3) O^T += V^T P^T.  K-step ks covers tokens 32ks..32ks+31; k-slot j of group g is
    // token 32ks + 4g + j (j < 4, from S^T tile 2ks) or 32ks + 16 + 4g + j - 4 (tile 2ks+1).
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[dt] *= alpha;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8_t pf = cat4(*reinterpret_cast<const bf16x4_t *>(s_p[2 * ks] + 4 * lane),
                               *reinterpret_cast<const bf16x4_t *>(s_p[2 * ks + 1] + 4 * lane));
      const uint16_t *v0 = s_kt + (32 * ks + 4 * g + (hl >> 2)) * kKtLd + 4 * (hl & 3);
      const uint16_t *v1 = v0 + 16 * kKtLd;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const int d0 = 128 * wid + 16 * dt;
        const i16x4_t x0 = tr16(v0 + d0), x1 = tr16(v1 + d0);
        const bf16x8_t va = cat4(__builtin_bit_cast(bf16x4_t, x0), __builtin_bit_cast(bf16x4_t, x1));
        o[dt] = mfma_16x16x32_bf16(va, pf, o[dt]);
      }
    }
    __syncthreads();  // s_kt and s_p are rewritten by the next subtile
  }

  // (4) results: lane (head hl, group g) holds dims 128*wid + 16*dt + 4g + i
  if (!hvalid) return;
  if (nsplit == 1) {
    const float inv = l_run > 0.0f ? a.kv_scale / l_run : 0.0f;
    uint16_t *orow = a.out + ((int64_t)r * H + h) * kVDim;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      bf16x4_t v;
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = (__bf16)(o[dt][i] * inv);
      *reinterpret_cast<bf16x4_t *>(orow + 128 * wid + 16 * dt + 4 * g) = v;
    }
    if (wid == 0 && g == 0) a.lse[(int64_t)r * H + h] = lf_run > 0.0f ? (m_run + log2f(lf_run)) * kLn2 : -INFINITY;
  } else {
    const int64_t slot = ((int64_t)r * nsplit + sp) * H + h;
    float *po = w.o + slot * kVDim;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) *reinterpret_cast<f32x4_t *>(po + 128 * wid + 16 * dt + 4 * g) = o[dt];
    if (wid == 0 && g == 0) w.ml[slot] = make_float4(m_run, l_run, lf_run, 0.0f);
  }
}

// Wide variant for many heads (prefill: 96): one workgroup per (query row, token split)
// covers every head of the row, so each 64-token subtile is gathered and decoded once for
// all heads instead of once per 16-head tile.  Wave w owns heads 16 w .. 16 w + 15 (waves
// past the last head tile only help gather): QK over all 64 tokens of the subtile, an
// in-wave online softmax, and P.V into all 512 value dims.  FP8 queries stay as e4m3 codes
// in registers and are converted to bf16 per MFMA.
constexpr int kWideThreads = 512;                  // 8 waves: up to 8 head tiles (128 heads)
constexpr int kWideMaxTiles = kWideThreads / 64;

template <int LAT_FMT>
__global__ __launch_bounds__(kWideThreads) void mla_wide_kernel(const MlaArgs a, const int nsplit, const int tps,
                                                                MlaWs w) {
  constexpr int LB = LAT_FMT == 0 ? 576 : 352;
  constexpr int64_t LPB = (int64_t)kPage * LB;
  constexpr int kChunks = Gather<LAT_FMT>::kChunks;
  constexpr int kItems = kSub * kChunks;
  constexpr int kPer = (kItems + kWideThreads - 1) / kWideThreads;  // 5 / 3
  __shared__ __align__(16) uint16_t s_kt[kSub * kKtLd];
  __shared__ __align__(16) uint16_t s_p[kWideMaxTiles][4][64 * 4];
  extern __shared__ int64_t s_off[];  // [tps]

  const int sp = blockIdx.y, r = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int hl = lane & 15, g = lane >> 4;
  const int H = a.n_heads;
  const bool computes = wid * 16 < H;  // wave-uniform
  const int h = wid * 16 + hl;
  const bool hvalid = h < H;
  const int b = a.q_req ? a.q_req[r] : r;
  const bool rvalid = b >= 0 && b < a.n_req;
  if (!rvalid && tid == 0 && sp == 0) flag_error(a.err, DSA_DEVERR_REQUEST);
  const int ctx = rvalid ? a.ctx_len[b] : 0;
  const int t_beg = sp * tps;
  const int n_tok = max(0, min(a.k, t_beg + tps) - t_beg);

  // e4m3 query codes: lane (head hl, group g) holds dims 32 s + 8 g .. + 8 of head h; loaded
  // first, so that they travel together with the index and page-offset reads below
  u32x2_t qc[18];
  float qscale = 0.0f;
  if (hvalid) {
    const uint8_t *qr = static_cast<const uint8_t *>(a.q) + ((int64_t)r * H + h) * kLatDim;
#pragma unroll
    for (int s = 0; s < 18; ++s) qc[s] = *reinterpret_cast<const u32x2_t *>(qr + 32 * s + 8 * g);
    qscale = a.q_scale[(int64_t)r * H + h];
  } else {
#pragma unroll
    for (int s = 0; s < 18; ++s) qc[s] = u32x2_t{};
  }
  for (int j = tid; j < n_tok; j += kWideThreads) {
    int64_t off = -1;
    if (rvalid) {
      const int t = a.idx[(int64_t)r * a.idx_ld + t_beg + j];
      if (t >= 0) {
        const int pg = t >> 6;
        if (t >= ctx || pg >= a.off_ld) {
          flag_error(a.err, DSA_DEVERR_INDEX);
        } else {
          const int64_t po = a.lat_off[(int64_t)b * a.off_ld + pg];
          if (po < 0 || po + LPB > a.pool_bytes || (po & 15))
            flag_error(a.err, DSA_DEVERR_PAGE_OFFSET);
          else
            off = po + (int64_t)(t & 63) * LB;
        }
      }
    }
    s_off[j] = off;
  }

  const float c2 = a.sm_scale * a.kv_scale * qscale * kLog2e;
  __syncthreads();
  __builtin_amdgcn_s_waitcnt(0x0F70);

  u32x4_t raw[kPer];
  uint32_t bsc[kPer];
  auto issue = [&](int t0) {
    // the tokens' pool offsets first (clamped reads: all LDS reads in flight together)
    int64_t offs[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int item = tid + kWideThreads * i;
      const int j = t0 + item / kChunks;
      const int64_t o = s_off[min(j, n_tok - 1)];
      offs[i] = (item < kItems && j < n_tok) ? o : -1;
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int item = tid + kWideThreads * i;
      const int tok = item / kChunks, c = item - tok * kChunks;
      const int64_t off = offs[i];
      const uint8_t *base = a.pool + (off < 0 ? 0 : off);  // every lane loads: fixed wait counts
      const int cc = c < kChunks ? c : 0;
      if constexpr (LAT_FMT == 0) {
        raw[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(base + 16 * cc));
      } else {
        const int boff = cc < 16 ? 16 * cc : 288 + 16 * (cc - 16);
        raw[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(base + boff));
        bsc[i] = *reinterpret_cast<const uint16_t *>(base + 256 + 2 * (cc < 16 ? cc : 0));
      }
    }
  };
  auto park = [&](int t0) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int item = tid + kWideThreads * i;
      if (item >= kItems) continue;
      const int tok = item / kChunks, c = item - tok * kChunks;
      const int j = t0 + tok;
      const bool ok = j < n_tok && s_off[j] >= 0;
      uint16_t *dst = s_kt + tok * kKtLd;
      if constexpr (LAT_FMT == 0) {
        bf16x8_t lo = e4m3x8_bf16(raw[i][0], raw[i][1]), hi = e4m3x8_bf16(raw[i][2], raw[i][3]);
        if (!ok) lo = hi = bf16x8_t{};
        *reinterpret_cast<bf16x8_t *>(dst + 16 * c) = lo;
        *reinterpret_cast<bf16x8_t *>(dst + 16 * c + 8) = hi;
      } else if (c < 16) {
        const float s0 = e4m3_f32(bsc[i] & 0xFFu), s1 = e4m3_f32((bsc[i] >> 8) & 0xFFu);
        bf16x8_t v0 = nvfp4x8_bf16(raw[i][0], s0), v1 = nvfp4x8_bf16(raw[i][1], s0);
        bf16x8_t v2 = nvfp4x8_bf16(raw[i][2], s1), v3 = nvfp4x8_bf16(raw[i][3], s1);
        if (!ok) v0 = v1 = v2 = v3 = bf16x8_t{};
        *reinterpret_cast<bf16x8_t *>(dst + 32 * c) = v0;
        *reinterpret_cast<bf16x8_t *>(dst + 32 * c + 8) = v1;
        *reinterpret_cast<bf16x8_t *>(dst + 32 * c + 16) = v2;
        *reinterpret_cast<bf16x8_t *>(dst + 32 * c + 24) = v3;
      } else {
        bf16x8_t lo = e4m3x8_bf16(raw[i][0], raw[i][1]), hi = e4m3x8_bf16(raw[i][2], raw[i][3]);
        if (!ok) lo = hi = bf16x8_t{};
        *reinterpret_cast<bf16x8_t *>(dst + 512 + 16 * (c - 16)) = lo;
        *reinterpret_cast<bf16x8_t *>(dst + 512 + 16 * (c - 16) + 8) = hi;
      }
    }
  };

  float m_run = -INFINITY, l_run = 0.0f, lf_run = 0.0f;
  f32x4_t o[32];
#pragma unroll
  for (int dt = 0; dt < 32; ++dt) o[dt] = f32x4_t{};
  uint16_t *my_p = s_p[wid][0];

  if (n_tok > 0) issue(0);
  for (int t0 = 0; t0 < n_tok; t0 += kSub) {
    park(t0);
    __syncthreads();
    if (t0 + kSub < n_tok) issue(t0 + kSub);
    if (computes) {
      // S^T: 4 groups of 16 tokens x this wave's 16 heads
      float z[4][4], mx = -INFINITY;
#pragma unroll
      for (int tg = 0; tg < 4; ++tg) {
        // the codes are converted again for every token group: hoisting the bf16 query out
        // of this loop would hold 72 registers instead of 36
#pragma unroll
        for (int s = 0; s < 18; ++s) asm volatile("" : "+v"(qc[s]));
        const uint16_t *krow = s_kt + (16 * tg + hl) * kKtLd + 8 * g;
        f32x4_t acc = {};
#pragma unroll
        for (int s = 0; s < 18; ++s)
          acc = mfma_16x16x32_bf16(*reinterpret_cast<const bf16x8_t *>(krow + 32 * s), e4m3x8_bf16(qc[s][0], qc[s][1]),
                                   acc);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = t0 + 16 * tg + 4 * g + i;
          z[tg][i] = (j < n_tok && s_off[j] >= 0) ? acc[i] * c2 : -INFINITY;
          mx = fmaxf(mx, z[tg][i]);
        }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run, mx);
      const float alpha = m_new == -INFINITY ? 1.0f : exp2f(m_run - m_new);
      float ps = 0.0f, pf = 0.0f;
#pragma unroll
      for (int tg = 0; tg < 4; ++tg) {
        bf16x4_t pb;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = z[tg][i] == -INFINITY ? 0.0f : exp2f(z[tg][i] - m_new);
          pb[i] = (__bf16)p;
          ps += (float)pb[i];
          pf += p;
        }
        *reinterpret_cast<bf16x4_t *>(my_p + 256 * tg + 4 * lane) = pb;
      }
      ps += __shfl_xor(ps, 16, 64);
      ps += __shfl_xor(ps, 32, 64);
      pf += __shfl_xor(pf, 16, 64);
      pf += __shfl_xor(pf, 32, 64);
      l_run = l_run * alpha + ps;
      lf_run = lf_run * alpha + pf;
      m_run = m_new;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");  // P written by the whole wave
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      // O^T += V^T P^T, 32-token K-steps
#pragma unroll
      for (int dt = 0; dt < 32; ++dt) o[dt] *= alpha;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8_t pf = cat4(*reinterpret_cast<const bf16x4_t *>(my_p + 256 * (2 * ks) + 4 * lane),
                                 *reinterpret_cast<const bf16x4_t *>(my_p + 256 * (2 * ks + 1) + 4 * lane));
        const uint16_t *v0 = s_kt + (32 * ks + 4 * g + (hl >> 2)) * kKtLd + 4 * (hl & 3);
        const uint16_t *v1 = v0 + 16 * kKtLd;
#pragma unroll
        for (int dt = 0; dt < 32; ++dt) {
          const i16x4_t x0 = tr16(v0 + 16 * dt), x1 = tr16(v1 + 16 * dt);
          const bf16x8_t va = cat4(__builtin_bit_cast(bf16x4_t, x0), __builtin_bit_cast(bf16x4_t, x1));
          o[dt] = mfma_16x16x32_bf16(va, pf, o[dt]);
        }
      }
    }
    __syncthreads();  // s_kt is rewritten by the next subtile
  }

  // lane (head hl, group g) holds dims 16 dt + 4 g + i
  if (!computes || !hvalid) return;
  if (nsplit == 1) {
    const float inv = l_run > 0.0f ? a.kv_scale / l_run : 0.0f;
    uint16_t *orow = a.out + ((int64_t)r * H + h) * kVDim;
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) {
      bf16x4_t vv;
#pragma unroll
      for (int i = 0; i < 4; ++i) vv[i] = (__bf16)(o[dt][i] * inv);
      *reinterpret_cast<bf16x4_t *>(orow + 16 * dt + 4 * g) = vv;
    }
    if (g == 0) a.lse[(int64_t)r * H + h] = lf_run > 0.0f ? (m_run + log2f(lf_run)) * kLn2 : -INFINITY;
  } else {
    const int64_t slot = ((int64_t)r * nsplit + sp) * H + h;
    float *po = w.o + slot * kVDim;
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) *reinterpret_cast<f32x4_t *>(po + 16 * dt + 4 * g) = o[dt];
    if (g == 0) w.ml[slot] = make_float4(m_run, l_run, lf_run, 0.0f);
  }
}

// ---- prefill, FP8 latents: every head of a row per workgroup ----
//
// One 256-thread workgroup per (row, split), one wave per SIMD.  The work of a 32-token
// subtile is split two ways:
//   QK  wave t < ceil(H / 32) owns head tile t (heads 32t .. 32t+31):
//         S^T[token][head] = K Q^T   9 v_mfma_scale_f32_32x32x64_f8f6f4 (scales 1): A = 32 raw
//                                    e4m3 bytes of a K row per lane from LDS, B = 32 bytes of
//                                    the row's e4m3 query codes per lane from registers.  The
//                                    FP8 MFMA rounds inside its sums (~1e-5 of sum |q k|); the
//                                    logits then move the attention output far less than its
//                                    1e-2 tolerance.
//       then the softmax weights P (bf16, rounded once; the same rounded values feed the row
//       sum) go to LDS as the P^T operand fragments of the tile.
//   PV  wave w owns value dims 128w .. 128w+127 of every head:
//         O^T[dim][head] += V^T P^T  8 x (head tiles) v_mfma_f32_32x32x16_bf16: A = 8 tokens x
//                                    1 dim of V per lane by ds_read_b64_tr_b8, decoded e4m3 ->
//                                    bf16 (exact) once per wave and used for every head tile;
//                                    B = P^T of the tile from LDS.
//       Its accumulators (4 dim blocks x up to 4 head tiles of 32 x 32 fp32) stay in the
//       MFMA accumulator registers for the whole row.
// So every SIMD takes part in P.V, and each value byte is decoded once per workgroup, where
// a wave holding all 512 dims of its own heads would leave one SIMD idle at 96 heads and
// decode every value byte once per head tile.
// S^T's accumulator row rho = 8q + 4p + i holds token 16 (q / 2) + 8 p + 4 (q % 2) + i (the
// K operand's lanes read their rows in that order), so lane half p's elements 8 s2 .. 8 s2+7
// are the 8 consecutive tokens 16 s2 + 8 p .. + 7 -- the K order of one transposing read, and
// S^T's lane layout is already the B layout of P^T.
// Gather: rows go straight to LDS by direct loads into a ring of six subtile slots, four
// subtiles ahead of the one whose softmax runs; one barrier per subtile both frees the oldest
// slot and publishes P (the pipeline is described at the loop).  Rows sit 592 B apart in a
// slot, which spreads the 16 rows of one K read over distinct banks.
// Softmax reference: p = 2^(z - m_ref) with m_ref fixed at the head's max over its first
// subtile with a valid token, so the accumulators are never rescaled.  O / l and
// m_ref + log2 l do not depend on the reference, and p <= 2^64 keeps p (bf16), l and O (fp32)
// far from overflow.  If a later max passes m_ref by more than 2^64, the workgroup computes
// the row again with m_ref = the row's true max (a second pass that real data never needs).
constexpr int kPfSub = 32;
constexpr int kPfThreads = 256;
constexpr float kRefSlack = 64.0f;                  // log2 units
constexpr int kPfRow = 592;                         // bytes per row in a slot (576 + 16)
constexpr int kPfChunks = kPfRow / 16;              // 37 16-byte chunks, the last one padding
constexpr int kPfLoads = (kPfSub * kPfChunks + 63) / 64;  // 19 wave loads per subtile
constexpr int kPfPer = (kPfLoads + 3) / 4;          // 5 per wave (padded to 20)
constexpr int kPfSlot = 4 * kPfPer * 1024;          // 20 KB
constexpr int kPfSlots = 6;                         // 120 KB; with P (16 KB) and s_off (16 KB) within 160 KB
constexpr int kPfAhead = kPfSlots - 2;              // subtiles issued ahead of the one whose softmax runs
constexpr int kPfMaxSubs = kMaxTps / kPfSub;        // 64
constexpr int kPfBlocks = kVDim / 32 / 4;           // 32-dim blocks of V per wave: 4

// s_waitcnt vmcnt(K), other counters untouched (K < 64)
template <int K>
__device__ __forceinline__ void wait_vm() {
  static_assert(K >= 0 && K < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (K & 15) | ((K >> 4) << 14));
}

typedef __attribute__((ext_vector_type(2))) int i32x2_t;

// 16 bytes from global memory straight into LDS (global_load_lds_dwordx4 with M0 = `lds`, a
// wave-uniform LDS byte address; the wave's 64 lanes fill lds .. lds + 1 KB).  Issued from inline asm: the compiler then does not make every
// later LDS read wait for all such loads in flight (it cannot tell ring slots apart), which
// would expose the gather's full latency each subtile.  Every read of a ring slot is ordered
// after its loads by an explicit vmcnt wait and a barrier instead.
// (m0 is set right before its one use here; the compiler also sets it before each of its own
// uses, so the clobber is harmless)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_dma16(const void *src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds) : "memory", "m0");
}
#pragma clang diagnostic pop

// 32-bit LDS address of a __shared__ object
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void *)p;
}

template <int NHT>  // head tiles of 32: 2..4
__global__ __launch_bounds__(kPfThreads, 1) void mla_prefill_kernel(const MlaArgs a, const int nsplit, const int tps,
                                                                     MlaWs w) {
  constexpr int LB = 576;
  constexpr int64_t LPB = (int64_t)kPage * LB;
  __shared__ __align__(16) uint8_t s_raw[kPfSlots][kPfSlot];
  __shared__ __align__(16) u32x4_t s_p[2][4][2][64];  // P^T fragments: [subtile & 1][wave][K-step][lane]
  __shared__ float s_l[NHT * 32];                    // row sums, for the PV waves' outputs
  __shared__ uint32_t s_ok[kPfMaxSubs];  // valid tokens of each subtile
  __shared__ int s_redo;                 // some head's max passed its reference by > 2^64
  extern __shared__ int64_t s_off[];     // [tps]

  const int sp = blockIdx.y, r = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int n = lane & 31, g = lane >> 5;
  const int H = a.n_heads;
  const bool computes = wid < NHT;        // this wave forms S and P of head tile wid
  const int h = wid * 32 + n;
  const bool hvalid = computes && h < H;
  const int b = a.q_req ? a.q_req[r] : r;
  const bool rvalid = b >= 0 && b < a.n_req;
  if (!rvalid && tid == 0 && sp == 0) flag_error(a.err, DSA_DEVERR_REQUEST);
  const int ctx = rvalid ? a.ctx_len[b] : 0;
  const int t_beg = sp * tps;
  const int n_tok = max(0, min(a.k, t_beg + tps) - t_beg);
  const int n_sub = (n_tok + kPfSub - 1) / kPfSub;

  // e4m3 query codes: lane (head n, half g) holds dims 64 s + 32 g .. + 32 of head h
  i32x8_t qc[9];
  float qscale = 0.0f;
  if (hvalid) {
    const uint8_t *qr = static_cast<const uint8_t *>(a.q) + ((int64_t)r * H + h) * kLatDim;
#pragma unroll
    for (int s = 0; s < 9; ++s) {
      const u32x4_t lo = *reinterpret_cast<const u32x4_t *>(qr + 64 * s + 32 * g);
      const u32x4_t hi = *reinterpret_cast<const u32x4_t *>(qr + 64 * s + 32 * g + 16);
      qc[s] = i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
    qscale = a.q_scale[(int64_t)r * H + h];
  } else {
#pragma unroll
    for (int s = 0; s < 9; ++s) qc[s] = i32x8_t{};
  }
  for (int j = tid; j < n_tok; j += kPfThreads) {
    int64_t off = -1;
    if (rvalid) {
      const int t = a.idx[(int64_t)r * a.idx_ld + t_beg + j];
      if (t >= 0) {
        const int pg = t >> 6;
        if (t >= ctx || pg >= a.off_ld) {
          flag_error(a.err, DSA_DEVERR_INDEX);
        } else {
          const int64_t po = a.lat_off[(int64_t)b * a.off_ld + pg];
          if (po < 0 || po + LPB > a.pool_bytes || (po & 15))
            flag_error(a.err, DSA_DEVERR_PAGE_OFFSET);
          else
            off = po + (int64_t)(t & 63) * LB;
        }
      }
    }
    s_off[j] = off;
  }
  const float c2 = a.sm_scale * a.kv_scale * qscale * kLog2e;
  if (tid == 0) s_redo = 0;
  __syncthreads();
  for (int sub = wid; sub < n_sub; sub += 4) {
    const int j = sub * kPfSub + lane;
    const uint32_t okm = (uint32_t)__ballot(lane < kPfSub && j < n_tok && s_off[j] >= 0);
    if (lane == 0) s_ok[sub] = okm;
  }
  // Subtile `sub`'s rows -> ring slot sub % kPfSlots, rows kPfRow bytes apart: load kk (of
  // 20; wave w issues kk = 5w .. 5w+4) fills slot chunks 64 kk .. 64 kk + 63.  Lanes on a row's
  // padding chunk, past the rows, or on an invalid token read the pool's first bytes instead
  // (P.V clears an invalid token's value bytes; its logit is masked).
  // LDS address of this wave's first 1 KB in slot 0 (wave w fills loads 5w .. 5w+4 of a slot)
  const uint32_t wave_lds = __builtin_amdgcn_readfirstlane(lds_addr(s_raw[0]) + 1024 * kPfPer * wid);
  auto issue = [&](int sub) {
    const uint32_t slot_lds = wave_lds + kPfSlot * (uint32_t)(sub % kPfSlots);
    // the row offsets first, all reads in flight together (the index is clamped into s_off;
    // a clamped read is not used)
    int64_t offs[kPfPer];
#pragma unroll
    for (int i = 0; i < kPfPer; ++i) {
      const int tok = (64 * (wid * kPfPer + i) + lane) / kPfChunks;
      offs[i] = s_off[min(sub * kPfSub + min(tok, kPfSub - 1), n_tok - 1)];
    }
#pragma unroll
    for (int i = 0; i < kPfPer; ++i) {
      const int kk = wid * kPfPer + i, q = 64 * kk + lane;
      const int tok = q / kPfChunks, c = q - tok * kPfChunks;
      const bool ok = tok < kPfSub && c < LB / 16 && sub * kPfSub + tok < n_tok && offs[i] >= 0;
      lds_dma16(a.pool + (ok ? offs[i] + 16 * c : 0), slot_lds + 1024 * i);
    }
  };
  // lane rho of the K operand reads slot row pi(rho); S^T element e of half g is token
  // 16 (e / 8) + 8 g + e % 8
  const int krow = 16 * (n >> 4) + 8 * ((n >> 2) & 1) + 4 * ((n >> 3) & 1) + (n & 3);

  // PV operand: lane l of a 16-lane group points at token row 16 s2 + 8 g + (l & 15) / 2 and
  // dims 16 ((l >> 4) & 1) + 8 (l & 1) of a 32-dim block; the transposing read then gives
  // lane l dim (l & 31) of the block at the 8 tokens 16 s2 + 8 g .. + 7.  This wave's blocks
  // are 4 wid .. 4 wid + 3 (byte 128 wid of a row).
  const int vofs = (8 * g + ((lane & 15) >> 1)) * kPfRow + 16 * ((lane >> 4) & 1) + 8 * (lane & 1) + 128 * wid;

  float m_ref = -INFINITY, m_true = -INFINITY, l_run = 0.0f, lf_run = 0.0f;
  f32x16_t o[NHT][kPfBlocks];
  for (int pass = 0; pass < 2; ++pass) {
    bool over = false;
    l_run = 0.0f;
    lf_run = 0.0f;
#pragma unroll
    for (int t = 0; t < NHT; ++t)
#pragma unroll
      for (int db = 0; db < kPfBlocks; ++db) o[t][db] = f32x16_t{};
    // S^T of subtile j (head tile wid) on FP8: rows = the subtile's 32 tokens (permuted),
    // columns = 32 heads; 9 MFMAs over the slot's rows
    auto qk = [&](int j) {
      f32x16_t acc = {};
      const uint8_t *kr = s_raw[j % kPfSlots] + krow * kPfRow + 32 * g;
#pragma unroll
      for (int s = 0; s < 9; ++s) {
        const u32x4_t lo = *reinterpret_cast<const u32x4_t *>(kr + 64 * s);
        const u32x4_t hi = *reinterpret_cast<const u32x4_t *>(kr + 64 * s + 16);
        const i32x8_t ka = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka, qc[s], acc, 0, 0, 0, 0x7f7f7f7f, 0, 0x7f7f7f7f);
      }
      return acc;
    };
    // softmax of subtile j from its S^T: running max, p = 2^(S c2 - m_ref) rounded to bf16 in
    // pairs, the row sum of the rounded values (a bf16 dot product with ones), and P^T to LDS.
    // okm: the subtile's valid tokens (an invalid token's p is 0; with okm = 0 the call changes
    // nothing but its P buffer).  Before the head's first valid token m_ref is -inf and every
    // token of the subtile is invalid.
    const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
    auto softmax = [&](const f32x16_t &acc, int j, uint32_t okm) {
      // this lane's 16 tokens 16 (e / 8) + 8 g + e % 8 as bits e of m16
      const uint32_t m16 = ((okm >> (8 * g)) & 0xFFu) | ((okm >> (8 + 8 * g)) & 0xFF00u);
      float z[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) z[e] = ((m16 >> e) & 1u) ? acc[e] * c2 : -INFINITY;
      float mx = -INFINITY;
#pragma unroll
      for (int e = 0; e < 16; e += 2) mx = fmaxf(mx, fmaxf(z[e], z[e + 1]));
      {  // max with the other half-wave (lanes l and l ^ 32 hold the same head)
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_int(mx), __float_as_int(mx), false, false);
        mx = fmaxf(__int_as_float(sw[0]), __int_as_float(sw[1]));
      }
      if (m_ref == -INFINITY) m_ref = mx;  // the head's first valid tokens: O and l are still 0
      m_true = fmaxf(m_true, mx);
      over |= mx > m_ref + kRefSlack;
      const float mr = m_ref == -INFINITY ? 0.0f : m_ref;
      float ls = 0.0f, lf = 0.0f;
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        u32x4_t pk;
#pragma unroll
        for (int m2 = 0; m2 < 4; ++m2) {
          const f32x2_t pp = {__builtin_amdgcn_exp2f(z[8 * s2 + 2 * m2] - mr),
                              __builtin_amdgcn_exp2f(z[8 * s2 + 2 * m2 + 1] - mr)};
          const bf16x2_t pb = __builtin_convertvector(pp, bf16x2_t);
          pk[m2] = __builtin_bit_cast(uint32_t, pb);
          ls = __builtin_amdgcn_fdot2_f32_bf16(pb, ones, ls, false);
          lf += pp[0] + pp[1];
        }
        s_p[j & 1][wid][s2][lane] = pk;
      }
      l_run += ls;
      lf_run += lf;
    };
    // O^T += V^T P^T of subtile j over this wave's 4 dim blocks: step st = 4 s2 + db
    auto pv = [&](int j) {
      const uint8_t *vb = s_raw[j % kPfSlots] + vofs;
      i32x2_t xv[8];
#pragma unroll
      for (int st = 0; st < 8; ++st)
        xv[st] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (__attribute__((address_space(3))) i32x2_t *)(vb + 16 * (st >> 2) * kPfRow + 32 * (st & 3)));
      // Byte i of xv[4 s2 + db] is token 16 s2 + 8 g + i.  A token outside the set (padding, or
      // past the set's end) has p = 0, but its bytes are whatever its gather lane read instead
      // (the pool's first bytes), and 0 times a NaN code is NaN: its bytes are cleared (+0).
      const uint32_t okm = s_ok[j];
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const uint32_t b8 = (okm >> (16 * s2 + 8 * g)) & 0xFFu;
        // bit i of a nibble -> byte i (the products' terms land on distinct bits, no carries)
        const uint32_t mlo = (((b8 & 15u) * 0x00204081u) & 0x01010101u) * 0xFFu;
        const uint32_t mhi = (((b8 >> 4) * 0x00204081u) & 0x01010101u) * 0xFFu;
#pragma unroll
        for (int db = 0; db < kPfBlocks; ++db) {
          xv[4 * s2 + db][0] &= (int)mlo;
          xv[4 * s2 + db][1] &= (int)mhi;
        }
      }
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        bf16x8_t pt[NHT];
#pragma unroll
        for (int t = 0; t < NHT; ++t) pt[t] = __builtin_bit_cast(bf16x8_t, s_p[j & 1][t][s2][lane]);
#pragma unroll
        for (int db = 0; db < kPfBlocks; ++db) {
          const bf16x8_t va = e4m3x8_bf16((uint32_t)xv[4 * s2 + db][0], (uint32_t)xv[4 * s2 + db][1]);
#pragma unroll
          for (int t = 0; t < NHT; ++t) o[t][db] = mfma_32x32x16_bf16(va, pt[t], o[t][db]);
        }
      }
    };

    // Pipeline over subtiles: iteration it runs P.V of subtile it - 1, the logits of it + 1,
    // the softmax of it and the loads of it + kPfAhead, all in one basic block, so that the
    // softmax and the load issue run between the matrix-core instructions.  P of it - 1 was
    // published by the barrier that ends iteration it - 1, subtile it + 1 landed before it, and
    // the logits of it were formed in iteration it - 1.  Every wave runs the same code: a wave
    // past the last head tile forms logits of zero queries and its softmax output is not used.
    // Past the last subtile the logits are formed from whatever a slot holds and discarded, the
    // softmax sees no valid token, and the loads read the pool's first bytes into a free slot,
    // so that every iteration issues the same loads and the wait counts stay fixed.
    // Slots in use during iteration it: it - 1 .. it + kPfAhead (six); P buffers it & 1
    // (written) and (it - 1) & 1 (read).
    if (n_sub > 0) {
      for (int s = 0; s < kPfAhead; ++s) issue(s);
      wait_vm<(kPfAhead - 2) * kPfPer>();  // subtiles 0 and 1 have landed
      __syncthreads();
      f32x16_t acc = qk(0);
      {  // iteration 0: no P.V yet
        const f32x16_t an = qk(1);
        softmax(acc, 0, s_ok[0]);
        issue(kPfAhead);
        acc = an;
      }
      for (int it = 1;; ++it) {
        wait_vm<(kPfAhead - 2) * kPfPer>();  // subtile it + 1 has landed (all but the last two subtiles issued)
        // P of subtile it - 1 is in LDS; every wave is done with subtile it - 2, its slot and
        // its P buffer
        __syncthreads();
        pv(it - 1);
        const f32x16_t an = qk(it + 1);
        softmax(acc, it, it < n_sub ? s_ok[it] : 0u);
        issue(it + kPfAhead);
        acc = an;
        // interleave: each of the 33 MFMAs (24 P.V, 9 logits) followed by up to 12 VALU
        // instructions (softmax, decode of V, load addresses); measured best of 6-12
#pragma unroll
        for (int q = 0; q < 33; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 12, 0);
        }
        // O lives in the accumulator registers across subtiles (without this the loop-carried
        // values are kept in VGPRs and copied around every MFMA)
#pragma unroll
        for (int t = 0; t < NHT; ++t)
#pragma unroll
          for (int db = 0; db < kPfBlocks; ++db) asm volatile("" : "+a"(o[t][db]));
        if (it == n_sub) break;
      }
      wait_vm<0>();  // no load into the ring still in flight
    }
    if (computes && __ballot(over) != 0 && lane == 0) s_redo = 1;
    __syncthreads();
    const bool redo = s_redo != 0;  // uniform over the workgroup
    if (!redo || pass == 1) break;
    m_ref = m_true;  // second pass: the true max, so p <= 1
    __syncthreads();  // every wave has read s_redo and left the last slot before the ring refills
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // nothing in flight into LDS

  // row sums of every head, from the QK waves to all
  float l_tot = 0.0f, lf_tot = 0.0f;
  if (computes) {
    l_tot = l_run + __shfl_xor(l_run, 32, 64);
    lf_tot = lf_run + __shfl_xor(lf_run, 32, 64);
    if (g == 0) s_l[32 * wid + n] = l_tot;
  }
  __syncthreads();
  // lane (head 32 t + n, half g) holds dims 32 (4 wid + db) + 8 (e / 4) + 4 g + e % 4
#pragma unroll
  for (int t = 0; t < NHT; ++t) {
    const int ht = 32 * t + n;
    if (ht >= H) continue;
    if (nsplit == 1) {
      const float lt = s_l[ht];
      const float inv = lt > 0.0f ? a.kv_scale / lt : 0.0f;
      uint16_t *orow = a.out + ((int64_t)r * H + ht) * kVDim + 128 * wid;
#pragma unroll
      for (int db = 0; db < kPfBlocks; ++db) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          bf16x4_t vv;
#pragma unroll
          for (int i = 0; i < 4; ++i) vv[i] = (__bf16)(o[t][db][4 * q + i] * inv);
          *reinterpret_cast<bf16x4_t *>(orow + 32 * db + 8 * q + 4 * g) = vv;
        }
      }
    } else {
      float *po = w.o + (((int64_t)r * nsplit + sp) * H + ht) * kVDim + 128 * wid;
#pragma unroll
      for (int db = 0; db < kPfBlocks; ++db) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          f32x4_t vv;
#pragma unroll
          for (int i = 0; i < 4; ++i) vv[i] = o[t][db][4 * q + i];
          *reinterpret_cast<f32x4_t *>(po + 32 * db + 8 * q + 4 * g) = vv;
        }
      }
    }
  }
  if (hvalid && g == 0) {
    if (nsplit == 1)
      a.lse[(int64_t)r * H + h] = lf_tot > 0.0f ? (m_ref + log2f(lf_tot)) * kLn2 : -INFINITY;
    else
      w.ml[((int64_t)r * nsplit + sp) * H + h] = make_float4(m_ref, l_tot, lf_tot, 0.0f);
  }
}

// Merge the token splits of one row in split order.  Thread = (head, 4 dims).
constexpr int kCombineMaxSplits = 64;
__global__ __launch_bounds__(256) void mla_combine_kernel(const MlaArgs a, const int nsplit, MlaWs w) {
  const int r = blockIdx.y, H = a.n_heads;
  const int q = blockIdx.x * 256 + threadIdx.x;  // (head, dim quad)
  if (q >= H * (kVDim / 4)) return;
  const int h = q / (kVDim / 4), d4 = q % (kVDim / 4);
  const int64_t base = (int64_t)r * nsplit * H + h;
  float M = -INFINITY;
#pragma unroll 8
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, w.ml[base + (int64_t)s * H].x);
  float L = 0.0f, LF = 0.0f;
  f32x4_t acc = {};
  if (M != -INFINITY) {
#pragma unroll 8
    for (int s = 0; s < nsplit; ++s) {
      const float4 ml = w.ml[base + (int64_t)s * H];  // second read hits the cache
      const float f = ml.x == -INFINITY ? 0.0f : exp2f(ml.x - M);
      L += ml.y * f;
      LF += ml.z * f;
      acc += *reinterpret_cast<const f32x4_t *>(w.o + (base + (int64_t)s * H) * kVDim + 4 * d4) * f;
    }
  }
  const float inv = L > 0.0f ? a.kv_scale / L : 0.0f;
  bf16x4_t v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = (__bf16)(acc[i] * inv);
  *reinterpret_cast<bf16x4_t *>(a.out + ((int64_t)r * H + h) * kVDim + 4 * d4) = v;
  if (d4 == 0) a.lse[(int64_t)r * H + h] = LF > 0.0f ? (M + log2f(LF)) * kLn2 : -INFINITY;
}

template <int LAT_FMT, int Q_FMT>
void launch_mla_t(const MlaArgs &a, int nsplit, int tps, MlaWs w, hipStream_t s) {
  dim3 grid((a.n_heads + 15) / 16, nsplit, a.n_q);
  hipLaunchKernelGGL((mla_kernel<LAT_FMT, Q_FMT>), grid, dim3(256), sizeof(int64_t) * (size_t)tps, s, a, nsplit, tps, w);
}

int split_count(int32_t k, int32_t tps) { return k <= 0 ? 1 : (k + tps - 1) / tps; }

}  // namespace

size_t mla_workspace_bytes(int32_t n_q, int32_t n_heads, int32_t k, int32_t tokens_per_split) {
  const int nsplit = split_count(k, tokens_per_split);
  if (nsplit == 1) return 0;
  return (size_t)(a16(4 * (int64_t)n_q * nsplit * n_heads * kVDim) + 16 * (int64_t)n_q * nsplit * n_heads);
}

hipError_t launch_mla(const MlaArgs &a, hipStream_t s) {
  if (a.n_q == 0) return hipSuccess;
  const int tps = a.tokens_per_split;
  const int nsplit = split_count(a.k, tps);
  if (tps > kMaxTps || tps % kSub != 0 || nsplit > kCombineMaxSplits) return hipErrorInvalidValue;
  const MlaWs w = mla_carve(a.ws, a.n_q, a.n_heads, nsplit);
  const int nht = (a.n_heads + 15) / 16;
  if (a.phys && a.q_fmt != 0) return hipErrorInvalidValue;  // physical rows: the decode kernel only
  if (a.q_fmt == 1 && nht > 2 && nht <= kWideMaxTiles) {
    // every head of a row per workgroup: one gather per subtile for all heads
    dim3 grid(1, nsplit, a.n_q);
    const size_t dyn = sizeof(int64_t) * (size_t)tps;
    if (a.lat_fmt == 0) {
      const int nht32 = (a.n_heads + 31) / 32;
      if (nht32 == 2)
        hipLaunchKernelGGL(mla_prefill_kernel<2>, grid, dim3(kPfThreads), dyn, s, a, nsplit, tps, w);
      else if (nht32 == 3)
        hipLaunchKernelGGL(mla_prefill_kernel<3>, grid, dim3(kPfThreads), dyn, s, a, nsplit, tps, w);
      else
        hipLaunchKernelGGL(mla_prefill_kernel<4>, grid, dim3(kPfThreads), dyn, s, a, nsplit, tps, w);
    } else
      hipLaunchKernelGGL(mla_wide_kernel<1>, grid, dim3(kWideThreads), dyn, s, a, nsplit, tps, w);
  } else if (a.lat_fmt == 0) {
    if (a.q_fmt == 0) launch_mla_t<0, 0>(a, nsplit, tps, w, s); else launch_mla_t<0, 1>(a, nsplit, tps, w, s);
  } else {
    if (a.q_fmt == 0) launch_mla_t<1, 0>(a, nsplit, tps, w, s); else launch_mla_t<1, 1>(a, nsplit, tps, w, s);
  }
  if (nsplit > 1) {
    dim3 grid((a.n_heads * (kVDim / 4) + 255) / 256, a.n_q);
    hipLaunchKernelGGL(mla_combine_kernel, grid, dim3(256), 0, s, a, nsplit, w);
  }
  return hipGetLastError();
}

}  // namespace dsa
