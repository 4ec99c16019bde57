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
// One workgroup = (query row, token split, 16-head tile); 4 waves.  Per 32-token
// subtile:
//   gather  the 32 selected latents (through the page table) are decoded to bf16
//           (exact for e4m3 and NVFP4) into LDS twice: token-major Kt[32][576] for
//           Q.K and dim-major Vt[512][32] for P.V (an MFMA fragment needs 8
//           consecutive contraction elements per lane);
//   QK      waves 0-1: S^T[16 tokens][16 heads] = Kt . Q^T, 18 v_mfma_f32_16x16x32_bf16;
//   softmax online, per head, in log2 units; P is rounded to bf16 once and the
//           same rounded values feed both P.V and the row sum;
//   PV      all 4 waves: O^T[128 dims][16 heads] += Vt . P^T over the 32 tokens;
//           the S^T accumulator layout is already the B-operand layout of P^T.
// kv_scale and the query's FP8 scale are applied in fp32 (logits and output),
// never folded into bf16 operands.  Token splits of fixed size are merged in
// a fixed order, so a row's result does not depend on the batch.
#include <math.h>

#include "dsa_device.hpp"
#include "dsa_kernels.hpp"

namespace dsa {

namespace {

constexpr int kSub = 32;     // tokens per subtile
constexpr int kKtLd = 584;   // bf16 per Kt row (576 + 8 pad) = 1168 B
constexpr int kVtLd = 40;    // bf16 per Vt row (32 + 8 pad) = 80 B

struct MlaWs {
  float *o;    // [n_q][nsplit][H][512] unnormalised partial outputs
  float2 *ml;  // [n_q][nsplit][H] (running max in log2 units, sum)
};

__host__ __device__ inline int64_t a16(int64_t x) { return (x + 15) & ~int64_t(15); }

__host__ __device__ inline MlaWs mla_carve(void *ws, int32_t n_q, int32_t H, int nsplit) {
  MlaWs w;
  uint8_t *p = static_cast<uint8_t *>(ws);
  w.o = reinterpret_cast<float *>(p);
  p += a16(4 * (int64_t)n_q * nsplit * H * kVDim);
  w.ml = reinterpret_cast<float2 *>(p);
  return w;
}

__device__ __forceinline__ uint32_t bf16_bits(__bf16 x) { return (uint32_t)__builtin_bit_cast(uint16_t, x); }

template <int LAT_FMT, int Q_FMT>
__global__ __launch_bounds__(256) void mla_kernel(const MlaArgs a, const int nsplit, const int tps, MlaWs w) {
  constexpr int LB = LAT_FMT == 0 ? 576 : 352;
  constexpr int64_t LPB = (int64_t)kPage * LB;
  __shared__ __align__(16) uint16_t s_kt[kSub * kKtLd];
  __shared__ __align__(16) uint16_t s_vt[kVDim * kVtLd];
  __shared__ __align__(16) uint16_t s_p[2][64 * 4];
  __shared__ int64_t s_off[kSub];
  __shared__ float s_red[2][2][16];

  const int ht = blockIdx.x, sp = blockIdx.y, r = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int hl = lane & 15, g = lane >> 4;
  const int H = a.n_heads;
  const int h = ht * 16 + hl;
  const bool hvalid = h < H;
  const int b = a.q_req ? a.q_req[r] : r;
  const bool rvalid = b >= 0 && b < a.n_req;
  if (!rvalid && tid == 0 && sp == 0 && ht == 0) flag_error(a.err, DSA_DEVERR_REQUEST);
  const int ctx = rvalid ? a.ctx_len[b] : 0;
  const int t_beg = sp * tps;
  const int t_end = min(a.k, t_beg + tps);

  // Q^T fragments: lane (head hl, group g) holds q[h][32s + 8g .. +8] for s < 18
  bf16x8_t qf[18];
  float qscale = 1.0f;
  if (hvalid) {
    if constexpr (Q_FMT == 0) {
      const uint16_t *qr = static_cast<const uint16_t *>(a.q) + ((int64_t)r * H + h) * kLatDim;
#pragma unroll
      for (int s = 0; s < 18; ++s) qf[s] = *reinterpret_cast<const bf16x8_t *>(qr + 32 * s + 8 * g);
    } else {
      const uint8_t *qr = static_cast<const uint8_t *>(a.q) + ((int64_t)r * H + h) * kLatDim;
#pragma unroll
      for (int s = 0; s < 18; ++s) {
        const u32x2_t d = *reinterpret_cast<const u32x2_t *>(qr + 32 * s + 8 * g);
        qf[s] = e4m3x8_bf16(d[0], d[1]);
      }
      qscale = a.q_scale[(int64_t)r * H + h];
    }
  } else {
#pragma unroll
    for (int s = 0; s < 18; ++s) qf[s] = bf16x8_t{};
  }
  const float c2 = a.sm_scale * a.kv_scale * qscale * kLog2e;  // logits in log2 units

  float m_run = -INFINITY, l_run = 0.0f;
  f32x4_t o[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) o[dt] = f32x4_t{};

  for (int t0 = t_beg; t0 < t_end; t0 += kSub) {
    // (a) pool offsets of this subtile's tokens (-1: padding or invalid)
    if (tid < kSub) {
      const int i = t0 + tid;
      int64_t off = -1;
      if (i < t_end && rvalid) {
        const int t = a.idx[(int64_t)r * a.idx_ld + i];
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
      s_off[tid] = off;
    }
    __syncthreads();

    // (b) gather + decode: item = (4-token group tg, 8-dim chunk c)
    for (int item = tid; item < (kSub / 4) * 72; item += 256) {
      const int tg = item / 72, c = item - tg * 72;
      bf16x8_t v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t off = s_off[4 * tg + j];
        if (off < 0) {
          v[j] = bf16x8_t{};
        } else if constexpr (LAT_FMT == 0) {
          const u32x2_t d = *reinterpret_cast<const u32x2_t *>(a.pool + off + 8 * c);
          v[j] = e4m3x8_bf16(d[0], d[1]);
        } else {
          if (c < 64) {
            const uint32_t dw = *reinterpret_cast<const uint32_t *>(a.pool + off + 4 * c);
            v[j] = nvfp4x8_bf16(dw, e4m3_f32(a.pool[off + 256 + (c >> 1)]));
          } else {
            const u32x2_t d = *reinterpret_cast<const u32x2_t *>(a.pool + off + 288 + 8 * (c - 64));
            v[j] = e4m3x8_bf16(d[0], d[1]);
          }
        }
        *reinterpret_cast<bf16x8_t *>(s_kt + (4 * tg + j) * kKtLd + 8 * c) = v[j];
      }
      if (c < 64) {
#pragma unroll
        for (int dd = 0; dd < 8; ++dd) {
          u32x2_t pr;
          pr[0] = bf16_bits(v[0][dd]) | (bf16_bits(v[1][dd]) << 16);
          pr[1] = bf16_bits(v[2][dd]) | (bf16_bits(v[3][dd]) << 16);
          *reinterpret_cast<u32x2_t *>(s_vt + (8 * c + dd) * kVtLd + 4 * tg) = pr;
        }
      }
    }
    __syncthreads();

    // (c) S^T = K Q^T on waves 0-1 (16 tokens each)
    float z[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    if (wid < 2) {
      f32x4_t acc = {};
      const uint16_t *krow = s_kt + (16 * wid + hl) * kKtLd + 8 * g;
#pragma unroll
      for (int s = 0; s < 18; ++s) acc = mfma_16x16x32_bf16(*reinterpret_cast<const bf16x8_t *>(krow + 32 * s), qf[s], acc);
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = 16 * wid + 4 * g + i;
        z[i] = s_off[tok] >= 0 ? acc[i] * c2 : -INFINITY;
        mx = fmaxf(mx, z[i]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      if (g == 0) s_red[0][wid][hl] = mx;
    }
    __syncthreads();
    const float m_new = fmaxf(m_run, fmaxf(s_red[0][0][hl], s_red[0][1][hl]));
    const float alpha = m_new == -INFINITY ? 1.0f : exp2f(m_run - m_new);
    if (wid < 2) {
      float ps = 0.0f;
      bf16x4_t pb;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = z[i] == -INFINITY ? 0.0f : exp2f(z[i] - m_new);
        pb[i] = (__bf16)p;
        ps += (float)pb[i];
      }
      *reinterpret_cast<bf16x4_t *>(s_p[wid] + 4 * lane) = pb;
      ps += __shfl_xor(ps, 16, 64);
      ps += __shfl_xor(ps, 32, 64);
      if (g == 0) s_red[1][wid][hl] = ps;
    }
    __syncthreads();
    l_run = l_run * alpha + s_red[1][0][hl] + s_red[1][1][hl];
    m_run = m_new;

    // (d) O^T += Vt . P^T; k-slot j of group g is token 4g+j (j<4) or 16+4g+j-4 (j>=4)
    const bf16x8_t pf = cat4(*reinterpret_cast<const bf16x4_t *>(s_p[0] + 4 * lane),
                             *reinterpret_cast<const bf16x4_t *>(s_p[1] + 4 * lane));
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const uint16_t *vrow = s_vt + (128 * wid + 16 * dt + hl) * kVtLd + 4 * g;
      const bf16x8_t va = cat4(*reinterpret_cast<const bf16x4_t *>(vrow), *reinterpret_cast<const bf16x4_t *>(vrow + 16));
      o[dt] = mfma_16x16x32_bf16(va, pf, o[dt] * alpha);
    }
    __syncthreads();
  }

  // (e) results: lane (head hl, group g) holds dims 128*wid + 16*dt + 4g + i
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
    if (wid == 0 && g == 0) a.lse[(int64_t)r * H + h] = l_run > 0.0f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
  } else {
    const int64_t slot = ((int64_t)r * nsplit + sp) * H + h;
    float *po = w.o + slot * kVDim;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) *reinterpret_cast<f32x4_t *>(po + 128 * wid + 16 * dt + 4 * g) = o[dt];
    if (wid == 0 && g == 0) w.ml[slot] = make_float2(m_run, l_run);
  }
}

// Merge the token splits of one (row, head) in split order: 128 threads x 4 dims.
__global__ __launch_bounds__(128) void mla_combine_kernel(const MlaArgs a, const int nsplit, MlaWs w) {
  const int h = blockIdx.x, r = blockIdx.y, H = a.n_heads;
  const int64_t base = (int64_t)r * nsplit * H + h;
  float M = -INFINITY;
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, w.ml[base + (int64_t)s * H].x);
  float L = 0.0f;
  f32x4_t acc = {};
  if (M != -INFINITY) {
    for (int s = 0; s < nsplit; ++s) {
      const float2 ml = w.ml[base + (int64_t)s * H];
      if (ml.x == -INFINITY) continue;
      const float f = exp2f(ml.x - M);
      L += ml.y * f;
      acc += *reinterpret_cast<const f32x4_t *>(w.o + (base + (int64_t)s * H) * kVDim + 4 * threadIdx.x) * f;
    }
  }
  const float inv = L > 0.0f ? a.kv_scale / L : 0.0f;
  bf16x4_t v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = (__bf16)(acc[i] * inv);
  *reinterpret_cast<bf16x4_t *>(a.out + ((int64_t)r * H + h) * kVDim + 4 * threadIdx.x) = v;
  if (threadIdx.x == 0) a.lse[(int64_t)r * H + h] = L > 0.0f ? (M + log2f(L)) * kLn2 : -INFINITY;
}

template <int LAT_FMT, int Q_FMT>
void launch_mla_t(const MlaArgs &a, int nsplit, int tps, MlaWs w, hipStream_t s) {
  dim3 grid((a.n_heads + 15) / 16, nsplit, a.n_q);
  hipLaunchKernelGGL((mla_kernel<LAT_FMT, Q_FMT>), grid, dim3(256), 0, s, a, nsplit, tps, w);
}

int split_count(int32_t k, int32_t tps) { return k <= 0 ? 1 : (k + tps - 1) / tps; }

}  // namespace

size_t mla_workspace_bytes(int32_t n_q, int32_t n_heads, int32_t k, int32_t tokens_per_split) {
  const int nsplit = split_count(k, tokens_per_split);
  if (nsplit == 1) return 0;
  return (size_t)(a16(4 * (int64_t)n_q * nsplit * n_heads * kVDim) + 8 * (int64_t)n_q * nsplit * n_heads);
}

hipError_t launch_mla(const MlaArgs &a, hipStream_t s) {
  if (a.n_q == 0) return hipSuccess;
  const int tps = a.tokens_per_split;
  const int nsplit = split_count(a.k, tps);
  const MlaWs w = mla_carve(a.ws, a.n_q, a.n_heads, nsplit);
  if (a.lat_fmt == 0) {
    if (a.q_fmt == 0) launch_mla_t<0, 0>(a, nsplit, tps, w, s); else launch_mla_t<0, 1>(a, nsplit, tps, w, s);
  } else {
    if (a.q_fmt == 0) launch_mla_t<1, 0>(a, nsplit, tps, w, s); else launch_mla_t<1, 1>(a, nsplit, tps, w, s);
  }
  if (nsplit > 1)
    hipLaunchKernelGGL(mla_combine_kernel, dim3(a.n_heads, a.n_q), dim3(128), 0, s, a, nsplit, w);
  return hipGetLastError();
}

}  // namespace dsa
