// dcp.hip -- the exact top-k merge across decode-context-parallel shards, emulated on one GPU.
//
// Page "vLLM 为 Kimi K3.1 Pro 提供 Day-0 支持":
//  * section "长上下文：带稀疏 indexer 的 decode 上下文并行": shard s of W holds every W-th
//    token (token t on shard t mod W), and the global top-2048 must be merged across shards
//    before attention;
//  * section "流量减少 10× 的精确 top-k 合并": each shard sends only its best 1.5 k / W
//    candidates, taken from BF16 scores and packed with their score into 32 bits; every shard
//    radix-selects the same global top-k from the gathered candidates; a shard that held more
//    of the top-k than it sent is detected and resends its full local top-k for the row.
// Here the W shards live in one process: shard s's local token i is the row's token
// t = W i + s.  The order is (BF16 score desc, token asc).  Launches:
//   local (row, shard)  the shard's best c = ceil(1.5 k / W) tokens under (BF16 score desc,
//                       local index asc) as 32-bit words key16 << 16 | (0xFFFF - i), written
//                       in local index order (all the shard's tokens if it holds <= c);
//   merge (row)         gathers the W lists and radix-selects the k-th largest word; words
//                       equal to it (the same key and local index on several shards) are taken
//                       in shard order.  Since t = W i + s with s < W, (word desc, shard asc)
//                       is exactly (key desc, t asc).  A shard that holds more than c tokens
//                       (so it sent c) and whose smallest sent word is kept is flagged; a row without a flag
//                       writes its output, a flagged row its flags;
//   local again         flagged (row, shard) pairs only, with k candidates (the resend);
//   merge again         flagged rows only, with the resent lists in place of the flagged
//                       shards' first lists.  More candidates can only raise the k-th word, so
//                       no shard becomes flagged anew: one resend round is enough.
// Limits: 1 <= W <= 8, k <= 2048, rows of at most 65536 W tokens (16-bit local index).
#include "dsa_device.hpp"
#include "dsa_kernels.hpp"

namespace dsa {

namespace {

constexpr int kLocThreads = 1024;
constexpr int kMrgThreads = 512;
constexpr int kMaxCand = kDcpMaxShards * kDcpMaxK;          // 16384 words (64 KB)
constexpr int kMaxBitWords = kDcpMaxShards * 65536 / 32;    // a row's token bitmap (64 KB)

struct DcpWs {
  int32_t *n1;     // [n_rows][8] words sent by each shard
  uint32_t *c1;    // [n_rows][8][c]
  uint32_t *flag;  // [n_rows] shards to resend
  int32_t *n2;     // [n_rows][8]
  uint32_t *c2;    // [n_rows][8][k]
};

__host__ __device__ inline int64_t al16(int64_t x) { return (x + 15) & ~int64_t(15); }

__host__ __device__ inline DcpWs dcp_carve(void *ws, int32_t n_rows, int32_t c, int32_t k) {
  uint8_t *p = static_cast<uint8_t *>(ws);
  DcpWs w;
  w.n1 = reinterpret_cast<int32_t *>(p);
  p += al16(4 * (int64_t)n_rows * kDcpMaxShards);
  w.c1 = reinterpret_cast<uint32_t *>(p);
  p += al16(4 * (int64_t)n_rows * kDcpMaxShards * c);
  w.flag = reinterpret_cast<uint32_t *>(p);
  p += al16(4 * (int64_t)n_rows);
  w.n2 = reinterpret_cast<int32_t *>(p);
  p += al16(4 * (int64_t)n_rows * kDcpMaxShards);
  w.c2 = reinterpret_cast<uint32_t *>(p);
  return w;
}

// Order-preserving 16-bit key of a score's BF16 value (round to nearest even); -0 -> +0.
__device__ __forceinline__ uint32_t bf16_key(float f) {
  if (f == 0.0f) f = 0.0f;
  const uint32_t b = __builtin_bit_cast(uint16_t, (__bf16)f);
  return (b & 0x8000u) ? (~b & 0xFFFFu) : (b | 0x8000u);
}

__device__ __forceinline__ int row_len_checked(const DcpArgs &a, int r) {
  int len = a.row_len[r];
  if (len < 0 || len > a.ld) {
    if (threadIdx.x == 0) flag_error(a.err, DSA_DEVERR_ROW_LEN);
    len = len < 0 ? 0 : (int)a.ld;
  }
  return len;
}

// 256-bin histograms are kept as kCopies copies (one per lane mod kCopies, kHistLd ints per
// bin): the keys of one row share their leading bits, and one copy would send most of a
// wave's atomics to the same address.
constexpr int kCopies = 16;
constexpr int kHistLd = kCopies + 1;

__device__ __forceinline__ void hist_clear(int *h, int nt) {
  for (int q = threadIdx.x; q < 256 * kHistLd; q += nt) h[q] = 0;
}
__device__ __forceinline__ void hist_add(int *h, uint32_t bin) {
  atomicAdd(&h[bin * kHistLd + (threadIdx.x & (kCopies - 1))], 1);
}

// Bin of a 256-bin histogram (counted over keys with the prefix fixed so far) that holds the
// rem-th largest key: thread t < 256 owns bin 255 - t, so an inclusive scan over threads is a
// suffix sum over bins.  Returns the bin and, in `above`, the count in higher bins.
template <int NT>
__device__ int find_bin(const int *h, int rem, int *tmp, int *sh, int &above) {
  const int tid = threadIdx.x;
  int c = 0;
  if (tid < 256)
#pragma unroll
    for (int q = 0; q < kCopies; ++q) c += h[(255 - tid) * kHistLd + q];
  int total;
  const int incl = block_scan_incl<NT>(c, tmp, total);
  if (tid < 256 && incl - c < rem && incl >= rem) {
    sh[0] = 255 - tid;
    sh[1] = incl - c;
  }
  __syncthreads();
  above = sh[1];
  const int b = sh[0];
  __syncthreads();
  return b;
}

// ---- local: one workgroup per (shard, row) ----
// Workgroup ids go round-robin over the eight XCDs (id mod 8), each with its own L2.  A row's
// shards read interleaved elements of the same score lines, so all shards of row r get ids
// congruent to r mod 8: the row is fetched from HBM once, into one L2.
__global__ __launch_bounds__(kLocThreads) void dcp_local_kernel(const DcpArgs a, DcpWs w, int cap, int resend) {
  constexpr int NT = kLocThreads;
  __shared__ uint16_t s_key[65536];  // the shard's keys, local index order
  __shared__ int s_hist[256 * kHistLd];
  __shared__ int s_tmp[NT / 64];
  __shared__ int s_sh[2];
  const int tid = threadIdx.x;
  const int W = a.n_shards;
  const int m = blockIdx.x >> 3, q = m / W, s = m - q * W, r = (blockIdx.x & 7) + 8 * q;
  if (r >= a.n_rows) return;                       // uniform
  if (resend && !((w.flag[r] >> s) & 1u)) return;  // uniform
  const int len = row_len_checked(a, r);
  const float *row = a.scores + (int64_t)r * a.ld;
  int32_t *n_out = (resend ? w.n2 : w.n1) + (int64_t)r * kDcpMaxShards + s;
  uint32_t *out = (resend ? w.c2 : w.c1) + ((int64_t)r * kDcpMaxShards + s) * cap;
  const int ls = len > s ? (len - 1 - s) / W + 1 : 0;  // the shard's tokens in this row (<= 65536)
  if (ls <= cap) {  // the shard sends everything
    for (int i = tid; i < ls; i += NT) out[i] = (bf16_key(row[(int64_t)W * i + s]) << 16) | (uint32_t)(0xFFFF - i);
    if (tid == 0) *n_out = ls;
    return;
  }
  // the keys to LDS, 16 loads in flight per thread
  for (int i0 = 0; i0 < ls; i0 += 16 * NT) {
    float v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int i = i0 + u * NT + tid;
      v[u] = i < ls ? row[(int64_t)W * i + s] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int i = i0 + u * NT + tid;
      if (i < ls) s_key[i] = (uint16_t)bf16_key(v[u]);
    }
  }
  // the cap-th largest key: two 8-bit radix passes over the 16-bit keys
  int tau = 0, gt = 0;
  for (int pass = 0; pass < 2; ++pass) {
    hist_clear(s_hist, NT);
    __syncthreads();  // (the first time also: the keys are in LDS)
    for (int i = tid; i < ls; i += NT) {
      const uint32_t kk = s_key[i];
      if (pass == 0)
        hist_add(s_hist, kk >> 8);
      else if ((int)(kk >> 8) == tau)
        hist_add(s_hist, kk & 255u);
    }
    __syncthreads();
    int above;
    const int b = find_bin<NT>(s_hist, cap - gt, s_tmp, s_sh, above);
    gt += above;
    tau = pass == 0 ? b : (tau << 8) | b;
  }
  const int need_eq = cap - gt;  // tokens with key == tau to take, lowest local index first
  // ordered compaction: thread j takes local indices [j chunk, (j + 1) chunk)
  const int chunk = (ls + NT - 1) / NT;
  const int i0 = min(ls, tid * chunk), i1 = min(ls, i0 + chunk);
  int ng = 0, ne = 0;
  for (int i = i0; i < i1; ++i) {
    const int kk = s_key[i];
    ng += kk > tau;
    ne += kk == tau;
  }
  int tot;
  const int eq_before = block_scan_incl<NT>(ne, s_tmp, tot) - ne;
  const int take_eq = min(ne, max(0, need_eq - eq_before));
  const int cs = ng + take_eq;
  int pos = block_scan_incl<NT>(cs, s_tmp, tot) - cs;
  int eq_seen = 0;
  for (int i = i0; i < i1; ++i) {
    const int kk = s_key[i];
    if (kk > tau || (kk == tau && eq_seen++ < take_eq)) out[pos++] = ((uint32_t)kk << 16) | (uint32_t)(0xFFFF - i);
  }
  if (tid == 0) *n_out = cap;
}

// ---- merge: one workgroup per row ----
__global__ __launch_bounds__(kMrgThreads) void dcp_merge_kernel(const DcpArgs a, DcpWs w, int c, int resend) {
  constexpr int NT = kMrgThreads;
  __shared__ uint32_t s_w[kMaxCand];
  __shared__ uint32_t s_bits[kMaxBitWords];
  __shared__ int s_hist[256 * kHistLd];
  __shared__ int s_tmp[NT / 64];
  __shared__ int s_sh[2];
  __shared__ int s_off[kDcpMaxShards + 1];
  __shared__ uint32_t s_min[kDcpMaxShards];
  __shared__ int s_tie[kDcpMaxShards];
  __shared__ int s_ntie;
  __shared__ uint32_t s_flag;
  const int r = blockIdx.x, tid = threadIdx.x;
  const int W = a.n_shards, k = a.k;
  const uint32_t flagged = resend ? w.flag[r] : 0u;
  if (resend && flagged == 0u) return;  // uniform: the row was finished by the first merge
  const int len = row_len_checked(a, r);
  const int keep = min(k, len);
  int32_t *out = a.idx + (int64_t)r * a.idx_ld;
  if (keep == len) {  // the row holds at most k tokens: all are kept, nobody resends
    for (int i = tid; i < k; i += NT) out[i] = i < len ? i : -1;
    if (tid == 0) {
      w.flag[r] = 0u;
      if (a.resend_mask) a.resend_mask[r] = 0u;
    }
    return;
  }
  // (1) gather the shards' lists in shard order
  if (tid < W)
    s_tie[tid] = ((flagged >> tid) & 1u) ? w.n2[(int64_t)r * kDcpMaxShards + tid] : w.n1[(int64_t)r * kDcpMaxShards + tid];
  if (tid < kDcpMaxShards) s_min[tid] = 0xFFFFFFFFu;
  __syncthreads();
  if (tid == 0) {
    int o = 0;
    for (int s = 0; s < W; ++s) {
      s_off[s] = o;
      o += s_tie[s];  // (s_tie holds the list lengths until the ties are collected)
    }
    s_off[W] = o;
    s_ntie = 0;
    s_flag = 0u;
  }
  __syncthreads();
  const int n = s_off[W];
  // one flat pass over all lists, 8 loads in flight per thread
  for (int j0 = 0; j0 < n; j0 += 8 * NT) {
    uint32_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = j0 + u * NT + tid;
      v[u] = 0u;
      if (j < n) {
        int s = 0;
        while (s + 1 < W && s_off[s + 1] <= j) ++s;
        const int e = j - s_off[s];
        v[u] = ((flagged >> s) & 1u) ? w.c2[((int64_t)r * kDcpMaxShards + s) * k + e]
                                     : w.c1[((int64_t)r * kDcpMaxShards + s) * c + e];
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = j0 + u * NT + tid;
      if (j < n) s_w[j] = v[u];
    }
  }
  __syncthreads();
  // (2) the keep-th largest word: four 8-bit radix passes
  uint32_t prefix = 0u, mask = 0u;
  int rem = keep;
  for (int sh = 24; sh >= 0; sh -= 8) {
    hist_clear(s_hist, NT);
    __syncthreads();
    for (int j = tid; j < n; j += NT) {
      const uint32_t x = s_w[j];
      if ((x & mask) == prefix) hist_add(s_hist, (x >> sh) & 255u);
    }
    __syncthreads();
    int above;
    const int b = find_bin<NT>(s_hist, rem, s_tmp, s_sh, above);
    rem -= above;
    prefix |= (uint32_t)b << sh;
    mask |= 255u << sh;
  }
  const uint32_t tau = prefix;
  const int need_eq = rem;  // words equal to tau to keep, in shard order
  // (3) words equal to tau (at most one per shard) and each shard's smallest word: per-thread
  // minima, then a wave minimum per shard, then one LDS atomic per wave and shard
  uint32_t mn[kDcpMaxShards];
#pragma unroll
  for (int s = 0; s < kDcpMaxShards; ++s) mn[s] = 0xFFFFFFFFu;
#pragma unroll
  for (int s = 0; s < kDcpMaxShards; ++s) {
    if (s < W) {
      for (int j = s_off[s] + tid; j < s_off[s + 1]; j += NT) {
        const uint32_t x = s_w[j];
        mn[s] = min(mn[s], x);
        if (x == tau) s_tie[atomicAdd(&s_ntie, 1)] = s;
      }
    }
  }
#pragma unroll
  for (int s = 0; s < kDcpMaxShards; ++s) {
    if (s < W) {
      const uint32_t m = wave_min_u32(mn[s]);
      if ((tid & 63) == 0) atomicMin(&s_min[s], m);
    }
  }
  __syncthreads();
  // a tied word of shard s is kept iff fewer than need_eq tied words come from lower shards
  auto tie_kept = [&](int s) {
    int lower = 0;
    for (int q = 0; q < s_ntie; ++q) lower += s_tie[q] < s;
    return lower < need_eq;
  };
  auto kept = [&](uint32_t x, int s) { return x > tau || (x == tau && tie_kept(s)); };
  // (4) first merge: a shard that did not send all its tokens and whose smallest sent word is
  // kept may hold more of the top-k
  if (!resend) {
    if (tid < W) {
      const int s = tid;
      const int ls = len > s ? (len - 1 - s) / W + 1 : 0;
      if (s_off[s + 1] - s_off[s] < ls && kept(s_min[s], s)) atomicOr(&s_flag, 1u << s);
    }
    __syncthreads();
    if (tid == 0) {
      w.flag[r] = s_flag;
      if (a.resend_mask) a.resend_mask[r] = s_flag;
    }
    if (s_flag != 0u) return;  // uniform: the second merge writes this row
  }
  // (5) the kept tokens, ascending: a bitmap over the row, then an ordered scan of it
  const int nwords = (len + 31) >> 5;
  for (int q = tid; q < nwords; q += NT) s_bits[q] = 0u;
  __syncthreads();
  for (int s = 0; s < W; ++s)
    for (int j = s_off[s] + tid; j < s_off[s + 1]; j += NT) {
      const uint32_t x = s_w[j];
      if (kept(x, s)) {
        const int t = W * (int)(0xFFFFu - (x & 0xFFFFu)) + s;
        atomicOr(&s_bits[t >> 5], 1u << (t & 31));
      }
    }
  __syncthreads();
  const int per = (nwords + NT - 1) / NT;
  const int q0 = min(nwords, tid * per), q1 = min(nwords, q0 + per);
  int cnt = 0;
  for (int q = q0; q < q1; ++q) cnt += __popc(s_bits[q]);
  int tot;
  int pos = block_scan_incl<NT>(cnt, s_tmp, tot) - cnt;
  for (int q = q0; q < q1; ++q) {
    uint32_t m = s_bits[q];
    while (m) {
      const int b = __ffs(m) - 1;
      m &= m - 1u;
      if (pos < k) out[pos] = 32 * q + b;
      ++pos;
    }
  }
  for (int i = keep + tid; i < k; i += NT) out[i] = -1;
}

}  // namespace

int32_t dcp_candidates(int32_t k, int32_t n_shards) { return (3 * k + 2 * n_shards - 1) / (2 * n_shards); }

size_t dcp_workspace_bytes(int32_t n_rows, int32_t k, int32_t n_shards) {
  const int64_t c = dcp_candidates(k, n_shards);
  return (size_t)(al16(4 * (int64_t)n_rows * kDcpMaxShards) * 2 + al16(4 * (int64_t)n_rows * kDcpMaxShards * c) +
                  al16(4 * (int64_t)n_rows) + 4 * (int64_t)n_rows * kDcpMaxShards * k);
}

hipError_t launch_dcp_topk(const DcpArgs &a, hipStream_t st) {
  if (a.n_rows == 0) return hipSuccess;
  const int c = dcp_candidates(a.k, a.n_shards);
  const DcpWs w = dcp_carve(a.ws, a.n_rows, c, a.k);
  const dim3 lg(8 * ((a.n_rows + 7) / 8) * a.n_shards);
  hipLaunchKernelGGL(dcp_local_kernel, lg, dim3(kLocThreads), 0, st, a, w, c, 0);
  hipLaunchKernelGGL(dcp_merge_kernel, dim3(a.n_rows), dim3(kMrgThreads), 0, st, a, w, c, 0);
  hipLaunchKernelGGL(dcp_local_kernel, lg, dim3(kLocThreads), 0, st, a, w, a.k, 1);
  hipLaunchKernelGGL(dcp_merge_kernel, dim3(a.n_rows), dim3(kMrgThreads), 0, st, a, w, c, 1);
  return hipGetLastError();
}

}  // namespace dsa
