// topk.hip -- exact top-k per row of fp32 scores, lower index wins ties, output ascending.
//
// Page "vLLM 为 Kimi K3.1 Pro 提供 Day-0 支持":
//  * section "K3.1 Pro 中的稀疏注意力": the 2048 best-scoring tokens are kept;
//  * section "低延迟解码：融合的 DSA 解码路径": scorer and an exact top-k are two kernels;
//  * section "流量减少 10× 的精确 top-k 合并": the global top-2048 is radix-selected
//    from a candidate set, and the selection detects when a part held more of the
//    top-k than it offered and redoes that part -- the same shape as here;
//  * section "day 0 零失配 RL": a batch-invariant top-k (a token's result does not
//    depend on its batch) -- here the result is a pure function of the row.
//
// Scores map to order-preserving uint32 keys (-0 -> +0), so the selection is an
// integer problem on (key desc, index asc).  Launches:
//   sample   (one workgroup per long row; skipped for a few short-enough rows, where
//            every collect workgroup draws the same sample itself): runs of 64 scores
//            spread evenly over the row give S sample keys; the threshold `est` is the
//            sample key of rank m(k, len, S), set so that the row holds at least k
//            elements >= est except with negligible probability, and a few k at most.
//   collect  (one workgroup per 8192-score slice): the slice is loaded in one round trip
//            and every element with key >= est (a float compare with est's value; NaNs
//            too) is appended, in index order, to the slice's candidate list (ballot ranks;
//            one barrier).
//   finalize (one workgroup per row): the slices' candidates, concatenated in slice
//            order, are in index order.  The first B entries of every list come in one
//            round trip with the counts; the entries past B, numbered through a prefix
//            over the slices, in a second.  A slice that had more candidates than its list
//            holds is filtered again from the scores.  An LDS radix select finds the
//            exact k-th key tau and the number of ties at tau to keep; an ordered
//            compaction writes the kept indices ascending (and, for the fused decode path
//            -- section "低延迟解码：融合的 DSA 解码路径": the top-k emits the physical KV
//            rows attention reads -- each kept token's pool row * 64 + slot, looked up in
//            the block table as it is written).  Rows of <= 12288 scores skip
//            sample and collect and are loaded whole.  If the candidates are fewer than k
//            or more than LDS holds, the row is selected from the full row instead
//            (always correct, slower).
// The radix passes take their digits from key - min over the keys being selected,
// starting at the top bit of max - min, and count into 16 copies of the histogram
// (one per lane mod 16, odd stride): scores of one row share their leading bits, and a
// plain histogram would send most of a wave's atomics to one address.
// The result is exact whatever est is, so which launches a row goes through never
// changes its output.
#include <type_traits>

#include "dsa_device.hpp"
#include "dsa_kernels.hpp"

namespace dsa {

namespace {

constexpr int kOwnSamples = 4096;     // samples a collect workgroup draws itself
constexpr int kOwnMaxLd = 524288;     // ... when rows are at most this long
constexpr int kOwnMaxRows = 64;       // ... and there are at most this many
constexpr int kMaxSamples = 16384;    // samples of the sample launch
constexpr int kMaxSlices = 1024;
constexpr int kRep = 16;              // histogram copies (one per lane mod 16)
constexpr int kBinLd = 20;            // ints per bin: 16 copies + 4 pad (80-B rows, 16-B aligned)
constexpr int kEstPasses = 2;         // 16 leading bits of the threshold are enough
constexpr int kFinThreads = 512;
constexpr int kFinPer = kShortRow / kFinThreads + 1;  // 25: candidates a finalize thread holds
constexpr int kMidRow = 32768;                        // rows the finalize filters whole (64 scores a thread)

struct TopkWs {
  uint32_t *est;  // [n_rows]
  uint32_t *cnt;  // [n_rows][n_slices] candidates of the slice (may exceed cap)
  uint2 *cand;    // [n_rows][n_slices][cap] (key, index)
  int slice, cap; // tokens per slice, list entries per slice: kSlice, kSliceCap (collect) or
                  // kTileTokens, kTileCap (lists written by the FP8 prefill GEMM)
};

__host__ __device__ inline int64_t align16(int64_t x) { return (x + 15) & ~int64_t(15); }

__host__ __device__ inline TopkWs carve(void *ws, int32_t n_rows, int32_t n_slices, int slice, int cap) {
  uint8_t *p = static_cast<uint8_t *>(ws);
  TopkWs w;
  w.est = reinterpret_cast<uint32_t *>(p);
  p += align16(4 * (int64_t)n_rows);
  w.cnt = reinterpret_cast<uint32_t *>(p);
  p += align16(4 * (int64_t)n_rows * n_slices);
  w.cand = reinterpret_cast<uint2 *>(p);
  w.slice = slice;
  w.cap = cap;
  return w;
}

template <int NT>
struct RadixLds {
  __align__(16) int hist[256 * kBinLd];  // [bin][copy]; never cleared (see radix_select)
  int tmp[NT / 64];
  int tmp2[2][NT / 64];
  int sh[3];
  int list_n;
  uint32_t mm[2 * (NT / 64)];
};

__device__ __forceinline__ int row_len_of(const TopkArgs &a, int r) {
  int len = a.row_len[r];
  // with physical rows the block table must cover the row too
  const int64_t max_len = a.phys != nullptr && a.bt_ld * kPage < a.ld ? a.bt_ld * kPage : a.ld;
  if (len < 0 || len > max_len) {
    if (threadIdx.x == 0 && blockIdx.x == 0) flag_error(a.err, DSA_DEVERR_ROW_LEN);
    len = len < 0 ? 0 : (int)max_len;
  }
  return len;
}

// Band mode helpers.  key_floor / key_ceil give the key of the largest float <= v / smallest
// float >= v, so thresholds computed in fp64 round outward.
__device__ __forceinline__ uint32_t key_floor(double v) {
  float f = (float)v;
  if ((double)f > v) f = nextafterf(f, -INFINITY);
  return score_key(f);
}
__device__ __forceinline__ uint32_t key_ceil(double v) {
  float f = (float)v;
  if ((double)f < v) f = nextafterf(f, INFINITY);
  return score_key(f);
}
// E_r, or +inf when it is not a finite non-negative number (then every token is in the band)
__device__ __forceinline__ double band_bound(const TopkArgs &a, int r) {
  const float e = a.band.e[r];
  return e >= 0.0f && e <= 3.402823466e38f ? (double)e : (double)INFINITY;
}
// In band mode the candidate threshold is lowered by 2 E_r, so the candidates hold every
// token within 2 E_r below the k-th largest score whenever they hold the k largest.
__device__ __forceinline__ uint32_t band_est(const TopkArgs &a, int r, uint32_t est) {
  if (a.band.e == nullptr || est == 0u) return est;
  return key_floor((double)key_score(est) - 2.0 * band_bound(a, r));
}

// Sample rank of the threshold: with x = k S / len sample elements expected above the
// row's k-th score, m = 1.25 x + 6 sqrt(x) + 8 puts the k-th score below est only if a
// Poisson(x) count exceeds its mean by > 6 standard deviations.
__device__ __forceinline__ int sample_rank(int keff, int len, int S) {
  const float x = (float)keff * (float)S / (float)len;
  return (int)ceilf(1.25f * x + 6.0f * sqrtf(x) + 8.0f);
}

// Block-wide (min, max) of one key per thread.
template <int NT>
__device__ __forceinline__ void block_minmax(uint32_t &lo, uint32_t &hi, RadixLds<NT> &R) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  lo = wave_min_u32(lo);
  hi = wave_max_u32(hi);
  if (lane == 0) {
    R.mm[wid] = lo;
    R.mm[NW + wid] = hi;
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    lo = min(lo, R.mm[w]);
    hi = max(hi, R.mm[NW + w]);
  }
  __syncthreads();
}

// Sum of the kRep copies of one histogram bin (one 80-B row), modulo 2^32.
__device__ __forceinline__ uint32_t bin_total(const int *h, int bin) {
  const uint4 *row = reinterpret_cast<const uint4 *>(h + bin * kBinLd);
  uint32_t c = 0;
#pragma unroll
  for (int k = 0; k < kRep / 4; ++k) {
    const uint4 x = row[k];
    c += (x.x + x.y) + (x.z + x.w);
  }
  return c;
}

// Radix select over keys in [kmin, kmax]: `visit(f)` calls f(key) for each of this
// thread's keys.  Returns the m-th largest key (1-based) and in `gt` the number of keys
// strictly larger, using 8-bit digits of key - kmin from the top bit of kmax - kmin down.
// With max_passes below the number of digits the result is the lower edge of the bin that
// holds the m-th largest key: at least m keys are >= it.
// `list` (optional, LDS, list_cap + 64 keys): after the first pass the keys of the chosen bin
// are copied there, and later passes read only those.  visit may call f(key, valid) with
// valid false for a slot that holds no key.
// The histogram is never cleared: thread t reads bin 255 - t before and after each pass
// and takes the difference (wrap-around int arithmetic), which is cheaper than clearing
// 20 KB of LDS per pass.
template <int NT, class Visit>
__device__ __forceinline__ uint32_t radix_select(Visit visit, int m, uint32_t kmin, uint32_t kmax, int max_passes, RadixLds<NT> &R,
                                 int &gt, uint32_t *list = nullptr, int list_cap = 0) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  gt = 0;
  const uint32_t range = kmax - kmin;
  if (range == 0) return kmin;
  int *my = R.hist + (tid & (kRep - 1));
  uint32_t before = tid < 256 ? bin_total(R.hist, 255 - tid) : 0u;
  __syncthreads();  // every snapshot is taken before the first increment
  uint32_t prefix = 0;
  int rem = m, nl = -1;  // nl >= 0: later passes read list[0, nl)
  int hi = 31 - __clz((int)range);
  for (int p = 0; hi >= 0 && p < max_passes; ++p, hi -= 8) {
    const int lo = hi >= 7 ? hi - 7 : 0;
    const uint32_t above = ~((2u << hi) - 1u);  // bits already decided
    // every key takes an atomic (adding 0 unless it is valid and in the chosen bin so far):
    // no branch per key
    auto count = [&](uint32_t key, bool valid = true) {
      const uint32_t u = key - kmin;
      atomicAdd(&my[((u >> lo) & 255u) * kBinLd], valid && (u & above) == prefix ? 1 : 0);
    };
    if (nl >= 0) {
      for (int i = tid; i < nl; i += NT) count(list[i]);
    } else {
      visit(count);
    }
    __syncthreads();
    // thread t < 256 owns bin 255 - t: an inclusive prefix over threads is a suffix over bins
    int c = 0;
    if (tid < 256) {
      const uint32_t after = bin_total(R.hist, 255 - tid);
      c = (int)(after - before);
      before = after;
    }
    int *tmp = R.tmp2[p & 1];  // alternating: no barrier needed before its reuse
    const int incl0 = wave_scan_incl(c);
    if (lane == 63) tmp[wid] = incl0;
    __syncthreads();
    int base = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) base += w < wid ? tmp[w] : 0;
    const int incl = incl0 + base, excl = incl - c;
    if (tid < 256 && excl < rem && incl >= rem) {
      R.sh[0] = 255 - tid;
      R.sh[1] = excl;
      R.sh[2] = c;
      R.list_n = 0;
    }
    __syncthreads();
    prefix |= (uint32_t)R.sh[0] << lo;  // the digit's bits above hi repeat the prefix
    rem -= R.sh[1];
    gt += R.sh[1];
    if (list != nullptr && nl < 0 && lo > 0 && p + 1 < max_passes && R.sh[2] <= list_cap) {
      // the chosen bin's keys to the list, ranked by a block scan; a key outside the bin is
      // written to its lane's pad slot past list_cap (no branch per key)
      const uint32_t mask = ~((1u << lo) - 1u);
      int mine = 0;
      visit([&](uint32_t key, bool valid = true) { mine += valid && ((key - kmin) & mask) == prefix ? 1 : 0; });
      int tot;
      int pos = block_scan_incl<NT>(mine, R.tmp, tot) - mine;
      const int pad = list_cap + lane;
      visit([&](uint32_t key, bool valid = true) {
        const bool in = valid && ((key - kmin) & mask) == prefix;
        list[in ? pos : pad] = key;
        pos += in ? 1 : 0;
      });
      __syncthreads();
      nl = R.sh[2];
    }
  }
  return kmin + prefix;
}

// Exclusive rank of `f` among the block's threads (thread order) and the block total.
template <int NT>
__device__ __forceinline__ int block_rank(bool f, int *tmp, int &total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const unsigned long long bal = __ballot(f);
  const int rank = __popcll(bal & ((1ull << lane) - 1ull));
  if (lane == 0) tmp[wid] = __popcll(bal);
  __syncthreads();
  int off = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int t = tmp[w];
    off += w < wid ? t : 0;
    total += t;
  }
  __syncthreads();
  return off + rank;
}

// log2 of the sample count of a row of length len: about len / 32, from 4096 to kMaxSamples.
__host__ __device__ inline int sample_log2(int64_t len) {
  int lg = 12;
  while ((1 << lg) < kMaxSamples && ((int64_t)32 << lg) < len) ++lg;
  return lg;
}

// Sample position q (4 consecutive scores) of S: runs of 64 starting at multiples of 4,
// spread evenly from 0 to len - 64.
__device__ __forceinline__ float4 load_sample4(const float *row, bool vec, int len, int runs, int q) {
  const int c = q >> 4, part = q & 15;
  const int start = (int)((int64_t)(len - 64) * c / (runs - 1)) & ~3;
  const float *p = row + start + 4 * part;
  if (vec) return *reinterpret_cast<const float4 *>(p);
  return make_float4(p[0], p[1], p[2], p[3]);
}

// The sample buffer is dynamic LDS of 4 * sample_count(ld) bytes: a row never draws more
// samples than a row of length ld, and short rows leave room for more workgroups per CU.
__global__ __launch_bounds__(256) void topk_sample_kernel(const TopkArgs a, TopkWs w) {
  extern __shared__ __align__(16) uint32_t s_smp[];
  __shared__ RadixLds<256> R;
  const int r = blockIdx.x;
  const int len = row_len_of(a, r);
  const int keff = min(a.k, len);
  if (len <= kShortRow || keff >= len) return;  // uniform
  const float *row = a.scores + (int64_t)r * a.ld;
  const bool vec = (reinterpret_cast<uintptr_t>(row) & 15) == 0;
  const int lg = sample_log2(len);  // S = 2^lg samples, about len / 32
  const int S = 1 << lg, lg_runs = lg - 6;
  // runs of 64 start at multiples of 4 spread over [0, len - 64): run c at (len - 64) c / runs
  uint32_t lo = 0xFFFFFFFFu, hi = 0u, t1 = 0u, t2 = 0u;
  // every sample load in flight at once (S / 1024 = 4, 8 or 16 quads per thread): one round
  // trip instead of one per batch of four
  constexpr int kMaxQuads = kMaxSamples / 1024;
  const int nq = S >> 10;  // wave-uniform
  float4 v[kMaxQuads];
#pragma unroll
  for (int u = 0; u < kMaxQuads; ++u) {
    if (u < nq) {
      const int q = threadIdx.x + 256 * u, c = q >> 4, part = q & 15;
      const int start = (int)(((int64_t)(len - 64) * c) >> lg_runs) & ~3;
      const float *p = row + start + 4 * part;
      v[u] = vec ? *reinterpret_cast<const float4 *>(p) : make_float4(p[0], p[1], p[2], p[3]);
    }
  }
#pragma unroll
  for (int u = 0; u < kMaxQuads; ++u) {
    if (u < nq) {
      const uint4 k = make_uint4(score_key(v[u].x), score_key(v[u].y), score_key(v[u].z), score_key(v[u].w));
      *reinterpret_cast<uint4 *>(s_smp + 4 * (threadIdx.x + 256 * u)) = k;
      const uint32_t kk[4] = {k.x, k.y, k.z, k.w};
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        lo = min(lo, kk[e2]);
        hi = max(hi, kk[e2]);
        t2 = kk[e2] > t1 ? t1 : max(t2, kk[e2]);
        t1 = max(t1, kk[e2]);
      }
    }
  }
  const int m = sample_rank(keff, len, S);
  uint32_t est = 0u;
  int gt;
  if (m <= 128) {
    // the threads' top-2 keys are a subset of the sample: their m-th key is a lower bound
    uint32_t l2 = t2, h2 = t1;
    block_minmax<256>(l2, h2, R);
    est = radix_select<256>(
        [&](auto f) {
          f(t1);
          f(t2);
        },
        m, l2, h2, kEstPasses, R, gt);
  } else if (m < S) {
    block_minmax<256>(lo, hi, R);  // also orders the s_smp stores before the reads below
    est = radix_select<256>(
        [&](auto f) {
          for (int i = threadIdx.x; i < S; i += 256) f(s_smp[i]);
        },
        m, lo, hi, kEstPasses, R, gt);
  }
  if (threadIdx.x == 0) w.est[r] = band_est(a, r, est);
}

// Slice element (chunk j, lane quad e) of thread t is beg + 1024 j + 4 t + e.
template <bool OWN>
__global__ __launch_bounds__(256) void topk_collect_kernel(const TopkArgs a, TopkWs w, int n_slices) {
  __shared__ RadixLds<256> R;
  __shared__ __align__(16) int s_tot[8][4];
  __shared__ __align__(16) uint2 s_app[kSliceCap + 64];  // the slice's list, + a pad entry per lane
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int r = blockIdx.y, s = blockIdx.x;
  const int len = row_len_of(a, r);
  const int keff = min(a.k, len);
  if (len <= kShortRow || keff >= len) return;
  uint32_t *my_cnt = w.cnt + (int64_t)r * n_slices + s;
  const int beg = s * kSlice;
  if (beg >= len) {
    if (tid == 0) *my_cnt = 0;
    return;
  }
  const int end = min(len, beg + kSlice);
  const float *row = a.scores + (int64_t)r * a.ld;
  const bool vec = (reinterpret_cast<uintptr_t>(row) & 15) == 0;

  // (1) the slice and (own threshold) the row's samples, all loads in flight at once
  float4 v[8];
  if (vec && end - beg == kSlice) {
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = *reinterpret_cast<const float4 *>(row + beg + 1024 * j + 4 * tid);
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = beg + 1024 * j + 4 * tid;
      v[j].x = i < end ? row[i] : 0.0f;
      v[j].y = i + 1 < end ? row[i + 1] : 0.0f;
      v[j].z = i + 2 < end ? row[i + 2] : 0.0f;
      v[j].w = i + 3 < end ? row[i + 3] : 0.0f;
    }
  }
  uint32_t est;
  if constexpr (OWN) {
    constexpr int kQ = kOwnSamples / 4 / 256;  // 4 sample quads per thread
    uint32_t sk[4 * kQ];
#pragma unroll
    for (int u = 0; u < kQ; ++u) {
      const float4 t = load_sample4(row, vec, len, kOwnSamples / 64, tid + 256 * u);
      sk[4 * u] = score_key(t.x);
      sk[4 * u + 1] = score_key(t.y);
      sk[4 * u + 2] = score_key(t.z);
      sk[4 * u + 3] = score_key(t.w);
    }
    const int m = sample_rank(keff, len, kOwnSamples);
    est = 0u;
    if (m <= 256) {
      // the sample's m-th largest key is >= the m-th largest of the threads' top-3 keys
      // (a subset), so the top-3 keys give a valid, slightly lower threshold from 16/3x
      // fewer keys (at m <= 256 a thread holds about one of the sample's top m, and more
      // than three in about 2% of threads)
      uint32_t t1 = 0u, t2 = 0u, t3 = 0u;
#pragma unroll
      for (int q = 0; q < 4 * kQ; ++q) {
        const uint32_t x = sk[q];
        t3 = max(t3, min(t2, x));
        t2 = max(t2, min(t1, x));
        t1 = max(t1, x);
      }
      uint32_t lo = t3, hi = t1;
      block_minmax<256>(lo, hi, R);
      int gt;
      est = radix_select<256>(
          [&](auto f) {
            f(t1);
            f(t2);
            f(t3);
          },
          m, lo, hi, kEstPasses, R, gt);
    } else if (m < kOwnSamples) {
      uint32_t lo = sk[0], hi = sk[0];
#pragma unroll
      for (int q = 1; q < 4 * kQ; ++q) {
        lo = min(lo, sk[q]);
        hi = max(hi, sk[q]);
      }
      block_minmax<256>(lo, hi, R);
      int gt;
      est = radix_select<256>(
          [&](auto f) {
#pragma unroll
            for (int q = 0; q < 4 * kQ; ++q) f(sk[q]);
          },
          m, lo, hi, kEstPasses, R, gt);
    }
    est = band_est(a, r, est);
    if (s == 0 && tid == 0) w.est[r] = est;
  } else {
    est = w.est[r];
  }
  // (2) ordered append of the elements whose key is >= est.  score_key preserves order (and
  // -0 = +0), so that is a float compare with est's value; a NaN fails "f < e" and is kept
  // whatever its key -- extra candidates never change the selection, which works on keys.
  // Keys are formed only for the appended elements.
  const float ef = est == 0u ? -INFINITY : key_score(est);
  unsigned long long bal[8][4];
  auto take = [&](auto whole) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = beg + 1024 * j + 4 * tid;
      const float f[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
      int cj = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        bal[j][e] = __ballot((decltype(whole)::value || i + e < end) && !(f[e] < ef));
        cj += __popcll(bal[j][e]);
      }
      if (lane == 0) s_tot[j][wid] = cj;
    }
  };
  if (end - beg == kSlice) take(std::true_type{});
  else take(std::false_type{});
  __syncthreads();
  int4 tot[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) tot[j] = *reinterpret_cast<const int4 *>(s_tot[j]);
  const unsigned long long lt = (1ull << lane) - 1ull;
  uint2 *out = w.cand + ((int64_t)r * n_slices + s) * kSliceCap;
  // the list is staged in LDS without a branch per element (an element not kept writes its
  // lane's pad entry) and then written out with coalesced 16-B stores
  int base = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    int rank = base + (wid > 0 ? tot[j].x : 0) + (wid > 1 ? tot[j].y : 0) + (wid > 2 ? tot[j].z : 0);
#pragma unroll
    for (int e = 0; e < 4; ++e) rank += __popcll(bal[j][e] & lt);
    const int i = beg + 1024 * j + 4 * tid;
    const float f[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool keep = (bal[j][e] >> lane) & 1ull;
      s_app[keep && rank < kSliceCap ? rank : kSliceCap + lane] = make_uint2(score_key(f[e]), (uint32_t)(i + e));
      rank += keep ? 1 : 0;
    }
    base += tot[j].x + tot[j].y + tot[j].z + tot[j].w;
  }
  __syncthreads();
  const int n_out = min(base, kSliceCap);
  for (int i = 2 * tid; i < n_out; i += 512) {
    if (i + 1 < n_out)
      *reinterpret_cast<uint4 *>(out + i) = *reinterpret_cast<const uint4 *>(s_app + i);
    else
      out[i] = s_app[i];
  }
  if (tid == 0) *my_cnt = (uint32_t)base;
}

// Ordered compaction, 512 elements per round: keep key > tau and the first need_eq keys
// == tau in index order.  Used by the rare full-row path.
template <class Load, class Emit>
__device__ __forceinline__ void compact_rounds(Load load, int n, uint32_t tau, int need_eq, Emit emit, int *tmp) {
  const int tid = threadIdx.x;
  int written = 0, eq_seen = 0;
  for (int c0 = 0; c0 < n; c0 += kFinThreads) {
    const int i = c0 + tid;
    uint32_t key = 0;
    if (i < n) key = load(i);
    const bool gtf = i < n && key > tau;
    const bool eqf = i < n && key == tau;
    int eq_tot, sel_tot;
    const int eq_rank = block_rank<kFinThreads>(eqf, tmp, eq_tot);
    const bool sel = gtf || (eqf && eq_seen + eq_rank < need_eq);
    const int pos = block_rank<kFinThreads>(sel, tmp, sel_tot);
    if (sel) emit(written + pos, i);
    written += sel_tot;
    eq_seen += eq_tot;
  }
}

// Exact selection and ordered output of keys held in registers: thread t holds cnt keys rk[]
// whose indices idx_of(q) increase with q, and every key of thread t comes before every key of
// thread t + 1 in index order.  Keeps the keff largest (ties to the lower index): emit(pos, q,
// sel) is called for every slot q, and the kept ones (sel) get positions 0 .. keff - 1 in index
// order.  `list` (LDS, list_cap + 64 keys) is the radix select's list.
template <int PER, class IdxOf, class Emit>
__device__ __forceinline__ void select_from_regs(const uint32_t (&rk)[PER], int cnt, IdxOf idx_of, int keff,
                                                 RadixLds<kFinThreads> &R, Emit emit, uint32_t *list,
                                                 int list_cap) {
  constexpr int NT = kFinThreads;
  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    lo = min(lo, q < cnt ? rk[q] : 0xFFFFFFFFu);
    hi = max(hi, q < cnt ? rk[q] : 0u);
  }
  block_minmax<NT>(lo, hi, R);  // its barriers also end every earlier read of `list`
  int gt;
  const uint32_t tau = radix_select<NT>(
      [&](auto f) {
#pragma unroll
        for (int q = 0; q < PER; ++q) f(rk[q], q < cnt);
      },
      keff, lo, hi, 32, R, gt, list, list_cap);
  // ordered compaction: keep key > tau, and the first need_eq keys == tau in index order
  const int need_eq = keff - gt;
  int ce = 0, cg = 0;
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    cg += (q < cnt && rk[q] > tau) ? 1 : 0;
    ce += (q < cnt && rk[q] == tau) ? 1 : 0;
  }
  int tot;
  const int eq_excl = block_scan_incl<NT>(ce, R.tmp, tot) - ce;
  const int cs = cg + min(ce, max(0, need_eq - eq_excl));
  int pos = block_scan_incl<NT>(cs, R.tmp, tot) - cs;
  int eq_seen = eq_excl;
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const bool eq = q < cnt && rk[q] == tau;
    const bool sel = q < cnt && (rk[q] > tau || (eq && eq_seen < need_eq));
    eq_seen += eq ? 1 : 0;
    emit(pos, q, sel);
    pos += sel ? 1 : 0;
  }
}

// Exact selection and ordered output of the n >= 1 candidates in s_key / s_idx (index order;
// both arrays hold list_cap + 64 entries): thread t holds candidates [t per, t per + cnt) in
// registers (cnt <= per <= PER).  s_key doubles as the radix select's list once the registers
// are loaded.  pre(index) is evaluated for every slot as soon as its index is in a register (its
// loads fly during the radix passes).  The kept (index, pre(index)) pairs are staged in s_idx /
// s_key at their output positions (a slot not kept writes its lane's pad entry), and written out
// in order as emit(position, index, pre(index)): no branch per candidate.
template <int PER, class Pre, class Emit>
__device__ __forceinline__ void select_write(uint32_t *s_key, int32_t *s_idx, int n, int per, int keff,
                                             RadixLds<kFinThreads> &R, Pre pre, Emit emit, int list_cap) {
  const int tid = threadIdx.x;
  const int b0 = min(n, tid * per);
  const int cnt = min(n, b0 + per) - b0;
  uint32_t rk[PER];
  int32_t ri[PER], pv[PER];
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int j = min(b0 + q, n - 1);  // slots past cnt read a real candidate and are ignored
    rk[q] = s_key[j];
    ri[q] = s_idx[j];
  }
#pragma unroll
  for (int q = 0; q < PER; ++q) pv[q] = pre(ri[q]);
  const int pad = list_cap + (tid & 63);
  select_from_regs<PER>(
      rk, cnt, [&](int q) { return q; }, keff, R,
      [&](int pos, int q, bool sel) {
        const int d = sel ? pos : pad;
        s_idx[d] = ri[q];
        s_key[d] = (uint32_t)pv[q];
      },
      s_key, list_cap);
  __syncthreads();
  for (int i = tid; i < keff; i += kFinThreads) emit(i, s_idx[i], (int32_t)s_key[i]);
}

// select_write with the register bound picked from a few sizes (per = candidates per thread).
template <class Pre, class Emit>
__device__ __forceinline__ void select_write_any(uint32_t *s_key, int32_t *s_idx, int n, int per, int keff,
                                                 RadixLds<kFinThreads> &R, Pre pre, Emit emit,
                                                 int list_cap = kShortRow) {
  if (per <= 5) select_write<5>(s_key, s_idx, n, per, keff, R, pre, emit, list_cap);
  else if (per <= 9) select_write<9>(s_key, s_idx, n, per, keff, R, pre, emit, list_cap);
  else if (per <= 13) select_write<13>(s_key, s_idx, n, per, keff, R, pre, emit, list_cap);
  else if (per <= 17) select_write<17>(s_key, s_idx, n, per, keff, R, pre, emit, list_cap);
  else select_write<kFinPer>(s_key, s_idx, n, per, keff, R, pre, emit, list_cap);
}

// Band mode's first pass over the n candidates in s_key / s_idx (index order): thread t takes
// [t per, t per + cnt) into registers; T^ = the keff-th largest key by radix select (s_key
// doubles as its list); lo_key / hi_key = the band's edges.  When the band stays at or above
// `est` (the candidates' threshold; pass 0 when the candidates are the whole row), the surely
// kept tokens (key > hi_key) and the band are written in index order through two block scans
// and true is returned; otherwise nothing is written and the caller classifies the whole row.
template <int PER>
__device__ __forceinline__ bool band_from_regs(uint32_t *s_key, int32_t *s_idx, int n, int per, int keff,
                                               double e2, uint32_t est, RadixLds<kFinThreads> &R, uint2 *list,
                                               uint2 *bpos, int &written, int &bw, uint32_t &lo_key,
                                               uint32_t &hi_key) {
  constexpr int NT = kFinThreads;
  static_assert(kBandListCap + kBandCap <= kShortRow, "the list and the band positions are staged in s_key");
  const int tid = threadIdx.x;
  const int b0 = min(n, tid * per);
  const int cnt = min(n, b0 + per) - b0;
  uint32_t rk[PER];
  int32_t ri[PER];
  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int j = min(b0 + q, n - 1);  // slots past cnt read a real candidate and are ignored
    rk[q] = s_key[j];
    ri[q] = s_idx[j];
    lo = min(lo, q < cnt ? rk[q] : 0xFFFFFFFFu);
    hi = max(hi, q < cnt ? rk[q] : 0u);
  }
  block_minmax<NT>(lo, hi, R);  // its barriers also end every read of s_key
  int gt;
  const uint32_t tau = radix_select<NT>(
      [&](auto f) {
#pragma unroll
        for (int q = 0; q < PER; ++q) f(rk[q], q < cnt);
      },
      keff, lo, hi, 32, R, gt, s_key, kShortRow);
  const double tv = (double)key_score(tau);
  lo_key = key_floor(tv - e2);
  hi_key = key_ceil(tv + e2);
  if (lo_key < est) return false;  // uniform
  int cs = 0, cb = 0;
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const bool sure = q < cnt && rk[q] > hi_key;
    const bool band = q < cnt && !sure && rk[q] >= lo_key;
    cs += (sure || band) ? 1 : 0;
    cb += band ? 1 : 0;
  }
  int tot, btot;
  int pos = block_scan_incl<NT>(cs, R.tmp, tot) - cs;
  int bp = block_scan_incl<NT>(cb, R.tmp, btot) - cb;
  // staged in LDS without a branch per candidate: list entry p as (s_key[p] = sure, s_idx[p] =
  // index), band entry b as its list position in s_key[kBandListCap + b]; a slot that writes
  // nothing goes to its lane's pad entry.  Then both lists are written out coalesced.
  const int pad = kShortRow + (tid & 63);
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const bool sure = q < cnt && rk[q] > hi_key;
    const bool band = q < cnt && !sure && rk[q] >= lo_key;
    const bool keep = sure || band;
    const int d = keep && pos < kBandListCap ? pos : pad;
    s_idx[d] = ri[q];
    s_key[d] = sure ? 1u : 0u;
    s_key[band && bp < kBandCap ? kBandListCap + bp : pad] = (uint32_t)pos;
    pos += keep ? 1 : 0;
    bp += band ? 1 : 0;
  }
  __syncthreads();
  const int nlw = min(tot, kBandListCap), nbw = min(btot, kBandCap);
  for (int i = tid; i < nlw; i += NT) list[i] = make_uint2(s_key[i] ? 0xFFFFFFFFu : 0u, (uint32_t)s_idx[i]);
  for (int i = tid; i < nbw; i += NT) {
    const int p = (int)s_key[kBandListCap + i];  // a band entry past the list's capacity: none
    bpos[i] = p < kBandListCap ? make_uint2((uint32_t)p, (uint32_t)s_idx[p]) : make_uint2(0xFFFFFFFFu, 0u);
  }
  written = tot;
  bw = btot;
  return true;
}

template <class... Args>
__device__ __forceinline__ bool band_from_regs_any(int per, Args &&...args) {
  if (per <= 5) return band_from_regs<5>(args...);
  if (per <= 9) return band_from_regs<9>(args...);
  if (per <= 13) return band_from_regs<13>(args...);
  if (per <= 17) return band_from_regs<17>(args...);
  return band_from_regs<kFinPer>(args...);
}

// Ordered filter of scores [beg, end) of `row` against ef (collect's test: kept unless x < ef,
// so NaNs are kept) into s_key / s_idx from position `base`, keeping positions below `cap_end`;
// returns how many passed.  Wave w takes the contiguous range beg + 64 PERW w .. + 64 PERW, its
// lane l the scores 64 j + l of it (coalesced loads, clamped to the row so none is skipped by a
// branch), ranks come from ballots, and every lane stores: one that does not keep its score
// writes a pad slot past kShortRow (s_key / s_idx hold kShortRow + 64 entries).  The range must
// hold at most NT / 64 x 64 PERW scores.
template <int NT, int PERW>
__device__ __forceinline__ int filter_append(const float *row, int beg, int end, float ef, uint32_t *s_key,
                                             int32_t *s_idx, int base, int cap_end, int *tmp) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int w0 = beg + 64 * PERW * wid;
  float x[PERW];
#pragma unroll
  for (int j = 0; j < PERW; ++j) x[j] = row[min(w0 + 64 * j + lane, end - 1)];
  int cw = 0;
#pragma unroll
  for (int j = 0; j < PERW; ++j) cw += __popcll(__ballot(w0 + 64 * j + lane < end && !(x[j] < ef)));
  if (lane == 0) tmp[wid] = cw;
  __syncthreads();
  int run = base, total = 0;
#pragma unroll
  for (int v = 0; v < NW; ++v) {
    const int t = tmp[v];
    run += v < wid ? t : 0;
    total += t;
  }
  __syncthreads();
  const unsigned long long lt = (1ull << lane) - 1ull;
  const int pad = kShortRow + lane;
#pragma unroll
  for (int j = 0; j < PERW; ++j) {
    const int i = w0 + 64 * j + lane;
    const bool keep = i < end && !(x[j] < ef);
    const unsigned long long b = __ballot(keep);
    const int pos = run + __popcll(b & lt);
    const int dst = keep && pos < cap_end ? pos : pad;
    s_key[dst] = score_key(x[j]);
    s_idx[dst] = i;
    run += __popcll(b);
  }
  return total;
}

template <bool BAND>
__global__ __launch_bounds__(kFinThreads) void topk_finalize_kernel(const TopkArgs a, TopkWs w, int n_slices) {
  constexpr int NT = kFinThreads;
  constexpr int kBatch = 12;  // row-score loads in flight per thread (short rows)
  constexpr int kSpec = 20;   // speculative candidate loads per thread (B = 16 up to 640 slices)
  constexpr int kXBatch = 4;  // loads of entries past B in flight per thread
  static_assert(8 * kMaxSlices <= NT * kSpec, "a speculative share of 8 entries must cover every slice");
  static_assert(kMaxSlices <= 2 * NT, "the slice counts are loaded two per thread");
  __shared__ uint32_t s_key[kShortRow + 64];  // + a pad slot per lane (filter_append)
  __shared__ int32_t s_idx[kShortRow + 64];
  __shared__ int s_base[kMaxSlices + 1];
  __shared__ int s_xbase[kMaxSlices + 1];
  __shared__ RadixLds<NT> R;
  __shared__ int s_flag;
  const int tid = threadIdx.x;
  const int r = blockIdx.x;
  // When rows may be long, one round trip loads the row's length, the slice counts and,
  // speculatively, the first B entries of every slice's candidate list (B: a power of two,
  // B x n_slices <= NT x kSpec).  None of these addresses depends on the length, and all
  // are in bounds for every row: the lists are w.cap long, and entries past a slice's
  // count (or the whole of a short row's lists) are read but not used.
  const uint32_t *cnt = w.cnt + (int64_t)r * n_slices;
  const int cap = w.cap;
  const uint2 *cand = w.cand + (int64_t)r * n_slices * cap;
  int lgB = 3;  // B = 8 keeps B x n_slices <= NT x kSpec up to kMaxSlices = 1024 slices
  while ((2 << lgB) * n_slices <= NT * kSpec && (2 << lgB) <= cap) ++lgB;
  uint2 e[kSpec];
  int c_first = 0, c_second = 0;  // counts of slices tid and tid + NT (n_slices <= 2 NT)
  if (a.ld > kShortRow) {  // uniform
#pragma unroll
    for (int q = 0; q < kSpec; ++q) {
      const int x = tid + NT * q, s = x >> lgB, j = x & ((1 << lgB) - 1);
      e[q] = s < n_slices ? cand[(int64_t)s * cap + j] : make_uint2(0u, 0u);
    }
    c_first = tid < n_slices ? (int)cnt[tid] : 0;
    c_second = tid + NT < n_slices ? (int)cnt[tid + NT] : 0;
  }
  const int len = row_len_of(a, r);
  int32_t *out = a.idx + (int64_t)r * a.idx_ld;
  const float *row = a.scores + (int64_t)r * a.ld;
  // physical rows: the row's block-table row (NULL for a bad request: every entry -1)
  int32_t *pout = nullptr;
  const int32_t *btr = nullptr;
  if (a.phys != nullptr) {
    pout = a.phys + (int64_t)r * a.idx_ld;
    const int b = a.q_req[r];
    if (b >= 0 && b < a.n_req) btr = a.bt + (int64_t)b * a.bt_ld;
    else if (tid == 0) flag_error(a.err, DSA_DEVERR_REQUEST);
  }
  const int keff = min(a.k, len);
  // physical row of token t from its block id (read from the block table beforehand)
  auto phys_from = [&](int32_t blk, int t) -> int32_t {
    if (btr == nullptr) return -1;
    if (blk < 0 || blk >= a.pool_rows) {
      flag_error(a.err, DSA_DEVERR_BLOCK_RANGE);
      return -1;
    }
    return blk * kPage + (t & (kPage - 1));
  };
  auto block_of = [&](int32_t t) -> int32_t { return btr != nullptr ? btr[t >> 6] : -1; };
  auto emit3 = [&](int pos, int32_t i, int32_t blk) {
    out[pos] = i;
    if (pout) pout[pos] = phys_from(blk, i);
  };
  auto emit = [&](int pos, int32_t i) { emit3(pos, i, pout ? block_of(i) : -1); };

  if (keff >= len) {  // keep everything (also len == 0)
    if (BAND && tid == 0) {
      a.band.cnt[2 * r] = -1;
      a.band.cnt[2 * r + 1] = 0;
    }
    for (int i = tid; i < a.k; i += NT) {
      if (i < len) {
        emit(i, i);
      } else {
        out[i] = -1;
        if (pout) pout[i] = -1;
      }
    }
    return;
  }
  int n = 0;
  bool ok;
  if (len <= kShortRow) {
    // loads clamped to the row and stores to a pad slot past the row: no branch per element
    for (int i0 = 0; i0 < len; i0 += NT * kBatch) {
      float x[kBatch];
#pragma unroll
      for (int q = 0; q < kBatch; ++q) x[q] = row[min(i0 + NT * q + tid, len - 1)];
#pragma unroll
      for (int q = 0; q < kBatch; ++q) {
        const int i = i0 + NT * q + tid;
        const int dst = i < len ? i : kShortRow + (tid & 63);
        s_key[dst] = score_key(x[q]);
        s_idx[dst] = i;
      }
    }
    n = len;
    ok = true;
  } else if (len <= kMidRow) {
    // A row of up to kMidRow scores, where k is a large share of the row and the slices'
    // lists run long or overflow: filter the whole row against est instead, in index order,
    // in one round trip.
    const uint32_t est = w.est[r];
    const float ef = est == 0u ? -INFINITY : key_score(est);
    const int tot = filter_append<NT, kMidRow / NT>(row, 0, len, ef, s_key, s_idx, 0, kShortRow, R.tmp);
    n = tot;
    ok = n >= keff && n <= kShortRow;
  } else {
    // (len > kShortRow implies ld > kShortRow: e[] and c_first are loaded)
    if (tid == 0) s_flag = 0;
    __syncthreads();
    // exclusive prefix of the slices' candidate counts; s_flag bit 0: a list overflowed,
    // bit 1: a list is longer than B
    int run = 0;
    for (int s0 = 0; s0 < n_slices; s0 += NT) {
      const int s = s0 + tid;
      const int c = s0 == 0 ? c_first : s0 == NT ? c_second : s < n_slices ? (int)cnt[s] : 0;
      // one flag update per wave (a per-thread atomic on one word serialises)
      const bool ovf = __ballot(c > cap) != 0ull, lng = __ballot(c <= cap && c > (1 << lgB)) != 0ull;
      if ((tid & 63) == 0 && (ovf || lng)) atomicOr(&s_flag, (ovf ? 1 : 0) | (lng ? 2 : 0));
      int total;
      const int incl = block_scan_incl<NT>(c, R.tmp, total);
      if (s < n_slices) s_base[s] = run + incl - c;
      run += total;
    }
    if (tid == 0) s_base[n_slices] = run;
    __syncthreads();
    n = run;
    ok = n >= keff && n <= kShortRow;
    if (ok) {
      // every slice base first (all LDS reads in flight together), then the placements
      int sb0[kSpec], sb1[kSpec];
#pragma unroll
      for (int q = 0; q < kSpec; ++q) {
        const int s = min((tid + NT * q) >> lgB, n_slices - 1);
        sb0[q] = s_base[s];
        sb1[q] = s_base[s + 1];
      }
      const int pad = kShortRow + (tid & 63);  // where an entry not placed is written
#pragma unroll
      for (int q = 0; q < kSpec; ++q) {
        const int x = tid + NT * q, s = x >> lgB, j = x & ((1 << lgB) - 1);
        const int c = sb1[q] - sb0[q];
        const int d = s < n_slices && c <= cap && j < c ? sb0[q] + j : pad;
        s_key[d] = e[q].x;
        s_idx[d] = (int32_t)e[q].y;
      }
      if (s_flag & 2) {  // lists longer than B: only their entries past the first B
        // x(s) = entries of slice s past B (0 for short and for overflowed lists); the
        // extras are numbered 0..X-1 in slice order through the exclusive prefix s_xbase
        const int B = 1 << lgB;
        int xrun = 0;
        for (int s0 = 0; s0 < n_slices; s0 += NT) {
          const int s = s0 + tid;
          const int c = s < n_slices ? s_base[s + 1] - s_base[s] : 0;
          const int x = c > B && c <= cap ? c - B : 0;
          int total;
          const int incl = block_scan_incl<NT>(x, R.tmp, total);
          if (s < n_slices) s_xbase[s] = xrun + incl - x;
          xrun += total;
        }
        if (tid == 0) s_xbase[n_slices] = xrun;
        __syncthreads();
        int top = 1;  // largest power of two <= n_slices
        while (2 * top <= n_slices) top <<= 1;
        for (int p0 = 0; p0 < xrun; p0 += NT * kXBatch) {
          // extra p lies in the last slice sl with s_xbase[sl] <= p (the batch's searches
          // interleaved); positions past X load entry 0 of slice 0, so every load is in
          // bounds and none waits on a branch
          int sl[kXBatch];
#pragma unroll
          for (int q = 0; q < kXBatch; ++q) sl[q] = 0;
          for (int step = top; step > 0; step >>= 1) {
#pragma unroll
            for (int q = 0; q < kXBatch; ++q) {
              const int c = sl[q] + step;
              if (c <= n_slices && s_xbase[c] <= p0 + NT * q + tid) sl[q] = c;
            }
          }
          int dst[kXBatch];
          uint2 f[kXBatch];
#pragma unroll
          for (int q = 0; q < kXBatch; ++q) {
            const int p = p0 + NT * q + tid;
            const bool v = p < xrun;
            const int lo = v ? sl[q] : 0, j = v ? B + p - s_xbase[lo] : 0;
            dst[q] = v ? s_base[lo] + j : -1;
            f[q] = cand[(int64_t)lo * cap + j];
          }
#pragma unroll
          for (int q = 0; q < kXBatch; ++q) {
            const int d = dst[q] >= 0 ? dst[q] : pad;
            s_key[d] = f[q].x;
            s_idx[d] = (int32_t)f[q].y;
          }
        }
      }
      if (s_flag & 1) {  // slices whose list overflowed: filter them again from the scores
        const uint32_t est = w.est[r];
        const float ef = est == 0u ? -INFINITY : key_score(est);
        // each overflowing slice in one round trip (filter_append)
        static_assert(kSlice <= kFinThreads * 16 && kTileTokens <= kSlice, "a slice fits one pass");
        for (int s = 0; s < n_slices; ++s) {
          if (s_base[s + 1] - s_base[s] <= cap) continue;  // uniform
          const int beg = s * w.slice, end = min(len, beg + w.slice);
          filter_append<NT, kSlice / NT>(row, beg, end, ef, s_key, s_idx, s_base[s], s_base[s + 1], R.tmp);
        }
      }
    }
  }
  __syncthreads();
  if constexpr (BAND) {
    uint2 *list = a.band.list + (int64_t)r * kBandListCap;
    uint2 *bpos = a.band.pos + (int64_t)r * kBandCap;
    const double e2 = 2.0 * band_bound(a, r);
    int written = 0, bw = 0;
    uint32_t lo_key, hi_key;
    bool done = false;
    if (ok) {
      // the candidates hold the keff largest: T^ and the band from registers, unless the band
      // reaches below the collect's threshold (then the whole row is classified below)
      const int per = ((n + NT - 1) / NT) | 1;
      done = band_from_regs_any(per, s_key, s_idx, n, per, keff, e2, len <= kShortRow ? 0u : w.est[r], R, list,
                                bpos, written, bw, lo_key, hi_key);
    } else {
      // T^ over the whole row
      auto load = [&](int i) { return score_key(row[i]); };
      uint32_t lo = 0xFFFFFFFFu, hi = 0u;
      for (int i = tid; i < len; i += NT) {
        const uint32_t k = load(i);
        lo = min(lo, k);
        hi = max(hi, k);
      }
      block_minmax<NT>(lo, hi, R);
      int gt;
      const uint32_t tau = radix_select<NT>(
          [&](auto f) {
            for (int i = tid; i < len; i += NT) f(load(i));
          },
          keff, lo, hi, 32, R, gt, s_key, kShortRow);
      const double tv = (double)key_score(tau);
      lo_key = key_floor(tv - e2);
      hi_key = key_ceil(tv + e2);
    }
    if (!done) {
      // ordered compaction over the whole row of the surely kept tokens (key > hi_key, listed
      // with key all ones) and the band (listed with key 0 until rescored)
      for (int c0 = 0; c0 < len; c0 += NT) {
        const int i = c0 + tid;
        const uint32_t key = i < len ? score_key(row[i]) : 0u;
        const bool sure = i < len && key > hi_key;
        const bool band = i < len && !sure && key >= lo_key;
        int tot, btot;
        const int pos = written + block_rank<NT>(sure || band, R.tmp, tot);
        const int bp = bw + block_rank<NT>(band, R.tmp, btot);
        if ((sure || band) && pos < kBandListCap) list[pos] = make_uint2(sure ? 0xFFFFFFFFu : 0u, (uint32_t)i);
        if (band && bp < kBandCap && pos < kBandListCap) bpos[bp] = make_uint2((uint32_t)pos, (uint32_t)i);
        written += tot;
        bw += btot;
      }
    }
    if (tid == 0) {
      a.band.cnt[2 * r] = written;
      a.band.cnt[2 * r + 1] = bw;
    }
  } else if (ok) {
    // thread t takes candidates [t per, t per + cnt) into registers (per is odd, so the
    // strided LDS reads of a wave hit distinct banks); the loops are unrolled for a bound
    // on per picked from a few sizes
    const int per = ((n + NT - 1) / NT) | 1;
    select_write_any(s_key, s_idx, n, per, keff, R, block_of, emit3);
  } else {
    // exact selection over the whole row, straight from global memory
    auto load = [&](int i) { return score_key(row[i]); };
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
    for (int i = tid; i < len; i += NT) {
      const uint32_t k = load(i);
      lo = min(lo, k);
      hi = max(hi, k);
    }
    block_minmax<NT>(lo, hi, R);
    int gt;
    const uint32_t tau = radix_select<NT>(
        [&](auto f) {
          for (int i = tid; i < len; i += NT) f(load(i));
        },
        keff, lo, hi, 32, R, gt, s_key, kShortRow);
    compact_rounds(load, len, tau, keff - gt, emit, R.tmp);
  }
  if (BAND) return;  // the second pass writes the row
  for (int i = keff + tid; i < a.k; i += NT) {
    out[i] = -1;
    if (pout) pout[i] = -1;
  }
}

// Band mode, second pass (one workgroup per row): the kept tokens from the first pass's list,
// whose band keys are now exact, or -- for a row whose band overflowed and was rescored in
// place -- from the whole score row.
// The list arrays are dynamic LDS of cap + 64 entries each (cap = band_select_cap(k): the list
// is about k entries plus the band, so two workgroups fit per CU at k = 2048); a longer list
// takes the whole-row path.
__global__ __launch_bounds__(kFinThreads) void topk_band_select_kernel(const TopkArgs a, const int cap) {
  constexpr int NT = kFinThreads;
  extern __shared__ __align__(16) uint32_t s_dyn[];
  uint32_t *const s_key = s_dyn;                                              // [cap + 64]
  int32_t *const s_idx = reinterpret_cast<int32_t *>(s_dyn + cap + 64);       // [cap + 64]
  __shared__ RadixLds<NT> R;
  const int tid = threadIdx.x, r = blockIdx.x;
  const int len = row_len_of(a, r);
  const int keff = min(a.k, len);
  const int nl = a.band.cnt[2 * r], nb = a.band.cnt[2 * r + 1];
  if (nl < 0) return;  // the first pass kept the whole row
  int32_t *out = a.idx + (int64_t)r * a.idx_ld;
  auto emit = [&](int pos, int32_t i) { out[pos] = i; };
  if (nb <= kBandCap && nl >= keff && nl <= cap) {
    const uint2 *list = a.band.list + (int64_t)r * kBandListCap;
    for (int i = tid; i < nl; i += NT) {
      const uint2 e = list[i];
      s_key[i] = e.x;
      s_idx[i] = (int32_t)e.y;
    }
    __syncthreads();
    const int per = ((nl + NT - 1) / NT) | 1;
    select_write_any(
        s_key, s_idx, nl, per, keff, R, [](int32_t) { return 0; }, [&](int pos, int32_t i, int32_t) { emit(pos, i); },
        cap);
  } else if (nb <= kBandCap && nl >= keff) {
    // a list longer than the LDS arrays (nl <= keff + nb <= kBandListCap): the same selection
    // read straight from the list in global memory
    const uint2 *list = a.band.list + (int64_t)r * kBandListCap;
    auto lkey = [&](int i) { return list[i].x; };
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
    for (int i = tid; i < nl; i += NT) {
      const uint32_t k = lkey(i);
      lo = min(lo, k);
      hi = max(hi, k);
    }
    block_minmax<NT>(lo, hi, R);
    int gt;
    const uint32_t tau = radix_select<NT>(
        [&](auto f) {
          for (int i = tid; i < nl; i += NT) f(lkey(i));
        },
        keff, lo, hi, 32, R, gt, s_key, cap);
    compact_rounds(lkey, nl, tau, keff - gt, [&](int pos, int i) { emit(pos, (int32_t)list[i].y); }, R.tmp);
  } else {
    // the whole row (rescored exactly when the band overflowed; a list shorter than keff
    // means a score fell outside its bound, and the approximate row is used)
    if (nb <= kBandCap && tid == 0) flag_error(a.err, DSA_DEVERR_BOUND);
    const float *row = a.scores + (int64_t)r * a.ld;
    auto load = [&](int i) { return score_key(row[i]); };
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
    for (int i = tid; i < len; i += NT) {
      const uint32_t k = load(i);
      lo = min(lo, k);
      hi = max(hi, k);
    }
    block_minmax<NT>(lo, hi, R);
    int gt;
    const uint32_t tau = radix_select<NT>(
        [&](auto f) {
          for (int i = tid; i < len; i += NT) f(load(i));
        },
        keff, lo, hi, 32, R, gt, s_key, cap);
    compact_rounds(load, len, tau, keff - gt, emit, R.tmp);
  }
  for (int i = keff + tid; i < a.k; i += NT) out[i] = -1;
}

// Tile mode: the threshold of each long row from its block's sampled tiles (which the GEMM
// scored first): the m-th largest of the row's sampled keys, by the sample rank rule, lowered
// by 2 E_r.  One workgroup per row; thread t holds 16 scores of sampled tile t / 16.
__global__ __launch_bounds__(256) void topk_tile_est_kernel(const TopkArgs a, TopkWs w) {
  __shared__ RadixLds<256> R;
  const int r = blockIdx.x, tid = threadIdx.x;
  const int len = row_len_of(a, r);
  const int keff = min(a.k, len);
  if (len <= kShortRow || keff >= len) {  // the row's lists are not used
    if (tid == 0) w.est[r] = 0u;
    return;
  }
  // the block's longest row, as the GEMM's sample launch computes it
  const int r0 = r & ~31;
  uint32_t lm = 0u;
  if (tid < 32 && r0 + tid < a.n_rows) {
    const int64_t l = a.row_len[r0 + tid];
    lm = (uint32_t)(l < 0 ? 0 : (l > a.ld ? a.ld : l));
  }
  lm = wave_max_u32(lm);  // wave 0's lanes hold the 32 rows
  __shared__ uint32_t s_lm;
  if (tid == 0) s_lm = lm;
  __syncthreads();
  const int64_t lmax = s_lm;
  const int i = tid >> 4, part = tid & 15;
  const int tl = sample_tile(i, lmax);
  const float *row = a.scores + (int64_t)r * a.ld;
  uint32_t sk[16];
  const int t0 = tl * kTileTokens + 16 * part;
  const int valid = tl >= 0 && t0 < len ? min(16, len - t0) : 0;
  // loads clamped to the row (no branch per element); slots past `valid` are ignored
  const int tb = tl >= 0 ? t0 : 0;
#pragma unroll
  for (int q = 0; q < 16; ++q) sk[q] = score_key(row[min(tb + q, len - 1)]);
  int S;
  block_scan_incl<256>(valid, R.tmp, S);
  uint32_t est = 0u;
  const int m = sample_rank(keff, len, max(S, 1));
  if (S >= 64 && m < S) {
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      lo = min(lo, q < valid ? sk[q] : 0xFFFFFFFFu);
      hi = max(hi, q < valid ? sk[q] : 0u);
    }
    block_minmax<256>(lo, hi, R);
    int gt;
    est = radix_select<256>(
        [&](auto f) {
#pragma unroll
          for (int q = 0; q < 16; ++q) f(sk[q], q < valid);
        },
        m, lo, hi, kEstPasses, R, gt);
  }
  if (tid == 0) w.est[r] = band_est(a, r, est);
}

}  // namespace

hipError_t launch_topk_tile_est(const TopkArgs &a, hipStream_t s) {
  if (a.n_rows == 0) return hipSuccess;
  const int n_tiles = (int)((a.ld + kTileTokens - 1) / kTileTokens);
  if (a.band.e == nullptr || n_tiles > kMaxSlices || a.n_rows > 65535) return hipErrorInvalidValue;
  const TopkWs w = carve(a.ws, a.n_rows, n_tiles, kTileTokens, kTileCap);
  hipLaunchKernelGGL(topk_tile_est_kernel, dim3(a.n_rows), dim3(256), 0, s, a, w);
  return hipGetLastError();
}

size_t topk_tile_workspace_bytes(int32_t n_rows, int64_t ld) {
  const int64_t n_tiles = (ld + kTileTokens - 1) / kTileTokens;
  return (size_t)(align16(4 * (int64_t)n_rows) + align16(4 * (int64_t)n_rows * n_tiles) +
                  8 * (int64_t)n_rows * n_tiles * kTileCap);
}

TileLists tile_lists(void *ws, int32_t n_rows, int64_t ld, int32_t k) {
  const int n_tiles = (int)((ld + kTileTokens - 1) / kTileTokens);
  const TopkWs w = carve(ws, n_rows, n_tiles, kTileTokens, kTileCap);
  TileLists t;
  t.est = w.est;
  t.cnt = w.cnt;
  t.cand = w.cand;
  t.n_tiles = n_tiles;
  t.k = k;
  return t;
}

size_t topk_workspace_bytes(int32_t n_rows, int64_t ld) {
  const int64_t n_slices = (ld + kSlice - 1) / kSlice;
  return (size_t)(align16(4 * (int64_t)n_rows) + align16(4 * (int64_t)n_rows * n_slices) +
                  8 * (int64_t)n_rows * n_slices * kSliceCap);
}

hipError_t launch_topk(const TopkArgs &a, hipStream_t s) {
  if (a.n_rows == 0) return hipSuccess;
  if (a.tile_mode) {  // the GEMM wrote the lists and the thresholds: the band's first pass only
    const int n_tiles = (int)((a.ld + kTileTokens - 1) / kTileTokens);
    if (a.band.e == nullptr || n_tiles > kMaxSlices || a.n_rows > 65535) return hipErrorInvalidValue;
    const TopkWs w = carve(a.ws, a.n_rows, n_tiles, kTileTokens, kTileCap);
    hipLaunchKernelGGL(topk_finalize_kernel<true>, dim3(a.n_rows), dim3(kFinThreads), 0, s, a, w, n_tiles);
    return hipGetLastError();
  }
  const int n_slices = (int)((a.ld + kSlice - 1) / kSlice);
  if (n_slices > kMaxSlices || a.n_rows > 65535) return hipErrorInvalidValue;
  const TopkWs w = carve(a.ws, a.n_rows, n_slices, kSlice, kSliceCap);
  if (a.ld > kShortRow) {
    if (a.ld <= kOwnMaxLd && a.n_rows <= kOwnMaxRows) {
      hipLaunchKernelGGL(topk_collect_kernel<true>, dim3(n_slices, a.n_rows), dim3(256), 0, s, a, w, n_slices);
    } else {
      const size_t smp = sizeof(uint32_t) * ((size_t)1 << sample_log2(a.ld));
      hipLaunchKernelGGL(topk_sample_kernel, dim3(a.n_rows), dim3(256), smp, s, a, w);
      hipLaunchKernelGGL(topk_collect_kernel<false>, dim3(n_slices, a.n_rows), dim3(256), 0, s, a, w, n_slices);
    }
  }
  if (a.band.e != nullptr)
    hipLaunchKernelGGL(topk_finalize_kernel<true>, dim3(a.n_rows), dim3(kFinThreads), 0, s, a, w, n_slices);
  else
    hipLaunchKernelGGL(topk_finalize_kernel<false>, dim3(a.n_rows), dim3(kFinThreads), 0, s, a, w, n_slices);
  return hipGetLastError();
}

hipError_t launch_topk_band_select(const TopkArgs &a, hipStream_t s) {
  if (a.n_rows == 0) return hipSuccess;
  if (a.band.e == nullptr || a.n_rows > 65535) return hipErrorInvalidValue;
  // list capacity: k plus room for the band, in whole wave-widths (k + 512 <= kBandListCap)
  const int cap = min(kBandListCap, (a.k + 512 + 63) / 64 * 64);
  const size_t dyn = 2 * sizeof(uint32_t) * (size_t)(cap + 64);
  hipLaunchKernelGGL(topk_band_select_kernel, dim3(a.n_rows), dim3(kFinThreads), dyn, s, a, cap);
  return hipGetLastError();
}

}  // namespace dsa
