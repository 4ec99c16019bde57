// resolve.hip -- block table -> per-layer page byte offsets in the block-packed pool.
//
// Page "vLLM 为 Kimi K3.1 Pro 提供 Day-0 支持", section "面向三种状态的 KV 缓存":
// before each step the block tables and cache slots are turned into the page
// addresses the kernels read, so the kernels can walk the packed cache as it
// is.  One thread per (request, page); integer work only.
#include "dsa_device.hpp"
#include "dsa_kernels.hpp"

namespace dsa {

__global__ __launch_bounds__(256) void resolve_kernel(const ResolveArgs a) {
  const int32_t b = blockIdx.y;
  const int32_t p = blockIdx.x * 256 + threadIdx.x;
  if (p >= a.max_pages) return;
  // both loads in flight together: the table entry is in bounds (p < max_pages <= bt_ld)
  // whether or not the page is in use
  int32_t np = a.n_pages[b];
  const int64_t row = a.bt[(int64_t)b * a.bt_ld + p];
  uint32_t err = 0;
  if (np < 0 || np > a.max_pages) {
    err |= DSA_DEVERR_PAGE_COUNT;
    np = np < 0 ? 0 : a.max_pages;
  }
  int64_t lo = -1, ko = -1;
  if (p < np) {
    if (row >= 0 && row < a.pool_rows) {
      lo = row * a.row_stride + a.layer_off;
      ko = lo + a.lat_page_bytes;
    } else {
      err |= DSA_DEVERR_BLOCK_RANGE;
    }
  }
  a.lat_off[(int64_t)b * a.off_ld + p] = lo;
  a.key_off[(int64_t)b * a.off_ld + p] = ko;
  if (err) flag_error(a.err, err);
}

hipError_t launch_resolve(const ResolveArgs &a, hipStream_t s) {
  if (a.n_req == 0 || a.max_pages == 0) return hipSuccess;
  dim3 grid((a.max_pages + 255) / 256, a.n_req);
  hipLaunchKernelGGL(resolve_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace dsa
