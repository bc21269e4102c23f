// Visiting order for the fetch: the logical blocks listed by increasing
// destination page.  Blocks whose table entry is negative or not below the
// page count (skipped by the fetch) come last, in index order.  Any
// permutation gives the fetch the same result; this one makes neighbouring
// workgroups write neighbouring pages.
//
// Rank computation: thread b counts the blocks that sort before it, reading
// the table through LDS tiles of 256 entries.  O(n^2) comparisons in total,
// about 10 microseconds for a thousand blocks; meant for per-request tables of
// up to a few thousand blocks.
#include "hkv_device.h"
#include "hkv_launch.h"

namespace hkv {
namespace {

__global__ __launch_bounds__(kThreads) void page_order_kernel(const int32_t* table, int32_t n,
                                                             int32_t num_pages, int32_t* order) {
  __shared__ int32_t tile[kThreads];
  const int b = blockIdx.x * kThreads + threadIdx.x;
  const int32_t mine = b < n ? table[b] : -1;
  const bool live = mine >= 0 && mine < num_pages;
  int32_t before = 0;     // blocks that sort before b
  int32_t n_live = 0;     // live blocks in the whole table
  for (int base = 0; base < n; base += kThreads) {
    __syncthreads();
    const int j = base + threadIdx.x;
    tile[threadIdx.x] = j < n ? table[j] : -1;
    __syncthreads();
    const int cnt = min(kThreads, n - base);
    for (int k = 0; k < cnt; ++k) {
      const int32_t other = tile[k];
      const int idx = base + k;
      const bool other_live = other >= 0 && other < num_pages;
      n_live += other_live ? 1 : 0;
      if (live) {
        before += (other_live && (other < mine || (other == mine && idx < b))) ? 1 : 0;
      } else {
        before += (!other_live && idx < b) ? 1 : 0;
      }
    }
  }
  if (b < n) order[live ? before : n_live + before] = b;
}

}  // namespace

hipError_t launch_page_order(const int32_t* table, int32_t n_blocks, int32_t num_pages,
                             int32_t* order, hipStream_t stream) {
  const unsigned groups = static_cast<unsigned>((n_blocks + kThreads - 1) / kThreads);
  hipLaunchKernelGGL(page_order_kernel, dim3(groups), dim3(kThreads), 0, stream, table, n_blocks,
                     num_pages, order);
  return hipGetLastError();
}

}  // namespace hkv
