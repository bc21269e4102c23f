// Visiting order for the fetch: the logical blocks listed by increasing
// destination page.  Blocks whose table entry is negative or not below the
// page count (skipped by the fetch) come last, in index order.  Any
// permutation gives the fetch the same result; this one makes neighbouring
// workgroups write neighbouring pages.
//
// Rank computation: one wave per block b reads the whole table with coalesced
// loads, 64 entries per step, and counts the blocks that sort before b with
// a wave ballot and a population count.  O(n^2) comparisons in total, spread
// over n waves: a few microseconds for a thousand blocks; meant for
// per-request tables of up to a few thousand blocks.
#include "hkv_device.h"
#include "hkv_launch.h"

namespace hkv {
namespace {

constexpr int kBlocksPerGroup = kThreads / kWave;

__global__ __launch_bounds__(kThreads) void page_order_kernel(const int32_t* table, int32_t n,
                                                             int32_t num_pages, int32_t* order) {
  const int lane = threadIdx.x & (kWave - 1);
  const int b = blockIdx.x * kBlocksPerGroup + threadIdx.x / kWave;   // uniform per wave
  if (b >= n) return;                                                 // whole wave
  const int32_t mine = table[b];
  const bool live = mine >= 0 && mine < num_pages;
  uint32_t before = 0;     // blocks that sort before b
  uint32_t n_live = 0;     // live blocks in the whole table
  for (int base = 0; base < n; base += kWave) {
    const int j = base + lane;
    const int32_t other = j < n ? table[j] : -1;
    const bool other_live = other >= 0 && other < num_pages;
    const bool earlier = live ? (other_live && (other < mine || (other == mine && j < b)))
                              : (j < n && !other_live && j < b);
    before += __popcll(__ballot(earlier));
    n_live += __popcll(__ballot(other_live));
  }
  if (lane == 0) order[live ? before : n_live + before] = b;
}

}  // namespace

hipError_t launch_page_order(const int32_t* table, int32_t n_blocks, int32_t num_pages,
                             int32_t* order, hipStream_t stream) {
  const unsigned groups = static_cast<unsigned>((n_blocks + kBlocksPerGroup - 1) / kBlocksPerGroup);
  hipLaunchKernelGGL(page_order_kernel, dim3(groups), dim3(kThreads), 0, stream, table, n_blocks,
                     num_pages, order);
  return hipGetLastError();
}

}  // namespace hkv
