// A measurement aid, not a step of the method: a plain streaming kernel with
// the fetch's byte mix (one byte read for every two written), so that the
// fetch can be reported against what the memory system gives a kernel that
// does nothing but move bytes in that ratio.  Each thread reads 16 bytes and
// writes them twice (the second copy xor-ed with a constant) as two 16-byte
// non-temporal stores 128 bytes apart: eight lanes fill one 256-byte output
// row, as eight lanes fill one bf16 vector in the fetch.
#include "hkv_device.h"
#include "hkv_launch.h"

namespace hkv {
namespace {

__global__ __launch_bounds__(kThreads) void stream_expand_kernel(const u32x4* __restrict__ src,
                                                                  u32x4* __restrict__ dst,
                                                                  int64_t n) {
  const int64_t step = static_cast<int64_t>(gridDim.x) * kThreads;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i < n; i += step) {
    const u32x4 v = src[i];
    const u32x4 w = v ^ 0x5A5A5A5Au;
    const int64_t o = (i / 8) * 16 + (i % 8);
    __builtin_nontemporal_store(v, dst + o);
    __builtin_nontemporal_store(w, dst + o + 8);
  }
}

}  // namespace

hipError_t launch_stream_expand(const void* src, void* dst, int64_t units16, hipStream_t stream) {
  const int64_t groups = (units16 + kThreads - 1) / kThreads;
  const unsigned grid = static_cast<unsigned>(groups < 16384 ? groups : 16384);
  hipLaunchKernelGGL(stream_expand_kernel, dim3(grid), dim3(kThreads), 0, stream,
                     static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), units16);
  return hipGetLastError();
}

}  // namespace hkv
