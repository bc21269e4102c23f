// Measurement aids, not steps of the method: plain streaming kernels with the
// byte mixes of the fetch and of the put, so that each can be reported
// against what the memory system gives a kernel that does nothing but move
// bytes in that ratio with the same access pattern.
//
// Fetch mix (one byte read for every two written): each thread reads 16
// bytes and writes them twice (the second copy xor-ed with a constant) as two
// 16-byte non-temporal stores 128 bytes apart: eight lanes fill one 256-byte
// output row, as eight lanes fill one bf16 vector in the fetch.
//
// Put mix (two bytes read for every one written): eight lanes turn one
// 256-byte source row into one 128-byte output row; lane s reads the 16
// bytes at 16s and at 128 + 16s and stores two 8-byte halves of their xor
// mix, non-temporal, at 8s and 64 + 8s -- the put's loads of one bf16 vector
// and its stores of that vector's FP8 codes.
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

__global__ __launch_bounds__(kThreads) void stream_squeeze_kernel(const uint8_t* __restrict__ src,
                                                                   uint8_t* __restrict__ dst,
                                                                   int64_t rows) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  const int64_t r = t / 8;
  const int s = static_cast<int>(t % 8);
  if (r >= rows) return;
  const u32x4 x = *reinterpret_cast<const u32x4*>(src + r * 256 + 16 * s);
  const u32x4 y = *reinterpret_cast<const u32x4*>(src + r * 256 + 128 + 16 * s);
  const u32x2 lo = {x[0] ^ y[1], x[2] ^ y[3]};
  const u32x2 hi = {x[1] ^ y[0], x[3] ^ y[2]};
  __builtin_nontemporal_store(lo, reinterpret_cast<u32x2*>(dst + r * 128 + 8 * s));
  __builtin_nontemporal_store(hi, reinterpret_cast<u32x2*>(dst + r * 128 + 64 + 8 * s));
}

}  // namespace

hipError_t launch_stream_squeeze(const void* src, void* dst, int64_t rows, hipStream_t stream) {
  const int64_t groups = (rows * 8 + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(stream_squeeze_kernel, dim3(static_cast<unsigned>(groups)), dim3(kThreads), 0,
                     stream, static_cast<const uint8_t*>(src), static_cast<uint8_t*>(dst), rows);
  return hipGetLastError();
}

hipError_t launch_stream_expand(const void* src, void* dst, int64_t units16, hipStream_t stream) {
  const int64_t groups = (units16 + kThreads - 1) / kThreads;
  const unsigned grid = static_cast<unsigned>(groups < 16384 ? groups : 16384);
  hipLaunchKernelGGL(stream_expand_kernel, dim3(grid), dim3(kThreads), 0, stream,
                     static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), units16);
  return hipGetLastError();
}

}  // namespace hkv
