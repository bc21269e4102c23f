// Test kernel: the put's division routine (div_by_scale in hkv_device.h)
// against the correctly rounded IEEE fp32 quotient, for every fp32
// significand of x (2^23) against every fp16 significand of s (2^10) at one
// exponent pair per launch.  Built by the build step into
// tests/hip/libdiv_sweep.so; only the GPU tests load it.
//
// Thread i takes x = (1 + i / 2^23) * 2^x_exp and loops over the 1,024
// values s = (1 + j / 2^10) * 2^s_exp.  Each thread adds its count of
// differing quotients to out[0] and lowers out[1] (unsigned; the caller
// initialises it to all ones) to the smallest (i << 10 | j) that differed.
// The grid is exactly 2^23 threads; the only memory accesses are the two
// atomics on `out`.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hkv_device.h"

namespace {

constexpr int kSweepThreads = 256;
constexpr unsigned kXSignificands = 1u << 23;

__global__ __launch_bounds__(kSweepThreads) void div_sweep_kernel(int x_exp, int s_exp,
                                                                  unsigned long long* out) {
  const unsigned i = blockIdx.x * kSweepThreads + threadIdx.x;   // < 2^23 by the grid
  const float x = ldexpf(__builtin_bit_cast(float, 0x3F800000u | i), x_exp);
  unsigned long long bad = 0, first = ~0ull;
  for (unsigned j = 0; j < 1024; ++j) {
    const float s = ldexpf(__builtin_bit_cast(float, 0x3F800000u | (j << 13)), s_exp);
    const float r = __fdiv_rn(1.0f, s);
    const float q = hkv::div_by_scale(x, s, r);
    const float want = __fdiv_rn(x, s);
    if (__builtin_bit_cast(uint32_t, q) != __builtin_bit_cast(uint32_t, want)) {
      ++bad;
      const unsigned long long key = (static_cast<unsigned long long>(i) << 10) | j;
      first = key < first ? key : first;
    }
  }
  if (bad) {
    atomicAdd(&out[0], bad);
    atomicMin(&out[1], first);
  }
}

}  // namespace

// out: two unsigned 64-bit counters in device memory (out[1] preset to all
// ones).  Returns 0 or the HIP error code of the launch.
extern "C" int div_sweep(int x_exp, int s_exp, void* out, hipStream_t stream) {
  if (!out) return -1;
  hipLaunchKernelGGL(div_sweep_kernel, dim3(kXSignificands / kSweepThreads), dim3(kSweepThreads),
                     0, stream, x_exp, s_exp, static_cast<unsigned long long*>(out));
  return static_cast<int>(hipGetLastError());
}
