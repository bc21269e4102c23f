// CRC-32 helpers shared by the kernels that compute CRCs: the zlib
// polynomial in the reflected representation (bit 31 holds x^0), GF(2)
// multiplication modulo it, x^(8n) mod P, and byte tables for slicing by four.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hkv {

constexpr uint32_t kCrcPoly = 0xEDB88320u;     // reflected x^32 + x^26 + ... + 1

// a * b mod P, reflected; bit-serial (32 steps).  Usable on the host, on the
// device and at compile time.
__host__ __device__ constexpr uint32_t crc_mulmod(uint32_t a, uint32_t b) {
  uint32_t p = 0;
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    p ^= b & (0u - ((a >> (31 - j)) & 1u));
    b = (b >> 1) ^ (kCrcPoly & (0u - (b & 1u)));
  }
  return p;
}

// x^(8n) mod P, reflected: the shift of a CRC register over n zero bytes.
__host__ __device__ constexpr uint32_t crc_x8n(uint64_t n) {
  uint32_t result = 0x80000000u;               // x^0
  uint32_t sq = 0x00800000u;                   // x^8
  while (n) {
    if (n & 1u) result = crc_mulmod(result, sq);
    sq = crc_mulmod(sq, sq);
    n >>= 1;
  }
  return result;
}

// Byte tables for slicing by four: T[0] is the one-byte table and T[s][i]
// feeds T[s-1][i] one more zero byte.  Built by the first 256 threads of the
// workgroup (blockDim.x >= 256); ends with a barrier.
__device__ __forceinline__ void build_crc_tables(uint32_t (*T)[256]) {
  const int tid = threadIdx.x;
  if (tid < 256) {
    uint32_t c = static_cast<uint32_t>(tid);
#pragma unroll
    for (int k = 0; k < 8; ++k) c = (c >> 1) ^ (kCrcPoly & (0u - (c & 1u)));
    T[0][tid] = c;
  }
  __syncthreads();
#pragma unroll
  for (int s = 1; s < 4; ++s) {
    if (tid < 256) {
      const uint32_t prev = T[s - 1][tid];
      T[s][tid] = (prev >> 8) ^ T[0][prev & 0xFFu];
    }
    __syncthreads();
  }
}

// Feeds one little-endian word into the register c.
__device__ __forceinline__ uint32_t crc_feed_word(const uint32_t (*T)[256], uint32_t c,
                                                  uint32_t w) {
  c ^= w;
  return T[3][c & 0xFFu] ^ T[2][(c >> 8) & 0xFFu] ^ T[1][(c >> 16) & 0xFFu] ^ T[0][c >> 24];
}

}  // namespace hkv
