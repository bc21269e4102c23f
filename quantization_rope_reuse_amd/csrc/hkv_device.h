// Device-side helpers shared by the libhkv kernels (gfx950 only).
//
// Lane layout used by the put and fetch kernels: a 128-element head vector is
// owned by 8 consecutive lanes of a wave; lane s (0..7) owns elements
// [8s, 8s+8) and [64+8s, 64+8s+8).  With this split both RoPE pair
// conventions stay inside one lane (interleaved pairs (2i, 2i+1) sit in one
// 8-element run; split-halves pairs (i, i+64) sit in the two runs of the same
// lane), so rotation needs no cross-lane traffic, and each load or store
// instruction of a wave covers whole 64-byte or 128-byte segments.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hkv {

constexpr int kHeadDim = 128;
constexpr int kLanesPerVec = 8;
constexpr int kWave = 64;
constexpr int kThreads = 256;                          // 4 waves per workgroup
constexpr int kVecsPerWave = kWave / kLanesPerVec;     // 8
constexpr int kFetchMinGroupVecs = kVecsPerWave * 2;  // 16: smallest fetch chunk (one wave, two passes)

enum DType { kF32 = 0, kF16 = 1, kBF16 = 2 };
enum Format { kFP8 = 0, kINT4 = 1 };
enum Pairs { kInterleaved = 0, kHalfSplit = 1 };

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

template <int DT> struct ElemSize;
template <> struct ElemSize<kF32> { static constexpr int value = 4; };
template <> struct ElemSize<kF16> { static constexpr int value = 2; };
template <> struct ElemSize<kBF16> { static constexpr int value = 2; };

// ---------------------------------------------------------------------------
// Scalar conversions
// ---------------------------------------------------------------------------

// Quotient and remainder of v / d for 0 <= v <= 2^24 + 64 and 1 <= d <= 2^24,
// given rcp = 1/d rounded to fp32 (computed once on the host).  Rounding v,
// rcp and the product each move v * rcp by at most half an ulp, which keeps
// the truncated estimate within one of the quotient, and one correction each
// way makes it exact -- about 8 instructions instead of a 32-bit division.
struct DivMod {
  int q, r;
};
__device__ __forceinline__ DivMod divmod_small(int v, int d, float rcp) {
  int q = static_cast<int>(static_cast<float>(v) * rcp);
  int r = v - q * d;
  if (r < 0) {
    --q;
    r += d;
  } else if (r >= d) {
    ++q;
    r -= d;
  }
  return {q, r};
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
  _Float16 x = __builtin_bit_cast(_Float16, static_cast<uint16_t>(h));
  return static_cast<float>(x);                       // exact
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __builtin_bit_cast(float, b << 16);          // exact
}

// fp32 -> fp16 bits, round to nearest even (IEEE; overflow gives inf).
__device__ __forceinline__ uint32_t f32_to_f16_bits(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
}

// fp32 -> bf16 bits, round to nearest even.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

// x / s rounded to nearest even in fp32, given r = 1/s rounded to nearest
// even (one IEEE division per scale): q0 = x*r is within a few ulps of x/s,
// the remainder x - q0*s is exact in one fused multiply-add, and one
// correction step q0 + rem*r rounds to the correctly rounded quotient
// (Markstein's correction on a correctly rounded reciprocal).  A GPU test
// compares it with IEEE division for every fp32 significand of x against
// every fp16 significand of s at several exponent pairs (bitwise equal);
// power-of-two scaling carries that to every quotient whose remainder stays
// a normal number, which covers every quotient the put turns into a code.
// The sign is taken from x so that signed zeros agree.
__device__ __forceinline__ float div_by_scale(float x, float s, float r) {
  const float q0 = x * r;
  const float rem = __builtin_fmaf(-q0, s, x);
  return __builtin_copysignf(__builtin_fmaf(rem, r, q0), x);
}

// ---------------------------------------------------------------------------
// 8-element runs: load as fp32 / store from fp32
// ---------------------------------------------------------------------------

template <int DT>
__device__ __forceinline__ void load8(const char* p, float (&x)[8]) {
  if constexpr (DT == kF32) {
    // Element extraction goes through scalar temporaries: a vector element
    // is not an addressable object, so it is never the operand of a bit cast.
    u32x4 a = *reinterpret_cast<const u32x4*>(p);
    u32x4 b = *reinterpret_cast<const u32x4*>(p + 16);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t ua = a[j];
      const uint32_t ub = b[j];
      x[j] = __builtin_bit_cast(float, ua);
      x[4 + j] = __builtin_bit_cast(float, ub);
    }
  } else {
    u32x4 a = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t w = a[j];
      if constexpr (DT == kF16) {
        x[2 * j] = f16_bits_to_f32(w & 0xFFFFu);
        x[2 * j + 1] = f16_bits_to_f32(w >> 16);
      } else {
        x[2 * j] = bf16_bits_to_f32(w & 0xFFFFu);
        x[2 * j + 1] = bf16_bits_to_f32(w >> 16);
      }
    }
  }
}

template <bool NT>
__device__ __forceinline__ void store16(char* p, u32x4 v) {
  if constexpr (NT)
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
  else
    *reinterpret_cast<u32x4*>(p) = v;
}

// Store 8 fp32 values as the page dtype (round to nearest even); NT selects
// non-temporal stores.
template <int DT, bool NT = false>
__device__ __forceinline__ void store8(char* p, const float (&x)[8]) {
  if constexpr (DT == kF32) {
    u32x4 a, b;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float fa = x[j];
      const float fb = x[4 + j];
      a[j] = __builtin_bit_cast(uint32_t, fa);
      b[j] = __builtin_bit_cast(uint32_t, fb);
    }
    store16<NT>(p, a);
    store16<NT>(p + 16, b);
  } else {
    u32x4 a;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t lo, hi;
      if constexpr (DT == kF16) {
        lo = f32_to_f16_bits(x[2 * j]);
        hi = f32_to_f16_bits(x[2 * j + 1]);
      } else {
        lo = f32_to_bf16_bits(x[2 * j]);
        hi = f32_to_bf16_bits(x[2 * j + 1]);
      }
      a[j] = lo | (hi << 16);
    }
    store16<NT>(p, a);
  }
}

// ---------------------------------------------------------------------------
// FP8 E4M3FN (gfx950's fp8 conversions use the OCP encoding: max 448,
// no infinities).  Codes are little endian: element j of a run is byte j.
// ---------------------------------------------------------------------------

// 8 codes -> 8 fp32 values (exact).
__device__ __forceinline__ void fp8x8_to_f32(u32x2 c, float (&x)[8]) {
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(c[w]), false);
    f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(c[w]), true);
    x[4 * w + 0] = lo[0];
    x[4 * w + 1] = lo[1];
    x[4 * w + 2] = hi[0];
    x[4 * w + 3] = hi[1];
  }
}

// 8 fp32 values already clamped to [-448, 448] -> 8 codes, round to nearest
// even, sign of zero kept.
__device__ __forceinline__ u32x2 f32x8_to_fp8(const float (&q)[8]) {
  u32x2 c;
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    int r = __builtin_amdgcn_cvt_pk_fp8_f32(q[4 * w + 0], q[4 * w + 1], 0, false);
    r = __builtin_amdgcn_cvt_pk_fp8_f32(q[4 * w + 2], q[4 * w + 3], r, true);
    c[w] = static_cast<uint32_t>(r);
  }
  return c;
}

// ---------------------------------------------------------------------------
// INT4: nibble j of a 32-bit word is element j, two's complement.
// ---------------------------------------------------------------------------

__device__ __forceinline__ void int4x8_to_f32(uint32_t w, float (&x)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    int q = __builtin_amdgcn_sbfe(static_cast<int>(w), 4 * j, 4);
    x[j] = static_cast<float>(q);
  }
}

// ---------------------------------------------------------------------------
// Vector-wide max over the 8 lanes owning one vector, on magnitude bits
// (non-negative finite floats order like their bit patterns).
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint32_t max_bits_over_vector_lanes(uint32_t v) {
  v = max(v, static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), 1, kLanesPerVec)));
  v = max(v, static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), 2, kLanesPerVec)));
  v = max(v, static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), 4, kLanesPerVec)));
  return v;
}

}  // namespace hkv
