// Selection of the tokens to recompute after a chunk reorder.
//
// The HyperCache post ("HyperCache – Distributed KV-cache quantization and
// relative RoPE reuse"), Core Design, recompute paragraph: after the rotation
// the first layer's KV is exact, and the tokens whose first-layer hidden state
// drifts the most (about 15% of them, following CacheBlend) are recomputed
// through the deeper layers.  Here drift_t = || h_fresh[t] - h_cached[t] ||_2
// over the model width, and the k tokens with the largest drift are selected
// (ties to the lower token index), listed in increasing token order.
//
// drift_kernel: one wave per token, 16-byte loads four deep, fp32 sum of
// squares per lane, then a butterfly sum across the wave.  It reads
// 2 * d_model * element bytes per token and writes 4: HBM-bound.
//
// topk_kernel: one workgroup of 1024 threads.  Each value is mapped to a
// 32-bit key whose unsigned order is the selection order (NaN highest, -0 as
// +0).  The key of the k-th largest value is found by a most-significant-
// digit-first radix select: four passes of 8 bits, each building a 256-bin
// LDS histogram of the keys that still match the digits chosen so far, after
// which one wave finds the bin holding the k-th key with a suffix scan.
// A last pass over tiles of 1024 tokens writes every token whose key is above
// that threshold, and the lowest-indexed tokens equal to it, at the position
// given by the count of selected tokens before it (wave ballots plus a
// 16-entry LDS scan per tile), so the output is in increasing token order.
#include "hkv_device.h"
#include "hkv_launch.h"

namespace hkv {
namespace {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / kWave;

template <int DT>
__device__ __forceinline__ float sq_diff_sum(u32x4 wa, u32x4 wb, float acc) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t ua = wa[q];
    const uint32_t ub = wb[q];
    if constexpr (DT == kF32) {
      const float d = __builtin_bit_cast(float, ub) - __builtin_bit_cast(float, ua);
      acc = __builtin_fmaf(d, d, acc);
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t ha = (ua >> (16 * h)) & 0xFFFFu;
        const uint32_t hb = (ub >> (16 * h)) & 0xFFFFu;
        const float fa = DT == kF16 ? f16_bits_to_f32(ha) : bf16_bits_to_f32(ha);
        const float fb = DT == kF16 ? f16_bits_to_f32(hb) : bf16_bits_to_f32(hb);
        const float d = fb - fa;
        acc = __builtin_fmaf(d, d, acc);
      }
    }
  }
  return acc;
}

template <int DT>
__device__ __forceinline__ float elem(const char* row, int j) {
  if constexpr (DT == kF32) return reinterpret_cast<const float*>(row)[j];
  const uint32_t h = reinterpret_cast<const uint16_t*>(row)[j];
  return DT == kF16 ? f16_bits_to_f32(h) : bf16_bits_to_f32(h);
}

template <int DT>
__global__ __launch_bounds__(kThreads) void drift_kernel(const char* cached, const char* fresh,
                                                         int32_t n_tokens, int32_t d_model,
                                                         int64_t row_bytes, float* drift) {
  constexpr int ES = ElemSize<DT>::value;
  constexpr int kElems = 16 / ES;                   // elements per 16-byte load
  constexpr int kStep = kWave * kElems;             // elements per wave-wide load
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * (kThreads / kWave) + threadIdx.x / kWave;
  if (t >= n_tokens) return;                        // whole wave
  const char* a = cached + t * row_bytes;
  const char* b = fresh + t * row_bytes;
  const int d_vec = d_model - d_model % kElems;     // elements covered by 16-byte loads
  float acc = 0.0f;
  int j = lane * kElems;
  for (; j + 3 * kStep < d_vec; j += 4 * kStep) {
    u32x4 wa[4], wb[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      wa[u] = *reinterpret_cast<const u32x4*>(a + static_cast<int64_t>(j + u * kStep) * ES);
      wb[u] = *reinterpret_cast<const u32x4*>(b + static_cast<int64_t>(j + u * kStep) * ES);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) acc = sq_diff_sum<DT>(wa[u], wb[u], acc);
  }
  for (; j < d_vec; j += kStep) {
    const u32x4 wa = *reinterpret_cast<const u32x4*>(a + static_cast<int64_t>(j) * ES);
    const u32x4 wb = *reinterpret_cast<const u32x4*>(b + static_cast<int64_t>(j) * ES);
    acc = sq_diff_sum<DT>(wa, wb, acc);
  }
  if (d_vec + lane < d_model) {                     // ragged tail, fewer than kElems
    const float d = elem<DT>(b, d_vec + lane) - elem<DT>(a, d_vec + lane);
    acc = __builtin_fmaf(d, d, acc);
  }
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (lane == 0) drift[t] = __builtin_sqrtf(acc);
}

// Unsigned key whose order is the selection order: NaN above +inf, -0 equal
// to +0, negative values below non-negative ones.
__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t b = __builtin_bit_cast(uint32_t, x);
  if (x != x) return 0xFFFFFFFFu;
  if ((b & 0x7FFFFFFFu) == 0) b = 0;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(const float* drift, int32_t n,
                                                             int32_t k, int32_t* selected) {
  __shared__ int hist[256];
  __shared__ int wave_count[2][2][kTopkWaves];      // [tile parity][above, equal][wave]
  __shared__ uint32_t s_prefix;
  __shared__ int s_remaining;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;

  // Radix select.  Invariant: 1 <= remaining <= number of keys matching
  // `prefix` under `mask`; remaining counts how many of them are still to be
  // taken, the keys above them all being taken already.
  uint32_t prefix = 0, mask = 0;
  int remaining = k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += kTopkThreads) {
      const uint32_t key = order_key(drift[i]);
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 0xFFu], 1);
    }
    __syncthreads();
    if (wave == 0) {
      // lane l holds bins 4l..4l+3; suffix sums run from the top bin down
      const int c0 = hist[4 * lane], c1 = hist[4 * lane + 1];
      const int c2 = hist[4 * lane + 2], c3 = hist[4 * lane + 3];
      const int s = c0 + c1 + c2 + c3;
      int suf = s;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const int up = __shfl_down(suf, off);
        if (lane + off < kWave) suf += up;
      }
      int above = suf - s;                          // keys in the bins of higher lanes
      if (above < remaining && remaining <= suf) {  // exactly one lane
        int d;
        if (above + c3 >= remaining) {
          d = 4 * lane + 3;
        } else if (above + c3 + c2 >= remaining) {
          above += c3;
          d = 4 * lane + 2;
        } else if (above + c3 + c2 + c1 >= remaining) {
          above += c3 + c2;
          d = 4 * lane + 1;
        } else {
          above += c3 + c2 + c1;
          d = 4 * lane;
        }
        s_prefix = prefix | (static_cast<uint32_t>(d) << shift);
        s_remaining = remaining - above;
      }
    }
    __syncthreads();
    prefix = s_prefix;
    remaining = s_remaining;
    mask |= 0xFFu << shift;
  }
  const uint32_t thr = prefix;          // key of the k-th largest value
  // remaining = how many keys equal to thr are taken: the lowest-indexed ones

  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (kWave - lane));
  int above_done = 0, equal_done = 0;   // counts over earlier tiles
  for (int t0 = 0, par = 0; t0 < n; t0 += kTopkThreads, par ^= 1) {
    const int i = t0 + tid;
    const uint32_t key = i < n ? order_key(drift[i]) : 0u;
    const bool is_above = i < n && key > thr;
    const bool is_equal = i < n && key == thr;
    const uint64_t m_above = __ballot(is_above);
    const uint64_t m_equal = __ballot(is_equal);
    if (lane == 0) {
      wave_count[par][0][wave] = __popcll(m_above);
      wave_count[par][1][wave] = __popcll(m_equal);
    }
    __syncthreads();
    int above_before = above_done + __popcll(m_above & below);
    int equal_before = equal_done + __popcll(m_equal & below);
#pragma unroll
    for (int w = 0; w < kTopkWaves; ++w) {
      const int ca = wave_count[par][0][w];
      const int ce = wave_count[par][1][w];
      above_before += w < wave ? ca : 0;
      equal_before += w < wave ? ce : 0;
      above_done += ca;
      equal_done += ce;
    }
    const int pos = above_before + min(equal_before, remaining);
    if ((is_above || (is_equal && equal_before < remaining)) && pos < k) selected[pos] = i;
    // the other buffer is written next; this one again only after the next
    // tile's barrier, which every thread reaches after its reads here
  }
}

}  // namespace

hipError_t launch_drift(int dtype, const void* cached, const void* fresh, int32_t n_tokens,
                        int32_t d_model, int64_t row_bytes, float* drift, hipStream_t stream) {
  constexpr int kTokensPerGroup = kThreads / kWave;
  const unsigned groups = static_cast<unsigned>((n_tokens + kTokensPerGroup - 1) / kTokensPerGroup);
  const char* a = static_cast<const char*>(cached);
  const char* b = static_cast<const char*>(fresh);
  switch (dtype) {
    case kF32:
      hipLaunchKernelGGL(drift_kernel<kF32>, dim3(groups), dim3(kThreads), 0, stream, a, b,
                         n_tokens, d_model, row_bytes, drift);
      break;
    case kF16:
      hipLaunchKernelGGL(drift_kernel<kF16>, dim3(groups), dim3(kThreads), 0, stream, a, b,
                         n_tokens, d_model, row_bytes, drift);
      break;
    default:
      hipLaunchKernelGGL(drift_kernel<kBF16>, dim3(groups), dim3(kThreads), 0, stream, a, b,
                         n_tokens, d_model, row_bytes, drift);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_topk(const float* drift, int32_t n, int32_t k, int32_t* selected,
                       hipStream_t stream) {
  hipLaunchKernelGGL(topk_kernel, dim3(1), dim3(kTopkThreads), 0, stream, drift, n, k, selected);
  return hipGetLastError();
}

}  // namespace hkv
