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
// digit-first radix select: three passes over the keys with digits of 11, 11
// and 10 bits, each building a 2048-bin LDS histogram of the keys that still
// match the digits chosen so far, after which one wave finds the bin holding
// the k-th key with a suffix scan.  A last pass writes every token whose key
// is above that threshold, and the lowest-indexed tokens equal to it, at the
// position given by the number of selected tokens before it (wave ballots
// plus a block scan per batch of 16 keys per thread), so the output is in
// increasing token order.  Keys are read in batches of 16 independent loads
// per thread, so each pass waits for memory once per batch.
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

// Adds one to hist[d] for every lane with `live` set.  Keys of nearby values
// share a digit, so the wave's two most common digits among the first lanes
// are added with one atomic each and only the remaining lanes one by one.
__device__ __forceinline__ void wave_histogram_add(int* hist, bool live, uint32_t d, int lane) {
  uint64_t todo = __ballot(live);
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    if (todo == 0) return;
    const int leader = __builtin_ctzll(todo);
    const uint32_t dl = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(d), leader));
    const uint64_t same = __ballot(live && d == dl);   // a subset of todo
    if (lane == leader) atomicAdd(&hist[dl], __popcll(same));
    todo &= ~same;
  }
  if ((todo >> lane) & 1u) atomicAdd(&hist[d], 1);
}

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(const float* drift, int32_t n,
                                                             int32_t k, int32_t* selected) {
  constexpr int kSlots = 16;                         // keys per thread per batch
  constexpr int kBatch = kSlots * kTopkThreads;      // token b0 + r * 1024 + tid in slot r
  constexpr int kEntries = kSlots * kTopkWaves;      // (slot, wave) counts per batch, in token order
  constexpr int kBins = 2048;
  __shared__ __align__(16) int hist[kBins];
  __shared__ int count_a[kEntries];
  __shared__ int count_e[kEntries];
  __shared__ int wave_sum[2][kTopkWaves];
  __shared__ uint32_t s_prefix;
  __shared__ int s_remaining;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;

  // Radix select, digits of 11, 11 and 10 bits.  Invariant: 1 <= remaining
  // <= number of keys matching `prefix` under `mask`; the keys above those
  // are all taken, and `remaining` more are to be taken among them.
  uint32_t prefix = 0, mask = 0;
  int remaining = k;
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const uint32_t dmask = pass == 2 ? 0x3FFu : 0x7FFu;
    hist[tid] = 0;
    hist[tid + kTopkThreads] = 0;
    __syncthreads();
    for (int b0 = 0; b0 < n; b0 += kBatch) {
      uint32_t key[kSlots];
#pragma unroll
      for (int r = 0; r < kSlots; ++r) {
        const int i = b0 + r * kTopkThreads + tid;
        key[r] = i < n ? order_key(drift[i]) : 0u;
      }
#pragma unroll
      for (int r = 0; r < kSlots; ++r) {
        const bool live = b0 + r * kTopkThreads + tid < n && (key[r] & mask) == prefix;
        wave_histogram_add(hist, live, (key[r] >> shift) & dmask, lane);
      }
    }
    __syncthreads();
    if (wave == 0) {
      // lane l holds bins 32l .. 32l+31, read as eight 4-bin groups; suffix
      // sums run from the top bin down
      const int4* h4 = reinterpret_cast<const int4*>(hist) + 8 * lane;
      int sum = 0;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int4 v = h4[q];
        sum += v.x + v.y + v.z + v.w;
      }
      int suf = sum;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const int up = __shfl_down(suf, off);
        if (lane + off < kWave) suf += up;
      }
      int above = suf - sum;                          // keys in the bins of higher lanes
      if (above < remaining && remaining <= suf) {    // exactly one lane
        int d = 32 * lane;
        for (int q = 7; q >= 0; --q) {
          const int4 v = h4[q];
          const int c[4] = {v.x, v.y, v.z, v.w};
          int j = 3;
          for (; j >= 0; --j) {
            if (above + c[j] >= remaining) break;
            above += c[j];
          }
          if (j >= 0) {
            d = 32 * lane + 4 * q + j;
            break;
          }
        }
        s_prefix = prefix | (static_cast<uint32_t>(d) << shift);
        s_remaining = remaining - above;
      }
    }
    __syncthreads();
    prefix = s_prefix;
    remaining = s_remaining;
    mask |= dmask << shift;
  }
  const uint32_t thr = prefix;          // key of the k-th largest value
  // remaining = how many keys equal to thr are taken: the lowest-indexed ones

  // Output, batch by batch: the selected tokens before token i are the keys
  // above thr before it plus min(keys equal to thr before it, remaining).
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (kWave - lane));
  int done_a = 0, done_e = 0;           // counts over earlier batches
  for (int b0 = 0; b0 < n; b0 += kBatch) {
    uint32_t key[kSlots];
#pragma unroll
    for (int r = 0; r < kSlots; ++r) {
      const int i = b0 + r * kTopkThreads + tid;
      key[r] = i < n ? order_key(drift[i]) : 0u;
    }
#pragma unroll
    for (int r = 0; r < kSlots; ++r) {
      const bool valid = b0 + r * kTopkThreads + tid < n;
      const uint64_t ma = __ballot(valid && key[r] > thr);
      const uint64_t me = __ballot(valid && key[r] == thr);
      if (lane == 0) {
        count_a[r * kTopkWaves + wave] = __popcll(ma);
        count_e[r * kTopkWaves + wave] = __popcll(me);
      }
    }
    __syncthreads();
    // exclusive scan over the kEntries entries, entry e held by thread e
    const int va = tid < kEntries ? count_a[tid] : 0;
    const int ve = tid < kEntries ? count_e[tid] : 0;
    int ia = va, ie = ve;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int ua = __shfl_up(ia, off);
      const int ue = __shfl_up(ie, off);
      if (lane >= off) {
        ia += ua;
        ie += ue;
      }
    }
    if (lane == kWave - 1) {
      wave_sum[0][wave] = ia;
      wave_sum[1][wave] = ie;
    }
    __syncthreads();
    int base_a = 0, base_e = 0, total_a = 0, total_e = 0;
#pragma unroll
    for (int w = 0; w < kTopkWaves; ++w) {
      const int sa = wave_sum[0][w];
      const int se = wave_sum[1][w];
      base_a += w < wave ? sa : 0;
      base_e += w < wave ? se : 0;
      total_a += sa;
      total_e += se;
    }
    if (tid < kEntries) {
      count_a[tid] = done_a + base_a + ia - va;
      count_e[tid] = done_e + base_e + ie - ve;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kSlots; ++r) {
      const int i = b0 + r * kTopkThreads + tid;
      const bool valid = i < n;
      const bool is_above = valid && key[r] > thr;
      const bool is_equal = valid && key[r] == thr;
      const uint64_t ma = __ballot(is_above);
      const uint64_t me = __ballot(is_equal);
      const int above_before = count_a[r * kTopkWaves + wave] + __popcll(ma & below);
      const int equal_before = count_e[r * kTopkWaves + wave] + __popcll(me & below);
      const int pos = above_before + min(equal_before, remaining);
      if ((is_above || (is_equal && equal_before < remaining)) && pos < k) selected[pos] = i;
    }
    done_a += total_a;
    done_e += total_e;
    __syncthreads();                    // count_* and wave_sum are rewritten next batch
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
