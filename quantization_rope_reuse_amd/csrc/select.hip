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

constexpr int kSlots = 16;                           // keys per thread per batch
constexpr int kBatch = kSlots * kTopkThreads;        // token b0 + r * 1024 + tid in slot r
constexpr int kEntries = kSlots * kTopkWaves;        // (slot, wave) counts per batch
constexpr int kBins = 2048;

// Digit of each radix pass: 11, 11 and 10 bits from the top.
__device__ __forceinline__ int pass_shift(int pass) { return pass == 0 ? 21 : (pass == 1 ? 10 : 0); }
__device__ __forceinline__ uint32_t pass_dmask(int pass) { return pass == 2 ? 0x3FFu : 0x7FFu; }
__device__ __forceinline__ uint32_t mask_before(int pass) {
  return pass == 0 ? 0u : (pass == 1 ? 0xFFE00000u : 0xFFFFFC00u);
}

// Wave 0 only: the bin of hist (2048 bins, LDS) that holds the remaining-th
// largest key, as the new prefix and the count still to take inside it.
// Lane l holds bins 32l .. 32l+31, read as eight 4-bin groups; suffix sums
// run from the top bin down.  Requires 1 <= remaining <= total count.
__device__ __forceinline__ void digit_search(const int* hist, uint32_t prefix, int remaining,
                                             int shift, int lane, uint32_t* out_prefix,
                                             int* out_remaining) {
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
    *out_prefix = prefix | (static_cast<uint32_t>(d) << shift);
    *out_remaining = remaining - above;
  }
}

// Adds the pass's digit of every key in [lo, hi) that matches prefix under
// mask to hist (LDS).  Keys are read in batches of kSlots per thread.
__device__ __forceinline__ void histogram_range(const float* drift, int lo, int hi,
                                                uint32_t mask, uint32_t prefix, int shift,
                                                uint32_t dmask, int* hist, int tid, int lane) {
  for (int b0 = lo; b0 < hi; b0 += kBatch) {
    uint32_t key[kSlots];
#pragma unroll
    for (int r = 0; r < kSlots; ++r) {
      const int i = b0 + r * kTopkThreads + tid;
      key[r] = i < hi ? order_key(drift[i]) : 0u;
    }
#pragma unroll
    for (int r = 0; r < kSlots; ++r) {
      const bool live = b0 + r * kTopkThreads + tid < hi && (key[r] & mask) == prefix;
      wave_histogram_add(hist, live, (key[r] >> shift) & dmask, lane);
    }
  }
}

// Output for tokens [lo, hi): the selected tokens before token i are the
// keys above thr before it plus min(keys equal to thr before it, remaining);
// done_a / done_e count those before lo.  count_a / count_e: kEntries ints
// of LDS each; wave_sum: 2 x kTopkWaves.
__device__ __forceinline__ void write_range(const float* drift, int lo, int hi, uint32_t thr,
                                            int remaining, int k, int done_a, int done_e,
                                            int32_t* selected, int* count_a, int* count_e,
                                            int (*wave_sum)[kTopkWaves], int tid, int lane,
                                            int wave) {
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (kWave - lane));
  for (int b0 = lo; b0 < hi; b0 += kBatch) {
    uint32_t key[kSlots];
#pragma unroll
    for (int r = 0; r < kSlots; ++r) {
      const int i = b0 + r * kTopkThreads + tid;
      key[r] = i < hi ? order_key(drift[i]) : 0u;
    }
#pragma unroll
    for (int r = 0; r < kSlots; ++r) {
      const bool valid = b0 + r * kTopkThreads + tid < hi;
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
      const bool valid = i < hi;
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

// One workgroup does the whole selection.
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(const float* drift, int32_t n,
                                                             int32_t k, int32_t* selected) {
  __shared__ __align__(16) int hist[kBins];
  __shared__ int count_a[kEntries];
  __shared__ int count_e[kEntries];
  __shared__ int wave_sum[2][kTopkWaves];
  __shared__ uint32_t s_prefix;
  __shared__ int s_remaining;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;

  // Invariant: 1 <= remaining <= number of keys matching prefix under the
  // digits chosen so far; the keys above those are all taken.
  uint32_t prefix = 0;
  int remaining = k;
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    hist[tid] = 0;
    hist[tid + kTopkThreads] = 0;
    __syncthreads();
    histogram_range(drift, 0, n, mask_before(pass), prefix, pass_shift(pass), pass_dmask(pass),
                    hist, tid, lane);
    __syncthreads();
    if (wave == 0)
      digit_search(hist, prefix, remaining, pass_shift(pass), lane, &s_prefix, &s_remaining);
    __syncthreads();
    prefix = s_prefix;
    remaining = s_remaining;
  }
  write_range(drift, 0, n, prefix, remaining, k, 0, 0, selected, count_a, count_e, wave_sum,
              tid, lane, wave);
}

// ---- the same selection over many workgroups, with a caller's workspace ----
// Workgroup g owns tokens [g * slice, (g + 1) * slice).  Workspace (int32):
//   hist[3][groups][2048]   per-workgroup histograms of each pass
//   counts[groups][2]       per-workgroup counts above / equal to the threshold
//   state[4][2]             (prefix, remaining) before each pass; state[3] is
//                           (threshold key, equal keys to take)
// Kernel `pass` (0, 1, 2) sums the previous pass's histograms, chooses its
// digit (every workgroup the same; workgroup 0 records it), and histograms its
// own slice; the count kernel does the same for the last digit and counts;
// the write kernel places each workgroup's tokens after those of the
// workgroups before it.
struct SelectWs {
  int* hist;
  int* counts;
  int* state;
  int groups;
  int slice;
};

// Sums the groups' histograms of pass p into hist (LDS, 2048 bins).
__device__ __forceinline__ void reduce_histograms(const SelectWs& w, int p, int* hist, int tid) {
  const int* h = w.hist + static_cast<int64_t>(p) * w.groups * kBins;
  int a = 0, b = 0;
  for (int g0 = 0; g0 < w.groups; g0 += 8) {     // 16 independent loads in flight
    int va[8], vb[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const bool in = g0 + j < w.groups;
      va[j] = in ? h[(g0 + j) * kBins + tid] : 0;
      vb[j] = in ? h[(g0 + j) * kBins + tid + kTopkThreads] : 0;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      a += va[j];
      b += vb[j];
    }
  }
  hist[tid] = a;
  hist[tid + kTopkThreads] = b;
}

// (prefix, remaining) before pass p, from the recorded state and pass p-1's
// histograms; every workgroup computes it, workgroup 0 records it.
__device__ __forceinline__ void state_before(const SelectWs& w, int p, int k, int* hist,
                                             uint32_t* s_prefix, int* s_remaining, int tid,
                                             int lane, int wave, uint32_t* prefix,
                                             int* remaining) {
  if (p == 0) {
    *prefix = 0;
    *remaining = k;
    return;
  }
  reduce_histograms(w, p - 1, hist, tid);
  __syncthreads();
  if (wave == 0)
    digit_search(hist, static_cast<uint32_t>(w.state[2 * (p - 1)]), w.state[2 * (p - 1) + 1],
                 pass_shift(p - 1), lane, s_prefix, s_remaining);
  __syncthreads();
  *prefix = *s_prefix;
  *remaining = *s_remaining;
  if (blockIdx.x == 0 && tid == 0) {
    w.state[2 * p] = static_cast<int>(*prefix);
    w.state[2 * p + 1] = *remaining;
  }
  __syncthreads();                      // hist is rewritten next
}

__global__ __launch_bounds__(kTopkThreads) void select_pass_kernel(const float* drift, int32_t n,
                                                                    int32_t k, SelectWs w,
                                                                    int pass) {
  __shared__ __align__(16) int hist[kBins];
  __shared__ uint32_t s_prefix;
  __shared__ int s_remaining;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  if (pass == 0 && blockIdx.x == 0 && tid == 0) {
    w.state[0] = 0;
    w.state[1] = k;
  }
  uint32_t prefix;
  int remaining;
  state_before(w, pass, k, hist, &s_prefix, &s_remaining, tid, lane, wave, &prefix, &remaining);
  hist[tid] = 0;
  hist[tid + kTopkThreads] = 0;
  __syncthreads();
  const int lo = blockIdx.x * w.slice;
  const int hi = min(n - lo, w.slice) + lo;
  histogram_range(drift, lo, hi, mask_before(pass), prefix, pass_shift(pass), pass_dmask(pass),
                  hist, tid, lane);
  __syncthreads();
  int* row = w.hist + (static_cast<int64_t>(pass) * w.groups + blockIdx.x) * kBins;
  row[tid] = hist[tid];
  row[tid + kTopkThreads] = hist[tid + kTopkThreads];
}

__global__ __launch_bounds__(kTopkThreads) void select_count_kernel(const float* drift, int32_t n,
                                                                     int32_t k, SelectWs w) {
  __shared__ __align__(16) int hist[kBins];
  __shared__ uint32_t s_prefix;
  __shared__ int s_remaining;
  __shared__ int s_count[2][kTopkWaves];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  uint32_t thr;
  int remaining;
  state_before(w, 3, k, hist, &s_prefix, &s_remaining, tid, lane, wave, &thr, &remaining);
  const int lo = blockIdx.x * w.slice;
  const int hi = min(n - lo, w.slice) + lo;
  int na = 0, ne = 0;
  for (int i = lo + tid; i < hi; i += kTopkThreads) {
    const uint32_t key = order_key(drift[i]);
    na += key > thr ? 1 : 0;
    ne += key == thr ? 1 : 0;
  }
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) {
    na += __shfl_xor(na, off);
    ne += __shfl_xor(ne, off);
  }
  if (lane == 0) {
    s_count[0][wave] = na;
    s_count[1][wave] = ne;
  }
  __syncthreads();
  if (tid == 0) {
    int a = 0, e = 0;
    for (int q = 0; q < kTopkWaves; ++q) {
      a += s_count[0][q];
      e += s_count[1][q];
    }
    w.counts[2 * blockIdx.x] = a;
    w.counts[2 * blockIdx.x + 1] = e;
  }
}

__global__ __launch_bounds__(kTopkThreads) void select_write_kernel(const float* drift, int32_t n,
                                                                     int32_t k, int32_t* selected,
                                                                     SelectWs w) {
  __shared__ int count_a[kEntries];
  __shared__ int count_e[kEntries];
  __shared__ int wave_sum[2][kTopkWaves];
  __shared__ int s_done[2];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const uint32_t thr = static_cast<uint32_t>(w.state[6]);
  const int remaining = w.state[7];
  if (wave == 0) {                      // counts of the (at most 64) groups before this one
    const bool before = lane < static_cast<int>(blockIdx.x);
    int a = before ? w.counts[2 * lane] : 0;
    int e = before ? w.counts[2 * lane + 1] : 0;
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) {
      a += __shfl_xor(a, off);
      e += __shfl_xor(e, off);
    }
    if (lane == 0) {
      s_done[0] = a;
      s_done[1] = e;
    }
  }
  __syncthreads();
  const int done_a = s_done[0], done_e = s_done[1];
  const int lo = blockIdx.x * w.slice;
  const int hi = min(n - lo, w.slice) + lo;
  write_range(drift, lo, hi, thr, remaining, k, done_a, done_e, selected, count_a, count_e,
              wave_sum, tid, lane, wave);
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

void select_layout(int32_t n, int32_t* groups, int32_t* slice) {
  // 4,096 tokens per workgroup up to 16 workgroups, then at most 64
  // workgroups with slices in whole 1,024-token rows.
  const int64_t per = n <= 16 * 4096 ? 4096
                                     : ((static_cast<int64_t>(n) + 64 * 1024 - 1) / (64 * 1024)) * 1024;
  *slice = static_cast<int32_t>(per);
  *groups = static_cast<int32_t>((n + per - 1) / per);
}

int64_t select_workspace_bytes(int32_t n) {
  int32_t groups, slice;
  select_layout(n, &groups, &slice);
  return 4 * (static_cast<int64_t>(groups) * (3 * kBins + 2) + 8);
}

hipError_t launch_topk(const float* drift, int32_t n, int32_t k, int32_t* selected,
                       void* workspace, hipStream_t stream) {
  if (!workspace) {
    hipLaunchKernelGGL(topk_kernel, dim3(1), dim3(kTopkThreads), 0, stream, drift, n, k,
                       selected);
    return hipGetLastError();
  }
  SelectWs w;
  select_layout(n, &w.groups, &w.slice);
  w.hist = static_cast<int*>(workspace);
  w.counts = w.hist + static_cast<int64_t>(3) * w.groups * kBins;
  w.state = w.counts + 2 * w.groups;
  const dim3 grid(static_cast<unsigned>(w.groups)), block(kTopkThreads);
  for (int pass = 0; pass < 3; ++pass)
    hipLaunchKernelGGL(select_pass_kernel, grid, block, 0, stream, drift, n, k, w, pass);
  hipLaunchKernelGGL(select_count_kernel, grid, block, 0, stream, drift, n, k, w);
  hipLaunchKernelGGL(select_write_kernel, grid, block, 0, stream, drift, n, k, selected, w);
  return hipGetLastError();
}

}  // namespace hkv
