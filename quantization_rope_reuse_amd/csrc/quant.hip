// Put: quantize the K and V head vectors of blocks gathered from a paged
// buffer into compressed records, FP8 E4M3 or INT4, one fp16 scale per
// 128-element vector.
//
// Follows the HyperCache post ("HyperCache – Distributed KV-cache
// quantization and relative RoPE reuse"), Core Design, compression
// paragraph, and its Part B printout (FP8 E4M3 wire records at 1.97x and
// grouped INT4 disk records at 3.88x against fp16).  Per vector:
//   amax = max |x_j|; s = fp16_RNE(amax / qmax) (qmax 448 for E4M3, 7 for
//   INT4; IEEE fp32 division); code_j = round(x_j / s) to E4M3 (saturating
//   at +-448) or to an integer clamped to [-7, 7], where x_j / s is the
//   correctly rounded fp32 quotient.
//
// Work decomposition: one workgroup (4 waves) per (layer, block, K|V, chunk
// of 4 * PASSES * 8 vectors), PASSES * 8 consecutive vectors per wave, 8
// lanes per vector; the vector's amax is reduced over its 8 lanes with
// cross-lane max.  Passes per wave, measured on MI355X (one launch over all
// layers, permuted tables):
// * the FP8 put from fp16 or bf16 makes one pass (chunks of 32 vectors): 2-3.5%
//   faster than four passes at the Llama-3-70B and Qwen3-8B shapes;
// * the INT4 put makes four (chunks of 128) when the block's vector count is a
//   multiple of 128, else two: one pass is 10-20% slower, two 5% slower;
// * the fused put + CRC makes four (or two) as well: with one pass its CRC
//   tail, which holds the workgroup's LDS after the loads, follows every 8 KB
//   of source (12% slower); two passes measured within 3% either way
//   (Llama-3-70B shape 0.6% faster, Qwen3-8B shape 3% slower);
// * the FP8 put from fp32 sources (small workloads only) keeps four or two.
#include "crc_device.h"
#include "hkv_device.h"
#include "hkv_launch.h"

namespace hkv {
namespace {

struct QuantParams {
  const char* k_src;
  const char* v_src;
  int64_t s_layer, s_page, s_token, s_head;
  int32_t num_pages;
  const int32_t* table;
  int32_t table_blocks;  // n_blocks (records per layer)
  uint8_t* rec;
  int64_t rec_layer, rec_block;
  int32_t n_heads;
  float rcp_heads;       // 1 / n_heads in fp32, for divmod_small
  int32_t vecs;
  int32_t chunks;
  int32_t vecs_per_chunk;
  uint32_t* partials;    // fused CRC: raw CRC of every 128-byte unit of every record
  int32_t units;         // 128-byte units per record
};

// fp16 bits of the scale for a vector with max magnitude amax (fp32).
// Edge cases: amax == 0 -> 0; a positive amax whose scale underflows fp16 ->
// smallest subnormal (0x0001); a scale beyond the fp16 range -> 65504.
template <int QMAX>
__device__ __forceinline__ uint32_t scale_bits(float amax) {
  const float s32 = amax / static_cast<float>(QMAX);   // IEEE division
  uint32_t h = f32_to_f16_bits(s32);
  if (h == 0x7C00u) h = 0x7BFFu;
  if (h == 0u && amax > 0.0f) h = 0x0001u;
  return h;
}

// Source run of 8 elements (lane-owned half of a vector) as raw words.
template <int SDT> struct RawSrc;
template <> struct RawSrc<kF32> { u32x4 w0, w1; };
template <> struct RawSrc<kF16> { u32x4 w0; };
template <> struct RawSrc<kBF16> { u32x4 w0; };

template <int SDT>
__device__ __forceinline__ RawSrc<SDT> load_run(const char* p) {
  RawSrc<SDT> r;
  r.w0 = *reinterpret_cast<const u32x4*>(p);
  if constexpr (SDT == kF32) r.w1 = *reinterpret_cast<const u32x4*>(p + 16);
  return r;
}

template <int SDT>
__device__ __forceinline__ void run_to_f32(const RawSrc<SDT>& r, float (&x)[8]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t w = r.w0[j];
    if constexpr (SDT == kF32) {
      const uint32_t w1 = r.w1[j];
      x[j] = __builtin_bit_cast(float, w);
      x[4 + j] = __builtin_bit_cast(float, w1);
    } else if constexpr (SDT == kF16) {
      x[2 * j] = f16_bits_to_f32(w & 0xFFFFu);
      x[2 * j + 1] = f16_bits_to_f32(w >> 16);
    } else {
      x[2 * j] = bf16_bits_to_f32(w & 0xFFFFu);
      x[2 * j + 1] = bf16_bits_to_f32(w >> 16);
    }
  }
}

// Quantize one vector's lane-owned runs a (elements 8s..8s+7) and b
// (64+8s..64+8s+7); returns the fp16 scale bits (same in all 8 lanes).
// STAGE: the code bytes also go to `stage` (LDS) at the same offsets.
template <int FMT, bool STAGE>
__device__ __forceinline__ uint32_t quant_vector(float (&a)[8], float (&b)[8], uint8_t* c_ptr,
                                                 int sub, bool active, uint8_t* stage) {
  // |x| compared as integers: for finite values the magnitude bits order
  // exactly like the magnitudes.
  uint32_t mbits = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t ua = __builtin_bit_cast(uint32_t, a[j]) & 0x7FFFFFFFu;
    const uint32_t ub = __builtin_bit_cast(uint32_t, b[j]) & 0x7FFFFFFFu;
    mbits = max(mbits, max(ua, ub));
  }
  const float amax = __builtin_bit_cast(float, max_bits_over_vector_lanes(mbits));
  constexpr int QMAX = FMT == kFP8 ? 448 : 7;
  const uint32_t sbits = scale_bits<QMAX>(amax);
  if (!active) return sbits;
  // An all-zero vector (s = 0) keeps its signed zeros: divide by 1 instead.
  const float s = sbits == 0u ? 1.0f : f16_bits_to_f32(sbits);
  const float r = 1.0f / s;                              // IEEE division, once per vector
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = div_by_scale(a[j], s, r);
    b[j] = div_by_scale(b[j], s, r);
  }
  if constexpr (FMT == kFP8) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      a[j] = __builtin_amdgcn_fmed3f(a[j], -448.0f, 448.0f);
      b[j] = __builtin_amdgcn_fmed3f(b[j], -448.0f, 448.0f);
    }
    const u32x2 ca = f32x8_to_fp8(a);
    const u32x2 cb = f32x8_to_fp8(b);
    __builtin_nontemporal_store(ca, reinterpret_cast<u32x2*>(c_ptr + 8 * sub));
    __builtin_nontemporal_store(cb, reinterpret_cast<u32x2*>(c_ptr + 64 + 8 * sub));
    if constexpr (STAGE) {
      *reinterpret_cast<u32x2*>(stage + 8 * sub) = ca;
      *reinterpret_cast<u32x2*>(stage + 64 + 8 * sub) = cb;
    }
  } else {
    // q clamped to [-7, 7] (integers, so clamping before rounding is the
    // same as after), then 1.5 * 2^23 added: the fp32 sum has unit spacing
    // there, so the addition itself rounds q to the nearest integer, ties
    // to even, and the low four bits of the sum are that integer in two's
    // complement -- the nibble.
    uint32_t wa = 0, wb = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float ra = __builtin_amdgcn_fmed3f(a[j], -7.0f, 7.0f) + 12582912.0f;
      const float rb = __builtin_amdgcn_fmed3f(b[j], -7.0f, 7.0f) + 12582912.0f;
      wa |= (__builtin_bit_cast(uint32_t, ra) & 0xFu) << (4 * j);
      wb |= (__builtin_bit_cast(uint32_t, rb) & 0xFu) << (4 * j);
    }
    __builtin_nontemporal_store(wa, reinterpret_cast<uint32_t*>(c_ptr + 4 * sub));
    __builtin_nontemporal_store(wb, reinterpret_cast<uint32_t*>(c_ptr + 32 + 4 * sub));
    if constexpr (STAGE) {
      *reinterpret_cast<uint32_t*>(stage + 4 * sub) = wa;
      *reinterpret_cast<uint32_t*>(stage + 32 + 4 * sub) = wb;
    }
  }
  return sbits;
}

// Each wave owns PASSES * 8 consecutive vectors of its workgroup's chunk,
// moved in passes of 8 vectors.  Source loads are issued a batch of
// passes at a time before any store of the batch: one counter tracks a
// wave's loads and stores in issue order, so loads issued after a store
// cannot be waited for without also waiting for the store.  Lane L collects
// the scale of vector v0 + L and stores it once at the end.  Record stores
// are non-temporal.
//
// CRC (fused put + CRC-32, chunks of exactly 32 * PASSES vectors): the
// workgroup's codes form a contiguous run of the record (16 KB FP8, 8 KB INT4
// with four passes), staged in LDS as they are written; after a barrier one
// thread per 128-byte unit (128 FP8 units: the first two waves; 64 INT4
// units: the first wave; the other waves end there) feeds its unit into a
// zero CRC register (byte tables in LDS) and stores that raw value in
// `partials` at the unit's index in the record.  A workgroup in this tail
// holds its LDS and the chain waves' slots: measured variants that kept one
// more wave (for the scale units) or gave a lane a second chain ran 5-6%
// slower.  The byte tables are built
// while the source loads are in flight.  The scale units at the end of the
// record are left to the merge kernel (crc.hip), which reads them back: one
// more thread here for the chunk's scale unit would run a whole further
// wave's chain for one unit (measured 8% slower with chunks of 64).
template <int FMT, int SDT, bool CRC, int PASSES>
__global__ __launch_bounds__(kThreads) void quant_kernel(QuantParams p) {
  const int layer = blockIdx.y;
  const int chunk = blockIdx.x % p.chunks;
  const int bk = blockIdx.x / p.chunks;
  const int kv = bk & 1;
  const int blk = bk >> 1;
  const int page = p.table[blk];
  if (page < 0 || page >= p.num_pages) return;   // uniform over the workgroup

  constexpr int kCB = FMT == kFP8 ? kHeadDim : kHeadDim / 2;
  constexpr int kGroupVecs = kVecsPerWave * PASSES * (kThreads / kWave);
  __shared__ __align__(16) uint8_t stage[CRC ? kGroupVecs * kCB : 16];
  __shared__ uint32_t T[CRC ? 4 : 1][256];

  constexpr int CB = FMT == kFP8 ? kHeadDim : kHeadDim / 2;
  constexpr int ES = ElemSize<SDT>::value;
  constexpr int kBatch = SDT == kF32 ? (PASSES < 2 ? PASSES : 2) : PASSES;
  constexpr int kWaveVecs = kVecsPerWave * PASSES;
  const char* src = (kv ? p.v_src : p.k_src) + layer * p.s_layer + page * p.s_page;
  uint8_t* rec = p.rec + layer * p.rec_layer + blk * p.rec_block;
  uint8_t* codes = rec + static_cast<int64_t>(kv) * p.vecs * CB;
  uint16_t* scales = reinterpret_cast<uint16_t*>(rec + 2LL * p.vecs * CB + 2LL * kv * p.vecs);

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int sub = lane & (kLanesPerVec - 1);
  const int vsub = lane / kLanesPerVec;
  const int v_end = min((chunk + 1) * p.vecs_per_chunk, p.vecs);
  const int chunk_v0 = chunk * p.vecs_per_chunk;
  const int v0 = chunk_v0 + wave * kWaveVecs;
  if (!CRC && v0 >= v_end) return;              // whole wave idle (never with CRC)

  uint32_t my_scale = 0;
#pragma unroll
  for (int i0 = 0; i0 < PASSES; i0 += kBatch) {
    RawSrc<SDT> ra[kBatch], rb[kBatch];
    // Unconditional loads: lanes past the chunk's end load its last vector,
    // whose amax they compute for nothing and whose codes they do not store
    // (no zero fill, no branch around the conversion).
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int v = min(v0 + kVecsPerWave * (i0 + i) + vsub, v_end - 1);
      const DivMod th = divmod_small(v, p.n_heads, p.rcp_heads);
      const char* x_ptr = src + th.q * p.s_token + th.r * p.s_head + 8 * sub * ES;
      ra[i] = load_run<SDT>(x_ptr);
      rb[i] = load_run<SDT>(x_ptr + 64 * ES);
    }
    if constexpr (CRC) {
      if (i0 == 0) build_crc_tables(T);        // every thread; ends with a barrier
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int v = v0 + kVecsPerWave * (i0 + i) + vsub;
      const bool active = v < v_end;
      float a[8], b[8];
      run_to_f32<SDT>(ra[i], a);
      run_to_f32<SDT>(rb[i], b);
      const uint32_t sbits = quant_vector<FMT, CRC>(a, b, codes + static_cast<int64_t>(v) * CB,
                                                    sub, active, stage + (v - chunk_v0) * CB);
      // lane 8*(i0+i) + r keeps the scale of vector r of this pass
      const uint32_t got = __shfl(sbits, (lane & 7) * kLanesPerVec);
      if (lane / kLanesPerVec == i0 + i) my_scale = got;
    }
  }
  if (lane < kWaveVecs && v0 + lane < v_end) scales[v0 + lane] = static_cast<uint16_t>(my_scale);
  if constexpr (CRC) {
    __syncthreads();
    constexpr int kCodeUnits = kGroupVecs * CB / 128;
    const int u = threadIdx.x;
    if (u < kCodeUnits) {
      const u32x4* w = reinterpret_cast<const u32x4*>(stage + u * 128);
      uint32_t c = 0;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const u32x4 x = w[q];
        c = crc_feed_word(T, c, x[0]);
        c = crc_feed_word(T, c, x[1]);
        c = crc_feed_word(T, c, x[2]);
        c = crc_feed_word(T, c, x[3]);
      }
      const int64_t byte =
          static_cast<int64_t>(kv) * p.vecs * CB + static_cast<int64_t>(chunk_v0) * CB + u * 128;
      p.partials[(static_cast<int64_t>(layer) * (p.table_blocks) + blk) * p.units + byte / 128] = c;
    }
  }
}

template <int FMT, int SDT, bool CRC, int PASSES>
hipError_t launch_passes(QuantParams p, const Geometry& g, hipStream_t stream) {
  p.vecs_per_chunk = kVecsPerWave * PASSES * (kThreads / kWave);
  static_assert(kVecsPerWave * PASSES * (kThreads / kWave) >= kFetchMinGroupVecs,
                "the shape check bounds the chunk count with the smallest chunk");
  p.chunks = (g.vecs + p.vecs_per_chunk - 1) / p.vecs_per_chunk;
  dim3 grid(static_cast<unsigned>(g.n_blocks) * 2u * static_cast<unsigned>(p.chunks),
            static_cast<unsigned>(g.n_layers));
  hipLaunchKernelGGL((quant_kernel<FMT, SDT, CRC, PASSES>), grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

// One pass for the FP8 put from 16-bit sources; otherwise four passes when
// the block's vectors fill chunks of 128, else two (the fused path requires
// whole chunks: vecs % 64 == 0, checked by the caller).
template <int FMT, int SDT, bool CRC>
hipError_t launch_t(const QuantParams& p, const Geometry& g, hipStream_t stream) {
  if constexpr (FMT == kFP8 && SDT != kF32 && !CRC)
    return launch_passes<FMT, SDT, CRC, 1>(p, g, stream);
  else
    return g.vecs % 128 == 0 ? launch_passes<FMT, SDT, CRC, 4>(p, g, stream)
                             : launch_passes<FMT, SDT, CRC, 2>(p, g, stream);
}

template <int FMT, bool CRC>
hipError_t launch_dtype(int sdt, const QuantParams& p, const Geometry& g, hipStream_t s) {
  switch (sdt) {
    case kF32: return launch_t<FMT, kF32, CRC>(p, g, s);
    case kF16: return launch_t<FMT, kF16, CRC>(p, g, s);
    default: return launch_t<FMT, kBF16, CRC>(p, g, s);
  }
}

QuantParams make_params(const Geometry& g, const PageView& src, const int32_t* table,
                        const RecordView& dst) {
  QuantParams p;
  p.k_src = src.k;
  p.v_src = src.v;
  p.s_layer = src.layer;
  p.s_page = src.page;
  p.s_token = src.token;
  p.s_head = src.head;
  p.num_pages = src.num_pages;
  p.table = table;
  p.table_blocks = g.n_blocks;
  p.rec = dst.base;
  p.rec_layer = dst.layer;
  p.rec_block = dst.block;
  p.n_heads = g.n_heads;
  p.rcp_heads = 1.0f / static_cast<float>(g.n_heads);
  p.vecs = g.vecs;
  p.chunks = 0;                 // set per pass count at launch
  p.vecs_per_chunk = 0;
  p.partials = nullptr;
  p.units = 0;
  return p;
}

}  // namespace

hipError_t launch_quant(int fmt, int src_dtype, const Geometry& g, const PageView& src,
                        const int32_t* table, const RecordView& dst, hipStream_t stream) {
  const QuantParams p = make_params(g, src, table, dst);
  return fmt == kFP8 ? launch_dtype<kFP8, false>(src_dtype, p, g, stream)
                     : launch_dtype<kINT4, false>(src_dtype, p, g, stream);
}

hipError_t launch_quant_crc_units(int fmt, int src_dtype, const Geometry& g, const PageView& src,
                                  const int32_t* table, const RecordView& dst,
                                  int64_t record_bytes, uint32_t* partials, hipStream_t stream) {
  QuantParams p = make_params(g, src, table, dst);
  p.partials = partials;
  p.units = static_cast<int32_t>(record_bytes / 128);
  return fmt == kFP8 ? launch_dtype<kFP8, true>(src_dtype, p, g, stream)
                     : launch_dtype<kINT4, true>(src_dtype, p, g, stream);
}

}  // namespace hkv
