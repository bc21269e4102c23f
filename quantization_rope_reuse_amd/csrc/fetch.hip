// Fetch: dequantize records, rotate keys by the block's position delta, and
// scatter into a paged KV buffer.
//
// Follows the HyperCache post ("HyperCache – Distributed KV-cache
// quantization and relative RoPE reuse"), Core Design, relative-RoPE
// paragraph: a post-RoPE key cached at m_old becomes the key at m_new by
// rotating each pair i through (m_new - m_old) * theta_i, because plane
// rotations compose (the SO(2) identity printed there); values are not
// rotated.  theta_i = 1 / base^(2i/d) and the rotation's sign convention
// follow the KV-handoff module ("Модуль 13: KV-хэндофф: передача кеша между
// моделями и узлами"), module13.py listing, rope_cache / apply_rope.
//
// Work decomposition: one workgroup (4 waves) per (layer, block, K|V, chunk of
// vectors).  Each wave moves 8 vectors per pass, 8 lanes per vector.  Every
// lane of a key workgroup needs 8 (cos, sin) pairs; the 64 lanes of a wave
// first compute one pair each (i = lane) in double precision and then gather
// the 8 they need with cross-lane reads, so the angle setup costs one double
// sincos per lane per workgroup and no LDS.
//
// Memory: per vector the kernel reads the codes (128 B FP8 / 64 B INT4) and
// one fp16 scale, and writes 128 elements of the page dtype.  Loads of the
// next pass are issued before the current pass is converted and stored.
#include "hkv_device.h"
#include "hkv_launch.h"

namespace hkv {
namespace {

struct FetchParams {
  const uint8_t* rec;
  int64_t rec_layer, rec_block;
  const int32_t* table;
  const int32_t* delta;
  char* k_out;
  char* v_out;
  int64_t o_layer, o_page, o_token, o_head;
  int32_t num_pages;
  int32_t n_heads;
  int32_t vecs;
  int32_t chunks;
  int32_t vecs_per_chunk;
  double rope_base;
};

template <int FMT> struct RawVec;
template <> struct RawVec<kFP8> { u32x2 lo, hi; uint32_t scale; };
template <> struct RawVec<kINT4> { uint32_t lo, hi; uint32_t scale; };

template <int FMT>
__device__ __forceinline__ RawVec<FMT> load_vec(const uint8_t* codes, const uint16_t* scales,
                                                int v, int sub) {
  RawVec<FMT> r;
  if constexpr (FMT == kFP8) {
    const uint8_t* c = codes + static_cast<int64_t>(v) * kHeadDim + 8 * sub;
    r.lo = *reinterpret_cast<const u32x2*>(c);
    r.hi = *reinterpret_cast<const u32x2*>(c + 64);
  } else {
    const uint8_t* c = codes + static_cast<int64_t>(v) * (kHeadDim / 2) + 4 * sub;
    r.lo = *reinterpret_cast<const uint32_t*>(c);
    r.hi = *reinterpret_cast<const uint32_t*>(c + 32);
  }
  r.scale = scales[v];
  return r;
}

template <int FMT>
__device__ __forceinline__ void dequant(const RawVec<FMT>& r, float (&a)[8], float (&b)[8]) {
  if constexpr (FMT == kFP8) {
    fp8x8_to_f32(r.lo, a);
    fp8x8_to_f32(r.hi, b);
  } else {
    int4x8_to_f32(r.lo, a);
    int4x8_to_f32(r.hi, b);
  }
  const float s = f16_bits_to_f32(r.scale);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] *= s;   // exact: at most 4 + 11 significant bits
    b[j] *= s;
  }
}

__device__ __forceinline__ void rot(float& x, float& y, float c, float s) {
  const float nx = x * c - y * s;
  const float ny = x * s + y * c;
  x = nx;
  y = ny;
}

template <int FMT, int ODT, int PAIRS>
__global__ __launch_bounds__(kThreads) void fetch_kernel(FetchParams p) {
  const int layer = blockIdx.y;
  const int chunk = blockIdx.x % p.chunks;
  const int bk = blockIdx.x / p.chunks;
  const int kv = bk & 1;
  const int blk = bk >> 1;
  const int page = p.table[blk];
  if (page < 0 || page >= p.num_pages) return;

  constexpr int CB = FMT == kFP8 ? kHeadDim : kHeadDim / 2;
  constexpr int ES = ElemSize<ODT>::value;
  const uint8_t* rec = p.rec + layer * p.rec_layer + blk * p.rec_block;
  const uint8_t* codes = rec + static_cast<int64_t>(kv) * p.vecs * CB;
  const uint16_t* scales =
      reinterpret_cast<const uint16_t*>(rec + 2LL * p.vecs * CB + 2LL * kv * p.vecs);
  char* out = (kv ? p.v_out : p.k_out) + layer * p.o_layer + page * p.o_page;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int sub = lane & (kLanesPerVec - 1);
  const int vsub = lane / kLanesPerVec;
  const int v_begin = chunk * p.vecs_per_chunk;
  const int v_end = min(v_begin + p.vecs_per_chunk, p.vecs);

  int v = v_begin + wave * kVecsPerWave + vsub;
  RawVec<FMT> cur;
  if (v < v_end) cur = load_vec<FMT>(codes, scales, v, sub);

  // Angle setup for keys with a nonzero delta (uniform per workgroup).
  const int dm = kv == 0 ? p.delta[blk] : 0;
  const bool rotate = dm != 0;
  float cs[8], sn[8];
  if (rotate) {
    const double theta = 1.0 / pow(p.rope_base, static_cast<double>(2 * lane) / kHeadDim);
    double sd, cd;
    sincos(static_cast<double>(dm) * theta, &sd, &cd);
    const float cf = static_cast<float>(cd);
    const float sf = static_cast<float>(sd);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      int idx;
      if constexpr (PAIRS == kInterleaved)
        idx = j < 4 ? 4 * sub + j : 32 + 4 * sub + (j - 4);
      else
        idx = 8 * sub + j;
      cs[j] = __shfl(cf, idx);
      sn[j] = __shfl(sf, idx);
    }
  }

  while (v < v_end) {
    const int vn = v + kVecsPerPass;
    RawVec<FMT> nxt;
    if (vn < v_end) nxt = load_vec<FMT>(codes, scales, vn, sub);

    float a[8], b[8];
    dequant<FMT>(cur, a, b);
    if (rotate) {
      if constexpr (PAIRS == kInterleaved) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          rot(a[2 * j], a[2 * j + 1], cs[j], sn[j]);
          rot(b[2 * j], b[2 * j + 1], cs[4 + j], sn[4 + j]);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) rot(a[j], b[j], cs[j], sn[j]);
      }
    }
    const int t = v / p.n_heads;
    const int h = v - t * p.n_heads;
    char* dst = out + t * p.o_token + h * p.o_head + 8 * sub * ES;
    store8<ODT>(dst, a);
    store8<ODT>(dst + 64 * ES, b);

    cur = nxt;
    v = vn;
  }
}

template <int FMT, int ODT, int PAIRS>
hipError_t launch_t(const FetchParams& p, const Geometry& g, hipStream_t stream) {
  dim3 grid(static_cast<unsigned>(g.n_blocks) * 2u * static_cast<unsigned>(g.chunks),
            static_cast<unsigned>(g.n_layers));
  hipLaunchKernelGGL((fetch_kernel<FMT, ODT, PAIRS>), grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

template <int FMT, int ODT>
hipError_t launch_pairs(int pairs, const FetchParams& p, const Geometry& g, hipStream_t s) {
  return pairs == kInterleaved ? launch_t<FMT, ODT, kInterleaved>(p, g, s)
                               : launch_t<FMT, ODT, kHalfSplit>(p, g, s);
}

template <int FMT>
hipError_t launch_dtype(int odt, int pairs, const FetchParams& p, const Geometry& g,
                        hipStream_t s) {
  switch (odt) {
    case kF32: return launch_pairs<FMT, kF32>(pairs, p, g, s);
    case kF16: return launch_pairs<FMT, kF16>(pairs, p, g, s);
    default: return launch_pairs<FMT, kBF16>(pairs, p, g, s);
  }
}

}  // namespace

hipError_t launch_fetch(int fmt, int dst_dtype, int pairs, const Geometry& g,
                        const RecordView& src, const int32_t* table, const int32_t* delta_m,
                        double rope_base, const PageView& dst, hipStream_t stream) {
  FetchParams p;
  p.rec = src.base;
  p.rec_layer = src.layer;
  p.rec_block = src.block;
  p.table = table;
  p.delta = delta_m;
  p.k_out = dst.k;
  p.v_out = dst.v;
  p.o_layer = dst.layer;
  p.o_page = dst.page;
  p.o_token = dst.token;
  p.o_head = dst.head;
  p.num_pages = dst.num_pages;
  p.n_heads = g.n_heads;
  p.vecs = g.vecs;
  p.chunks = g.chunks;
  p.vecs_per_chunk = g.vecs_per_chunk;
  p.rope_base = rope_base;
  return fmt == kFP8 ? launch_dtype<kFP8>(dst_dtype, pairs, p, g, stream)
                     : launch_dtype<kINT4>(dst_dtype, pairs, p, g, stream);
}

}  // namespace hkv
