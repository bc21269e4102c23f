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
// Work decomposition: one workgroup per (layer, block, K|V, chunk of
// vectors); each wave owns 8 consecutive vectors per pass, 8 lanes per
// vector.  FP8 with per-block deltas: one pass, 4 waves per workgroup
// (chunks of 32 vectors, about 33k workgroups per Llama-3-70B-shaped layer);
// INT4 and per-token deltas: two passes, one wave per workgroup (chunks of
// 16).  Every lane
// of a key workgroup needs 8 (cos, sin) pairs; the 64 lanes of a wave first
// compute one pair each (i = lane) in double precision and then gather the 8
// they need with cross-lane reads, so the angle setup costs one double sincos
// per lane per wave and no LDS.  theta_i is computed once per call on the
// host, in double.
//
// Blocks may be visited in a caller-given order (a permutation of the
// logical blocks).  Results do not depend on it.  Listing blocks by
// increasing destination page makes concurrently running workgroups write
// neighbouring pages.  On a randomly permuted table that now measures under
// 1% faster than logical order: the order entry is one more dependent load
// at the head of every workgroup.
//
// Memory: per vector the kernel reads the codes (128 B FP8 / 64 B INT4) and
// one fp16 scale, and writes 128 elements of the page dtype.  A wave issues
// the loads of all its passes (and one coalesced load of its scales) before
// the first store; stores are non-temporal.
#include "hkv_device.h"
#include "hkv_launch.h"

namespace hkv {
namespace {

struct FetchParams {
  const uint8_t* rec;
  int64_t rec_layer, rec_block;
  const int32_t* table;
  const int32_t* delta;
  const int32_t* order;      // optional visiting order of the blocks
  int32_t n_blocks;
  int32_t block_tokens;
  char* k_out;
  char* v_out;
  int64_t o_layer, o_page, o_token, o_head;
  int32_t num_pages;
  int32_t n_heads;
  float rcp_heads;           // 1 / n_heads in fp32, for divmod_small
  int32_t vecs;
  int32_t chunks;
  int32_t vecs_per_chunk;
  double theta[kHeadDim / 2];   // 1 / base^(2i/128), computed on the host in double
};

template <int FMT> struct RawCodes;
template <> struct RawCodes<kFP8> { u32x2 lo, hi; };
template <> struct RawCodes<kINT4> { uint32_t lo, hi; };

template <int FMT>
__device__ __forceinline__ RawCodes<FMT> load_codes(const uint8_t* codes, int v, int sub) {
  RawCodes<FMT> r;
  if constexpr (FMT == kFP8) {
    const uint8_t* c = codes + static_cast<int64_t>(v) * kHeadDim + 8 * sub;
    r.lo = *reinterpret_cast<const u32x2*>(c);
    r.hi = *reinterpret_cast<const u32x2*>(c + 64);
  } else {
    const uint8_t* c = codes + static_cast<int64_t>(v) * (kHeadDim / 2) + 4 * sub;
    r.lo = *reinterpret_cast<const uint32_t*>(c);
    r.hi = *reinterpret_cast<const uint32_t*>(c + 32);
  }
  return r;
}

template <int FMT>
__device__ __forceinline__ void dequant(const RawCodes<FMT>& r, float s, float (&a)[8],
                                        float (&b)[8]) {
  if constexpr (FMT == kFP8) {
    fp8x8_to_f32(r.lo, a);
    fp8x8_to_f32(r.hi, b);
  } else {
    int4x8_to_f32(r.lo, a);
    int4x8_to_f32(r.hi, b);
  }
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

// cos and sin of phi = dm * theta for per-token deltas: phi and its
// reduction modulo pi/2 in double (pi/2 split into two doubles, so the
// reduced argument is accurate to about 1e-16 for |phi| < 2^31), then the
// Taylor series of sin (to r^9) and cos (to r^10) in fp32 on |r| <= pi/4,
// whose truncation errors are below 2e-9 and 1.2e-10; with r rounded to
// fp32 and fp32 Horner steps the results stay within 7e-8 of the exact sine
// and cosine (about one fp32 ulp), and the quadrant sets the signs.
__device__ __forceinline__ void sincos_reduced(int dm, double theta, float* c, float* s) {
  const double phi = static_cast<double>(dm) * theta;
  const double k = rint(phi * 0.63661977236758134308);          // 2 / pi
  double r = fma(-k, 1.5707963267948966192, phi);                // pi/2, high part
  r = fma(-k, 6.1232339957367658e-17, r);                        // pi/2, low part
  const float x = static_cast<float>(r);
  const float x2 = x * x;
  float ps = __builtin_fmaf(x2, 1.0f / 362880.0f, -1.0f / 5040.0f);   // 1/9!, -1/7!
  ps = __builtin_fmaf(ps, x2, 1.0f / 120.0f);
  ps = __builtin_fmaf(ps, x2, -1.0f / 6.0f);
  const float sr = __builtin_fmaf(x * x2, ps, x);
  float pc = __builtin_fmaf(x2, -1.0f / 3628800.0f, 1.0f / 40320.0f);  // -1/10!, 1/8!
  pc = __builtin_fmaf(pc, x2, -1.0f / 720.0f);
  pc = __builtin_fmaf(pc, x2, 1.0f / 24.0f);
  pc = __builtin_fmaf(pc, x2, -0.5f);
  const float cr = __builtin_fmaf(x2, pc, 1.0f);
  const int q = static_cast<int>(static_cast<int64_t>(k) & 3);
  *c = q == 0 ? cr : (q == 1 ? -sr : (q == 2 ? -cr : sr));
  *s = q == 0 ? sr : (q == 1 ? cr : (q == 2 ? -sr : -cr));
}

// Element-pair index of the j-th pair a lane rotates (see the lane layout in
// hkv_device.h).
template <int PAIRS>
__device__ __forceinline__ int pair_of(int sub, int j) {
  if constexpr (PAIRS == kInterleaved)
    return j < 4 ? 4 * sub + j : 32 + 4 * sub + (j - 4);
  else
    return 8 * sub + j;
}

// The per-token delta of vector v's token; the token index is clamped so
// that lanes past the end of the chunk read a valid delta whose result they
// then discard.
__device__ __forceinline__ int token_delta(const FetchParams& p, int blk, int v) {
  const int t = min(divmod_small(v, p.n_heads, p.rcp_heads).q, p.block_tokens - 1);
  return p.delta[static_cast<int64_t>(blk) * p.block_tokens + t];
}

// (cos, sin) of the 8 pairs this lane rotates, for the delta dm of its
// vector's token.  Called by every lane of the wave (the shared-token path
// exchanges values across lanes).
template <int PAIRS>
__device__ __forceinline__ void token_angles(const FetchParams& p, int dm, double theta_lane,
                                             int sub, float (&cs)[8], float (&sn)[8]) {
  if (p.n_heads % kVecsPerWave == 0) {
    // the pass's 8 vectors share one token: lane i computes pair i
    float cf, sf;
    sincos_reduced(dm, theta_lane, &cf, &sf);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      cs[j] = __shfl(cf, pair_of<PAIRS>(sub, j));
      sn[j] = __shfl(sf, pair_of<PAIRS>(sub, j));
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) sincos_reduced(dm, p.theta[pair_of<PAIRS>(sub, j)], &cs[j], &sn[j]);
  }
}

// Each wave owns PASSES * 8 consecutive vectors of its workgroup's chunk and
// moves them in PASSES passes of 8.  All loads of the wave
// are issued before its first store: one counter tracks a wave's loads and
// stores in issue order, so a load issued after a store could not be waited
// for without also waiting for that store.  Stores are non-temporal: the
// pages are not read again by this kernel.
//
// PER_TOKEN: delta is [n_blocks][block_tokens] and each key vector turns by
// its own token's delta.  When the head count is a multiple of 8 the 8
// vectors of a pass belong to one token and lane i computes pair i's angle
// once per pass; otherwise each lane computes the 8 angles it needs.
template <int FMT, int ODT, int PAIRS, bool PER_TOKEN, int PASSES, int THREADS>
__global__ __launch_bounds__(THREADS) void fetch_kernel(FetchParams p) {
  const int layer = blockIdx.y;
  const int chunk = blockIdx.x % p.chunks;
  const int bk = blockIdx.x / p.chunks;
  const int kv = bk & 1;
  const int slot = bk >> 1;
  const int blk = p.order ? p.order[slot] : slot;
  if (blk < 0 || blk >= p.n_blocks) return;
  // The page entry is a scalar load (the scalar cache holds the table after
  // the first workgroups), and the compiled kernel tests it before it issues
  // the code loads.  A variant that kept every load ahead of one exit test
  // (clamped block index, the loaded values used on the exit path as well)
  // measured no faster.
  const int page = p.table[blk];

  constexpr int CB = FMT == kFP8 ? kHeadDim : kHeadDim / 2;
  constexpr int ES = ElemSize<ODT>::value;
  const uint8_t* rec = p.rec + layer * p.rec_layer + blk * p.rec_block;
  const uint8_t* codes = rec + static_cast<int64_t>(kv) * p.vecs * CB;
  const uint16_t* scales =
      reinterpret_cast<const uint16_t*>(rec + 2LL * p.vecs * CB + 2LL * kv * p.vecs);

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int sub = lane & (kLanesPerVec - 1);
  const int vsub = lane / kLanesPerVec;
  constexpr int kWaveVecs = kVecsPerWave * PASSES;
  const int v_end = min((chunk + 1) * p.vecs_per_chunk, p.vecs);
  const int v0 = chunk * p.vecs_per_chunk + wave * kWaveVecs;
  if (v0 >= v_end) return;                      // whole wave idle

  // Loads complete in issue order, so everything the angle setup needs is
  // loaded before the codes (unconditionally: a load under a divergent branch
  // is waited for inside it), and the angles are computed while the codes are
  // in flight: this lane's theta, and for per-token deltas its tokens' deltas.
  const double theta_lane = p.theta[lane];
  int tok_dm[PASSES];
  if constexpr (PER_TOKEN) {
#pragma unroll
    for (int i = 0; i < PASSES; ++i)
      tok_dm[i] = token_delta(p, blk, v0 + kVecsPerWave * i + vsub);
  }

  // Lane L holds the scale of vector v0 + (L mod kWaveVecs) (clamped to the
  // chunk: lanes past its end load a valid scale they never use).
  const uint32_t my_scale = scales[min(v0 + (lane % kWaveVecs), v_end - 1)];
  // Unconditional as well (lanes past the chunk's end load its last vector
  // and discard it): the loads before them can then be waited for alone.
  RawCodes<FMT> raw[PASSES];
#pragma unroll
  for (int i = 0; i < PASSES; ++i)
    raw[i] = load_codes<FMT>(codes, min(v0 + kVecsPerWave * i + vsub, v_end - 1), sub);

  if (page < 0 || page >= p.num_pages) return;   // skipped block: nothing stored
  char* out = (kv ? p.v_out : p.k_out) + layer * p.o_layer + page * p.o_page;

  // Per-block deltas: angle setup for keys with a nonzero delta (uniform per
  // workgroup), overlapping the loads above: lane i forms phi_i = dm * theta_i
  // and its cos / sin in double precision (full range reduction), rounded to
  // fp32.
  const int dm = (kv == 0 && !PER_TOKEN) ? p.delta[blk] : 0;
  const bool rotate = dm != 0;
  float cs[8], sn[8];
  if (rotate) {
    double sd, cd;
    sincos(static_cast<double>(dm) * theta_lane, &sd, &cd);
    const float cf = static_cast<float>(cd);
    const float sf = static_cast<float>(sd);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      cs[j] = __shfl(cf, pair_of<PAIRS>(sub, j));
      sn[j] = __shfl(sf, pair_of<PAIRS>(sub, j));
    }
  }

#pragma unroll
  for (int i = 0; i < PASSES; ++i) {
    const int v = v0 + kVecsPerWave * i + vsub;
    const float s = f16_bits_to_f32(__shfl(my_scale, kVecsPerWave * i + vsub));
    if constexpr (PER_TOKEN) {
      if (kv == 0) token_angles<PAIRS>(p, tok_dm[i], theta_lane, sub, cs, sn);   // all lanes
    }
    if (v < v_end) {
      float a[8], b[8];
      dequant<FMT>(raw[i], s, a, b);
      if (rotate || (PER_TOKEN && kv == 0)) {
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
      const DivMod th = divmod_small(v, p.n_heads, p.rcp_heads);
      const int t = th.q;
      const int h = th.r;
      char* dst = out + t * p.o_token + h * p.o_head + 8 * sub * ES;
      store8<ODT, true>(dst, a);
      store8<ODT, true>(dst + 64 * ES, b);
    }
  }
}

// Passes per wave and workgroup size, measured on MI355X: per-block-delta
// FP8 fetches are fastest with one pass (8 vectors per wave) in workgroups of
// 4 waves (32 vectors); INT4 records (half the bytes per vector) and
// per-token deltas (more angle work per vector) need the second pass's loads
// in flight to cover their latency, and run 2-3% faster in one-wave
// workgroups (16 vectors) than in four-wave ones.
template <int FMT, bool PT>
constexpr int fetch_passes() {
  return (FMT == kFP8 && !PT) ? 1 : 2;
}
template <int FMT, bool PT>
constexpr int fetch_threads() {
  return (FMT == kFP8 && !PT) ? 4 * kWave : kWave;
}
static_assert(kVecsPerWave * 2 >= kFetchMinGroupVecs,
              "the shape check bounds the chunk count with the smallest fetch chunk");

template <int FMT, int ODT, int PAIRS, bool PT, int PASSES, int THREADS>
hipError_t launch_shape(FetchParams p, const Geometry& g, hipStream_t stream) {
  // Workgroups of THREADS / 64 waves x PASSES x 8 vectors.
  p.vecs_per_chunk = kVecsPerWave * PASSES * (THREADS / kWave);
  p.chunks = (g.vecs + p.vecs_per_chunk - 1) / p.vecs_per_chunk;
  dim3 grid(static_cast<unsigned>(g.n_blocks) * 2u * static_cast<unsigned>(p.chunks),
            static_cast<unsigned>(g.n_layers));
  hipLaunchKernelGGL((fetch_kernel<FMT, ODT, PAIRS, PT, PASSES, THREADS>), grid, dim3(THREADS), 0,
                     stream, p);
  return hipGetLastError();
}

template <int FMT, int ODT, int PAIRS, bool PT>
hipError_t launch_t(const FetchParams& p, const Geometry& g, hipStream_t stream) {
  return launch_shape<FMT, ODT, PAIRS, PT, fetch_passes<FMT, PT>(), fetch_threads<FMT, PT>()>(
      p, g, stream);
}

template <int FMT, int ODT, bool PT>
hipError_t launch_pairs(int pairs, const FetchParams& p, const Geometry& g, hipStream_t s) {
  return pairs == kInterleaved ? launch_t<FMT, ODT, kInterleaved, PT>(p, g, s)
                               : launch_t<FMT, ODT, kHalfSplit, PT>(p, g, s);
}

template <int FMT, bool PT>
hipError_t launch_dtype(int odt, int pairs, const FetchParams& p, const Geometry& g,
                        hipStream_t s) {
  switch (odt) {
    case kF32: return launch_pairs<FMT, kF32, PT>(pairs, p, g, s);
    case kF16: return launch_pairs<FMT, kF16, PT>(pairs, p, g, s);
    default: return launch_pairs<FMT, kBF16, PT>(pairs, p, g, s);
  }
}

template <bool PT>
hipError_t launch_fmt(int fmt, int odt, int pairs, const FetchParams& p, const Geometry& g,
                      hipStream_t s) {
  return fmt == kFP8 ? launch_dtype<kFP8, PT>(odt, pairs, p, g, s)
                     : launch_dtype<kINT4, PT>(odt, pairs, p, g, s);
}

}  // namespace

hipError_t launch_fetch(int fmt, int dst_dtype, int pairs, const Geometry& g,
                        const RecordView& src, const int32_t* table, const int32_t* delta_m,
                        bool delta_per_token, const int32_t* visit_order, double rope_base,
                        const PageView& dst, hipStream_t stream) {
  FetchParams p;
  p.rec = src.base;
  p.rec_layer = src.layer;
  p.rec_block = src.block;
  p.table = table;
  p.delta = delta_m;
  p.order = visit_order;
  p.n_blocks = g.n_blocks;
  p.block_tokens = g.block_tokens;
  p.k_out = dst.k;
  p.v_out = dst.v;
  p.o_layer = dst.layer;
  p.o_page = dst.page;
  p.o_token = dst.token;
  p.o_head = dst.head;
  p.num_pages = dst.num_pages;
  p.n_heads = g.n_heads;
  p.rcp_heads = 1.0f / static_cast<float>(g.n_heads);
  p.vecs = g.vecs;
  for (int i = 0; i < kHeadDim / 2; ++i)
    p.theta[i] = 1.0 / pow(rope_base, static_cast<double>(2 * i) / kHeadDim);
  return delta_per_token ? launch_fmt<true>(fmt, dst_dtype, pairs, p, g, stream)
                         : launch_fmt<false>(fmt, dst_dtype, pairs, p, g, stream);
}

}  // namespace hkv
