// Self-describing frames: a 64-byte header in front of each record.
//
// The HyperCache post's FP8 wire frame and INT4 disk file put a header of 68
// and 69 bytes around the payload (Part B byte counts) without giving its
// layout.  The header here is our own, little endian:
//    0 u32 magic "HKVF"   4 u16 version 1   6 u16 header bytes (64)
//    8 u8 format (0 FP8, 1 INT4)   9 u8 zero   10 u16 head_dim
//   12 u16 block_tokens   14 u16 n_kv_heads
//   16 u32 layer   20 u32 block   24 i32 m_old (cached position of the
//   block's first token)   28 u32 payload bytes   32 u32 payload CRC-32
//   36..59 zero   60 u32 CRC-32 of bytes 0..59
// With m_old in the frame, a reader computes the relative shift
// dm = m_new - m_old of the post's relative-RoPE paragraph from the frame
// alone.
//
// All three kernels handle one frame per thread: the work is a few words per
// frame, next to the record bytes the put, CRC and fetch kernels move.
#include "hkv_device.h"
#include "hkv_launch.h"

namespace hkv {
namespace {

constexpr uint32_t kPoly = 0xEDB88320u;
constexpr uint32_t kMagic = 0x46564B48u;        // "HKVF"
constexpr uint32_t kVersionWord = 1u | (64u << 16);

struct FrameParams {
  uint8_t* base;
  int64_t layer, block;          // byte strides between frames
  int32_t n_layers, n_blocks;
  uint32_t geometry_word0;       // bytes 8..11: format, 0, head_dim
  uint32_t geometry_word1;       // bytes 12..15: block_tokens, n_kv_heads
  uint32_t payload_bytes;
  uint32_t layer_base;
};

__device__ __forceinline__ void build_table(uint32_t* T) {
  for (int i = threadIdx.x; i < 256; i += blockDim.x) {
    uint32_t c = static_cast<uint32_t>(i);
#pragma unroll
    for (int k = 0; k < 8; ++k) c = (c >> 1) ^ (kPoly & (0u - (c & 1u)));
    T[i] = c;
  }
  __syncthreads();
}

// CRC-32 (zlib variant) of 15 little-endian words.
__device__ __forceinline__ uint32_t crc_of_words(const uint32_t* T, const uint32_t (&w)[15]) {
  uint32_t c = 0xFFFFFFFFu;
#pragma unroll
  for (int i = 0; i < 15; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) c = T[(c ^ (w[i] >> (8 * j))) & 0xFFu] ^ (c >> 8);
  }
  return ~c;
}

__device__ __forceinline__ uint8_t* frame_at(const FrameParams& p, int r) {
  const int l = r / p.n_blocks;
  const int b = r - l * p.n_blocks;
  return p.base + l * p.layer + b * p.block;
}

__global__ __launch_bounds__(kThreads) void frame_header_kernel(FrameParams p,
                                                                const uint32_t* crc,
                                                                const int32_t* m_old) {
  __shared__ uint32_t T[256];
  build_table(T);
  const int r = blockIdx.x * kThreads + threadIdx.x;
  if (r >= p.n_layers * p.n_blocks) return;
  const int l = r / p.n_blocks;
  const int b = r - l * p.n_blocks;
  uint32_t w[15] = {kMagic, kVersionWord, p.geometry_word0, p.geometry_word1,
                    p.layer_base + static_cast<uint32_t>(l), static_cast<uint32_t>(b),
                    static_cast<uint32_t>(m_old[b]), p.payload_bytes, crc[r],
                    0, 0, 0, 0, 0, 0};
  const uint32_t hcrc = crc_of_words(T, w);
  u32x4* dst = reinterpret_cast<u32x4*>(frame_at(p, r));
  dst[0] = u32x4{w[0], w[1], w[2], w[3]};
  dst[1] = u32x4{w[4], w[5], w[6], w[7]};
  dst[2] = u32x4{w[8], 0u, 0u, 0u};
  dst[3] = u32x4{0u, 0u, 0u, hcrc};
}

// status[r] holds the freshly computed payload CRC on entry and the flags
// on exit.
__global__ __launch_bounds__(kThreads) void frame_verify_kernel(FrameParams p,
                                                                uint32_t* status) {
  __shared__ uint32_t T[256];
  build_table(T);
  const int r = blockIdx.x * kThreads + threadIdx.x;
  if (r >= p.n_layers * p.n_blocks) return;
  const int l = r / p.n_blocks;
  const int b = r - l * p.n_blocks;
  const u32x4* src = reinterpret_cast<const u32x4*>(frame_at(p, r));
  const u32x4 h0 = src[0], h1 = src[1], h2 = src[2], h3 = src[3];
  const uint32_t w[15] = {h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3],
                          h2[0], h2[1], h2[2], h2[3], h3[0], h3[1], h3[2]};
  uint32_t f = 0;
  if (w[0] != kMagic || w[1] != kVersionWord) f |= 1u;
  if (crc_of_words(T, w) != h3[3]) f |= 2u;
  // byte 9 is reserved: covered by the header CRC only
  if ((w[2] & 0xFFFF00FFu) != p.geometry_word0 || w[3] != p.geometry_word1 ||
      w[7] != p.payload_bytes)
    f |= 4u;
  if (w[4] != p.layer_base + static_cast<uint32_t>(l) || w[5] != static_cast<uint32_t>(b))
    f |= 8u;
  if (w[8] != status[r]) f |= 16u;
  status[r] = f;
}

__global__ __launch_bounds__(kThreads) void frame_delta_kernel(FrameParams p,
                                                               const int32_t* m_new,
                                                               int32_t* delta) {
  const int b = blockIdx.x * kThreads + threadIdx.x;
  if (b >= p.n_blocks) return;
  const int32_t m_old = *reinterpret_cast<const int32_t*>(p.base + b * p.block + 24);
  const int64_t d = static_cast<int64_t>(m_new[b]) - m_old;
  delta[b] = static_cast<int32_t>(d > INT32_MAX ? INT32_MAX : (d < INT32_MIN ? INT32_MIN : d));
}

FrameParams make_params(int fmt, const Geometry& g, const RecordView& frames,
                        int64_t record_bytes, int32_t layer_base) {
  FrameParams p;
  p.base = frames.base;
  p.layer = frames.layer;
  p.block = frames.block;
  p.n_layers = g.n_layers;
  p.n_blocks = g.n_blocks;
  p.geometry_word0 = (fmt == kFP8 ? 0u : 1u) | (static_cast<uint32_t>(kHeadDim) << 16);
  p.geometry_word1 = static_cast<uint32_t>(g.block_tokens) |
                     (static_cast<uint32_t>(g.n_heads) << 16);
  p.payload_bytes = static_cast<uint32_t>(record_bytes);
  p.layer_base = static_cast<uint32_t>(layer_base);
  return p;
}

unsigned groups_for(int64_t n) { return static_cast<unsigned>((n + kThreads - 1) / kThreads); }

}  // namespace

hipError_t launch_frame_headers(int fmt, const Geometry& g, const RecordView& frames,
                                int64_t record_bytes, int32_t layer_base, const uint32_t* crc,
                                const int32_t* m_old, hipStream_t stream) {
  const FrameParams p = make_params(fmt, g, frames, record_bytes, layer_base);
  hipLaunchKernelGGL(frame_header_kernel,
                     dim3(groups_for(static_cast<int64_t>(g.n_layers) * g.n_blocks)),
                     dim3(kThreads), 0, stream, p, crc, m_old);
  return hipGetLastError();
}

hipError_t launch_frame_verify(int fmt, const Geometry& g, const RecordView& frames,
                               int64_t record_bytes, int32_t layer_base, uint32_t* status,
                               hipStream_t stream) {
  const RecordView payload{frames.base + kFrameHeaderBytes, frames.layer, frames.block};
  hipError_t e = launch_crc32(g, record_bytes, payload, nullptr, 0, status, stream);
  if (e != hipSuccess) return e;
  const FrameParams p = make_params(fmt, g, frames, record_bytes, layer_base);
  hipLaunchKernelGGL(frame_verify_kernel,
                     dim3(groups_for(static_cast<int64_t>(g.n_layers) * g.n_blocks)),
                     dim3(kThreads), 0, stream, p, status);
  return hipGetLastError();
}

hipError_t launch_frame_delta(const Geometry& g, const RecordView& frames, const int32_t* m_new,
                              int32_t* delta, hipStream_t stream) {
  FrameParams p{};
  p.base = frames.base;
  p.block = frames.block;
  p.n_blocks = g.n_blocks;
  hipLaunchKernelGGL(frame_delta_kernel, dim3(groups_for(g.n_blocks)), dim3(kThreads), 0,
                     stream, p, m_new, delta);
  return hipGetLastError();
}

}  // namespace hkv
