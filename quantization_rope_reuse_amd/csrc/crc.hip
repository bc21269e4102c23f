// CRC-32 of every compressed record.
//
// The HyperCache post ("HyperCache – Distributed KV-cache quantization and
// relative RoPE reuse") stores its INT4 disk records with a CRC32 (Part B,
// the L3-disk line) and tests tamper detection with it.  The variant here is
// the common zlib one: reflected polynomial 0xEDB88320, initial value and
// final xor 0xFFFFFFFF.
//
// Parallel form.  The CRC register update is linear over GF(2).  Writing
// raw(M) for the register after feeding message M into a zero register,
//   raw(A || B) = raw(A) * x^(8|B|) mod P  xor  raw(B),
// and the standard CRC is ~(0xFFFFFFFF * x^(8|M|) mod P  xor  raw(M)).
// One wave handles one record: lane i feeds its contiguous chunk of
// `chunk` bytes into a zero register, a word per three table lookups; the
// chunk is followed by 63 - i chunks, so lane i multiplies its value by
// x^(8 * chunk * (63 - i)) and the record's raw CRC is the xor of the 64
// products.  Leading zero bytes leave a zero register unchanged, so a record
// shorter than 64 * chunk is handled by treating it as preceded by `pad` zero
// bytes.  The 64 constants depend only on the record size and are computed
// once per launch on the host.
#include "crc_device.h"
#include "hkv_device.h"
#include "hkv_launch.h"

namespace hkv {
namespace {

constexpr int kRecordsPerGroup = kThreads / kWave;

struct CrcParams {
  const uint8_t* rec;
  int64_t rec_layer, rec_block;
  uint32_t* out;
  const int32_t* table;  // optional: skip the records of skipped blocks
  int32_t num_pages;
  int32_t n_blocks;
  int32_t n_records;
  int32_t chunk;         // bytes per lane (multiple of 4)
  int32_t pad;           // 64 * chunk - record bytes
  int32_t aligned;       // chunk and pad multiples of 16
  uint32_t lane_shift[kWave];   // x^(8 * chunk * (63 - i)) mod P, reflected
  uint32_t init_term;    // 0xFFFFFFFF * x^(8 * record bytes) mod P
};

// Feeding a little-endian word w into the register is c <- A(c ^ w), with A
// the linear map "shift through 32 zero bits".  A splits over the bit
// fields [0, 11), [11, 22) and [22, 32) of its argument, so one word costs
// three lookups in the tables T0[v] = A(v), T1[v] = A(v << 11),
// T2[v] = A(v << 22) (2,048 + 2,048 + 1,024 entries in LDS).
__device__ __forceinline__ uint32_t feed_word(const uint32_t* T0, const uint32_t* T1,
                                              const uint32_t* T2, uint32_t c, uint32_t w) {
  c ^= w;
  return T0[c & 0x7FFu] ^ T1[(c >> 11) & 0x7FFu] ^ T2[c >> 22];
}

// A(1 << k), k = 0..31, by 32 bit steps.
__device__ __forceinline__ uint32_t shift32(uint32_t x) {
#pragma unroll
  for (int k = 0; k < 32; ++k) x = (x >> 1) ^ (kCrcPoly & (0u - (x & 1u)));
  return x;
}

// Builds T0 | T1 | T2 (5,120 words) in LDS with 256 threads: the 32 basis
// values A(1 << k) first, then each thread fills runs of 8 consecutive
// entries, entry v0 + t being the run's first entry xor the basis
// combination of t.
__device__ __forceinline__ void build_tables(uint32_t* T, uint32_t* basis, int tid) {
  if (tid < 32) basis[tid] = shift32(1u << tid);
  __syncthreads();
  for (int run = tid; run < 5120 / 8; run += kThreads) {
    const int e0 = run * 8;                      // first entry of the run
    const int off = e0 < 2048 ? 0 : (e0 < 4096 ? 11 : 22);
    const int v0 = e0 - (off == 0 ? 0 : (off == 11 ? 2048 : 4096));
    uint32_t head = 0;
    const int bits = off == 22 ? 10 : 11;
    for (int j = 3; j < bits; ++j)
      if ((v0 >> j) & 1) head ^= basis[off + j];
    const uint32_t b0 = basis[off], b1 = basis[off + 1], b2 = basis[off + 2];
#pragma unroll
    for (int t = 0; t < 8; ++t)
      T[e0 + t] = head ^ ((t & 1) ? b0 : 0u) ^ ((t & 2) ? b1 : 0u) ^ ((t & 4) ? b2 : 0u);
  }
  __syncthreads();
}

__global__ __launch_bounds__(kThreads) void crc32_kernel(CrcParams p) {
  __shared__ uint32_t T[5120];
  __shared__ uint32_t basis[32];
  const int tid = threadIdx.x;
  build_tables(T, basis, tid);
  const uint32_t* T0 = T;
  const uint32_t* T1 = T + 2048;
  const uint32_t* T2 = T + 4096;

  const int lane = tid & (kWave - 1);
  const int r = blockIdx.x * kRecordsPerGroup + tid / kWave;
  if (r >= p.n_records) return;                 // whole wave, after the barriers
  const int layer = r / p.n_blocks;
  const int blk = r - layer * p.n_blocks;
  if (p.table) {
    const int page = p.table[blk];
    if (page < 0 || page >= p.num_pages) return;  // whole wave: a skipped block
  }
  const uint8_t* rec = p.rec + layer * p.rec_layer + blk * p.rec_block;

  const int64_t start = static_cast<int64_t>(lane) * p.chunk - p.pad;   // may be < 0
  int u = start < 0 ? static_cast<int>(min<int64_t>(-start, p.chunk)) : 0;
  uint32_t crc = 0;
  if (p.aligned) {
    const uint8_t* base = rec + start;
    for (; u + 128 <= p.chunk; u += 128) {
      u32x4 w[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) w[j] = *reinterpret_cast<const u32x4*>(base + u + 16 * j);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        crc = feed_word(T0, T1, T2, crc, w[j][0]);
        crc = feed_word(T0, T1, T2, crc, w[j][1]);
        crc = feed_word(T0, T1, T2, crc, w[j][2]);
        crc = feed_word(T0, T1, T2, crc, w[j][3]);
      }
    }
    for (; u < p.chunk; u += 16) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(base + u);
      crc = feed_word(T0, T1, T2, crc, w[0]);
      crc = feed_word(T0, T1, T2, crc, w[1]);
      crc = feed_word(T0, T1, T2, crc, w[2]);
      crc = feed_word(T0, T1, T2, crc, w[3]);
    }
  } else {
    const uint8_t* base = rec + start;
    for (; u < p.chunk; u += 4)
      crc = feed_word(T0, T1, T2, crc, *reinterpret_cast<const uint32_t*>(base + u));
  }

  // lane i's chunk is followed by 63 - i chunks
  crc = crc_mulmod(crc, p.lane_shift[lane]);
#pragma unroll
  for (int k = 0; k < 6; ++k) crc ^= __shfl_xor(crc, 1 << k);
  if (lane == 0) p.out[r] = ~(p.init_term ^ crc);
}

// Merge of the fused put + CRC.  A record is [codes][scales]: code_units
// 128-byte units of codes (a multiple of 64) whose raw CRCs the put wrote to
// `partials`, then scale_bytes of fp16 scales (a multiple of 256), which the
// merge reads back from the record.  One wave per record.  Lane i runs a
// Horner chain over its code units i, i+64, i+128, ...:
//   c <- c * x^(8*128*64) xor raw(unit)
// (the constant multiplication is four lookups in the tables M), and feeds
// its own scale_bytes/64 consecutive scale bytes into a zero register s
// (byte tables T).  Unit i + 64j sits 64(n-1-j) + (63-i) units before the
// end of the codes, so the record's raw CRC is the xor over the lanes of
//   c * x^(8*128*(63-i) + 8*scale_bytes)  xor  s * x^(8*(scale_bytes/64)*(63-i)),
// two GF(2) multiplications per lane by constants computed on the host, then
// a butterfly xor over the wave.  Records of skipped blocks (table entry
// negative or >= num_pages) are left alone.
struct MergeParams {
  const uint32_t* partials;
  const uint8_t* rec;
  int64_t rec_layer, rec_block;
  const int32_t* table;
  uint32_t* out;
  int32_t n_blocks, n_records, num_pages;
  int32_t units;               // partial slots per record (record bytes / 128)
  int32_t code_units;          // multiple of 64
  int32_t scale_bytes;         // multiple of 256
  uint32_t m_basis[4][8];      // (1 << (8k + i)) * x^(8 * 128 * 64) mod P
  uint32_t t_basis[4][8];      // (1 << i) * x^(8 * (s + 1)) mod P: the byte tables T
  uint32_t code_shift[kWave];  // x^(8*128*(63-i) + 8*scale_bytes) mod P
  uint32_t scale_shift[kWave]; // x^(8*(scale_bytes/64)*(63-i)) mod P
  uint32_t init_term;          // 0xFFFFFFFF * x^(8 * record bytes) mod P
};

constexpr int kMergeBatch = 24;

// One record's CRC in one wave (see above).
__device__ __forceinline__ void merge_record(const MergeParams& p, const uint32_t (*M)[256],
                                             const uint32_t (*T)[256], int r, int lane) {
  const int layer = r / p.n_blocks;
  const int blk = r - layer * p.n_blocks;
  const int page = p.table[blk];
  if (page < 0 || page >= p.num_pages) return;   // whole wave
  const uint32_t* part = p.partials + static_cast<int64_t>(r) * p.units + lane;
  const int per_lane = p.scale_bytes / kWave;    // bytes, a multiple of 4
  const uint32_t* sc = reinterpret_cast<const uint32_t*>(
      p.rec + layer * p.rec_layer + blk * p.rec_block + static_cast<int64_t>(p.code_units) * 128 +
      static_cast<int64_t>(lane) * per_lane);
  const uint32_t code_k = p.code_shift[lane];
  const uint32_t scale_k = p.scale_shift[lane];
  const int n = p.code_units / kWave;            // code units per lane
  const int words = per_lane / 4;                 // scale words per lane
  // Batches of kMergeBatch of each: a batch's loads are all issued before
  // either chain consumes them (one batch for up to 24 code units and 96
  // scale bytes per lane; the batch guards are uniform over the wave).
  uint32_t c = 0, sreg = 0;
  for (int j0 = 0; j0 < n || j0 < words; j0 += kMergeBatch) {
    uint32_t w[kMergeBatch], x[kMergeBatch];
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i)
      w[i] = j0 + i < n ? part[static_cast<int64_t>(kWave) * (j0 + i)] : 0u;
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i) x[i] = j0 + i < words ? sc[j0 + i] : 0u;
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i) {
      if (j0 + i < n)
        c = M[0][c & 0xFFu] ^ M[1][(c >> 8) & 0xFFu] ^ M[2][(c >> 16) & 0xFFu] ^ M[3][c >> 24] ^
            w[i];
      if (j0 + i < words) sreg = crc_feed_word(T, sreg, x[i]);
    }
  }
  uint32_t v = crc_mulmod(c, code_k) ^ crc_mulmod(sreg, scale_k);
#pragma unroll
  for (int k = 0; k < 6; ++k) v ^= __shfl_xor(v, 1 << k);
  if (lane == 0) p.out[r] = ~(p.init_term ^ v);
}

// One wave per record (several records per wave measured slower).
__global__ __launch_bounds__(kThreads) void crc32_merge_kernel(MergeParams p) {
  __shared__ uint32_t M[4][256];                 // M[k][b] = (b at byte k) * x^(8*128*64)
  __shared__ uint32_t T[4][256];                 // T[s][b] = b * x^(8(s+1))
  const int tid = threadIdx.x;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint32_t m = 0, t = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t bit = 0u - ((static_cast<uint32_t>(tid) >> i) & 1u);
      m ^= p.m_basis[k][i] & bit;
      t ^= p.t_basis[k][i] & bit;
    }
    M[k][tid] = m;
    T[k][tid] = t;
  }
  __syncthreads();
  const int r = blockIdx.x * kRecordsPerGroup + tid / kWave;
  if (r >= p.n_records) return;                  // whole wave, after the barrier
  merge_record(p, M, T, r, tid & (kWave - 1));
}

}  // namespace

hipError_t launch_crc32(const Geometry& g, int64_t record_bytes, const RecordView& src,
                        const int32_t* table, int32_t num_pages, uint32_t* out,
                        hipStream_t stream) {
  CrcParams p;
  p.rec = src.base;
  p.rec_layer = src.layer;
  p.rec_block = src.block;
  p.out = out;
  p.table = table;
  p.num_pages = num_pages;
  p.n_blocks = g.n_blocks;
  p.n_records = g.n_layers * g.n_blocks;
  // Lane chunks are whole 128-byte cache lines when the record size allows
  // (each batch of eight 16-byte loads then covers exactly one line), else
  // 16-byte or 4-byte multiples; the difference is made up by leading zeros.
  const int64_t per_lane = (record_bytes + kWave - 1) / kWave;
  const bool aligned = record_bytes % 16 == 0;
  const int64_t unit = record_bytes % 128 == 0 ? 128 : (aligned ? 16 : 4);
  const int64_t chunk = (per_lane + unit - 1) / unit * unit;
  p.chunk = static_cast<int32_t>(chunk);
  p.pad = static_cast<int32_t>(kWave * chunk - record_bytes);
  p.aligned = aligned ? 1 : 0;
  for (int i = 0; i < kWave; ++i)
    p.lane_shift[i] = crc_x8n(static_cast<uint64_t>(chunk) * static_cast<uint64_t>(kWave - 1 - i));
  p.init_term = crc_mulmod(0xFFFFFFFFu, crc_x8n(static_cast<uint64_t>(record_bytes)));
  const unsigned groups =
      static_cast<unsigned>((p.n_records + kRecordsPerGroup - 1) / kRecordsPerGroup);
  hipLaunchKernelGGL(crc32_kernel, dim3(groups), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_crc32_merge(const Geometry& g, int64_t record_bytes, const RecordView& src,
                              const int32_t* table, int32_t num_pages, const uint32_t* partials,
                              uint32_t* out, hipStream_t stream) {
  MergeParams p;
  p.partials = partials;
  p.rec = src.base;
  p.rec_layer = src.layer;
  p.rec_block = src.block;
  p.table = table;
  p.out = out;
  p.n_blocks = g.n_blocks;
  p.n_records = g.n_layers * g.n_blocks;
  p.num_pages = num_pages;
  // the scales (2 x vecs fp16) close the record; everything before is codes
  const int64_t scale_bytes = 4LL * g.vecs;
  const int64_t code_units = (record_bytes - scale_bytes) / 128;
  if (g.vecs % 64 != 0 || code_units % kWave != 0 || scale_bytes % (4 * kWave) != 0)
    return hipErrorInvalidValue;
  p.units = static_cast<int32_t>(record_bytes / 128);
  p.code_units = static_cast<int32_t>(code_units);
  p.scale_bytes = static_cast<int32_t>(scale_bytes);
  const uint32_t mul_lanes = crc_x8n(static_cast<uint64_t>(128) * kWave);
  for (int k = 0; k < 4; ++k)
    for (int i = 0; i < 8; ++i) p.m_basis[k][i] = crc_mulmod(1u << (8 * k + i), mul_lanes);
  for (int s = 0; s < 4; ++s)
    for (int i = 0; i < 8; ++i)
      p.t_basis[s][i] = crc_mulmod(1u << i, crc_x8n(static_cast<uint64_t>(s + 1)));
  for (int i = 0; i < kWave; ++i) {
    const uint64_t back = static_cast<uint64_t>(kWave - 1 - i);
    p.code_shift[i] = crc_x8n(128 * back + static_cast<uint64_t>(scale_bytes));
    p.scale_shift[i] = crc_x8n(static_cast<uint64_t>(scale_bytes / kWave) * back);
  }
  p.init_term = crc_mulmod(0xFFFFFFFFu, crc_x8n(static_cast<uint64_t>(record_bytes)));
  const unsigned groups =
      static_cast<unsigned>((p.n_records + kRecordsPerGroup - 1) / kRecordsPerGroup);
  hipLaunchKernelGGL(crc32_merge_kernel, dim3(groups), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace hkv
