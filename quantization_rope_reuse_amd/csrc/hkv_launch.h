// Internal launch interface between the validated C ABI (api.hip) and the
// kernel sources.  All strides here are in BYTES; the ABI layer converts the
// element strides of hkv_pages.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <initializer_list>

#include "hkv.h"

namespace hkv {

// Geometry of one call, after validation.
struct Geometry {
  int32_t n_layers;
  int32_t n_blocks;
  int32_t block_tokens;
  int32_t n_heads;
  int32_t vecs;            // block_tokens * n_heads vectors per (block, K|V)
};

struct PageView {          // byte addressing of a paged buffer
  char* k;
  char* v;
  int64_t layer, page, token, head;
  int32_t num_pages;
};

struct RecordView {
  uint8_t* base;
  int64_t layer, block;
};

hipError_t launch_quant(int fmt, int src_dtype, const Geometry& g, const PageView& src,
                        const int32_t* table, const RecordView& dst, hipStream_t stream);

hipError_t launch_fetch(int fmt, int dst_dtype, int pairs, const Geometry& g,
                        const RecordView& src, const int32_t* table, const int32_t* delta_m,
                        bool delta_per_token, const int32_t* visit_order, double rope_base,
                        const PageView& dst, hipStream_t stream);

hipError_t launch_page_order(const int32_t* table, int32_t n_blocks, int32_t num_pages,
                             int32_t* order, hipStream_t stream);

// table: NULL (every record), or the block table: records of blocks whose
// entry is negative or >= num_pages are skipped and their CRCs not written.
hipError_t launch_crc32(const Geometry& g, int64_t record_bytes, const RecordView& src,
                        const int32_t* table, int32_t num_pages, uint32_t* out,
                        hipStream_t stream);

// Fused put + CRC: the put also writes the raw CRC of every 128-byte unit of
// the codes of every record to `partials` (layer-major, record_bytes / 128
// slots per record, the scale units' slots unused); requires
// g.vecs % 64 == 0.  The merge reads the scale units back from the records
// and turns both into the records' CRCs.
hipError_t launch_quant_crc_units(int fmt, int src_dtype, const Geometry& g, const PageView& src,
                                  const int32_t* table, const RecordView& dst,
                                  int64_t record_bytes, uint32_t* partials, hipStream_t stream);

// The largest byte offset a view addresses, (count_i - 1) * stride_i summed
// plus `tail`, must stay below 2^47, beyond the device's virtual address
// space (no valid buffer reaches it); the kernels' 64-bit offset arithmetic
// then cannot overflow.  Strides are non-negative byte strides.
constexpr int64_t kMaxSpan = int64_t{1} << 47;
struct Extent {
  int64_t count, stride;
};
bool span_ok(std::initializer_list<Extent> dims, int64_t tail);

// Validated views of one fetch call (hkv_fetch_dequant_rope_shift's checks).
struct FetchViews {
  Geometry g;
  RecordView rv;
  PageView pv;
};
int fetch_check(const hkv_shape* shape, int32_t fmt, const hkv_records* src,
                const int32_t* block_table, const int32_t* delta_m, double rope_base,
                int32_t pairs, const hkv_pages* dst, int32_t dst_dtype, FetchViews* views);

// Host-side argument checks of the fused put + CRC (hkv_quant_*_crc), all
// but the workspace; on HKV_OK *workspace_bytes is the workspace it needs.
int quant_crc_validate(int32_t fmt, const hkv_shape* shape, const hkv_pages* src,
                       int32_t src_dtype, const int32_t* block_table, const hkv_records* dst,
                       const uint32_t* crc_out, int64_t* workspace_bytes);

hipError_t launch_crc32_merge(const Geometry& g, int64_t record_bytes, const RecordView& src,
                              const int32_t* table, int32_t num_pages, const uint32_t* partials,
                              uint32_t* out, hipStream_t stream);

// Measurement aid: read units16 x 16 bytes, write each twice (1:2 stream).
hipError_t launch_stream_expand(const void* src, void* dst, int64_t units16, hipStream_t stream);

// Measurement aid: rows of 256 source bytes -> rows of 128 bytes (2:1 stream).
hipError_t launch_stream_squeeze(const void* src, void* dst, int64_t rows, hipStream_t stream);

// Frames: a kFrameHeaderBytes header, then the record.
constexpr int64_t kFrameHeaderBytes = 64;

hipError_t launch_frame_headers(int fmt, const Geometry& g, const RecordView& frames,
                                int64_t record_bytes, int32_t layer_base, const uint32_t* crc,
                                const int32_t* m_old, hipStream_t stream);

hipError_t launch_frame_verify(int fmt, const Geometry& g, const RecordView& frames,
                               int64_t record_bytes, int32_t layer_base, uint32_t* status,
                               hipStream_t stream);

hipError_t launch_frame_delta(const Geometry& g, const RecordView& frames, const int32_t* m_new,
                              int32_t* delta, hipStream_t stream);

hipError_t launch_drift(int dtype, const void* cached, const void* fresh, int32_t n_tokens,
                        int32_t d_model, int64_t row_bytes, float* drift, hipStream_t stream);

// Workspace of the many-workgroup selection for n values.
int64_t select_workspace_bytes(int32_t n);

// workspace: NULL (one workgroup) or select_workspace_bytes(n) bytes.
hipError_t launch_topk(const float* drift, int32_t n, int32_t k, int32_t* selected,
                       void* workspace, hipStream_t stream);

}  // namespace hkv
