// libhkv C ABI: argument validation and dispatch to the kernel launchers.
// Every check runs on the host before any HIP call, so argument errors are
// reported without touching a device.
#include "hkv.h"

#include <math.h>
#include <stdint.h>

#include "hkv_device.h"
#include "hkv_launch.h"

namespace {

using hkv::Geometry;
using hkv::PageView;
using hkv::RecordView;

int elem_size(int32_t dtype) {
  switch (dtype) {
    case HKV_F32: return 4;
    case HKV_F16: return 2;
    case HKV_BF16: return 2;
    default: return 0;
  }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t code_bytes(int32_t fmt) { return fmt == HKV_FP8_E4M3 ? 128 : 64; }

bool valid_format(int32_t fmt) { return fmt == HKV_FP8_E4M3 || fmt == HKV_INT4; }

using hkv::span_ok;

// Shape checks common to every call; fills the launch geometry.
int check_shape(const hkv_shape* s, Geometry* g) {
  if (!s) return HKV_ERR_INVALID_ARG;
  if (s->n_layers < 0 || s->n_blocks < 0 || s->block_tokens < 1 || s->n_kv_heads < 1)
    return HKV_ERR_INVALID_ARG;
  if (s->head_dim != HKV_HEAD_DIM) return HKV_ERR_INVALID_ARG;
  if (s->n_layers > 65535) return HKV_ERR_UNSUPPORTED;            // grid.y limit
  const int64_t vecs = static_cast<int64_t>(s->block_tokens) * s->n_kv_heads;
  if (vecs > (1 << 24)) return HKV_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(s->n_layers) * s->n_blocks > INT32_MAX) return HKV_ERR_UNSUPPORTED;
  g->n_layers = s->n_layers;
  g->n_blocks = s->n_blocks;
  g->block_tokens = s->block_tokens;
  g->n_heads = s->n_kv_heads;
  g->vecs = static_cast<int32_t>(vecs);
  // the smallest chunk any kernel uses bounds the workgroup count
  const int64_t per_wg = hkv::kFetchMinGroupVecs;
  const int64_t chunks = (vecs + per_wg - 1) / per_wg;
  if (static_cast<int64_t>(s->n_blocks) * 2 * chunks > INT32_MAX) return HKV_ERR_UNSUPPORTED;
  return HKV_OK;
}

int check_pages(const hkv_pages* p, int32_t dtype, const hkv_shape* s, PageView* v) {
  if (!p) return HKV_ERR_INVALID_ARG;
  const int es = elem_size(dtype);
  if (es == 0) return HKV_ERR_INVALID_ARG;
  if (!p->k || !p->v || !aligned16(p->k) || !aligned16(p->v)) return HKV_ERR_INVALID_ARG;
  if (p->num_pages < 0) return HKV_ERR_INVALID_ARG;
  const int64_t st[4] = {p->layer_stride, p->page_stride, p->token_stride, p->head_stride};
  for (int64_t x : st) {
    if (x < 0 || x > (INT64_MAX / 8)) return HKV_ERR_INVALID_ARG;
    if ((x * es) % 16 != 0) return HKV_ERR_INVALID_ARG;
  }
  v->k = static_cast<char*>(p->k);
  v->v = static_cast<char*>(p->v);
  v->layer = p->layer_stride * es;
  v->page = p->page_stride * es;
  v->token = p->token_stride * es;
  v->head = p->head_stride * es;
  v->num_pages = p->num_pages;
  if (!span_ok({{s->n_layers, v->layer}, {p->num_pages, v->page}, {s->block_tokens, v->token},
                {s->n_kv_heads, v->head}},
               int64_t{HKV_HEAD_DIM} * es))
    return HKV_ERR_INVALID_ARG;
  return HKV_OK;
}

int check_records(const hkv_records* r, int32_t fmt, const hkv_shape* s, RecordView* v) {
  if (!r || !r->base || !aligned16(r->base)) return HKV_ERR_INVALID_ARG;
  if (r->layer_stride_bytes < 0 || r->block_stride_bytes < 0) return HKV_ERR_INVALID_ARG;
  if (r->layer_stride_bytes % 16 != 0 || r->block_stride_bytes % 16 != 0)
    return HKV_ERR_INVALID_ARG;
  const int64_t rb = hkv_record_bytes(fmt, s->block_tokens, s->n_kv_heads, s->head_dim);
  if (rb < 0) return HKV_ERR_INVALID_ARG;
  if (s->n_blocks > 1 && r->block_stride_bytes < rb) return HKV_ERR_INVALID_ARG;
  if (s->n_layers > 1 && r->layer_stride_bytes < rb) return HKV_ERR_INVALID_ARG;
  if (!span_ok({{s->n_layers, r->layer_stride_bytes}, {s->n_blocks, r->block_stride_bytes}}, rb))
    return HKV_ERR_INVALID_ARG;
  v->base = static_cast<uint8_t*>(r->base);
  v->layer = r->layer_stride_bytes;
  v->block = r->block_stride_bytes;
  return HKV_OK;
}

int to_status(hipError_t e) { return e == hipSuccess ? HKV_OK : HKV_ERR_HIP; }

constexpr int32_t kMaxSelectTokens = 1 << 30;
// hkv_page_visit_order compares every pair of blocks (n^2 / 64 wave steps).
constexpr int32_t kMaxOrderBlocks = 1 << 16;

// Frames: the records view describes the frames; each frame must hold the
// header and the record.  Fills the launch geometry and the frame view.
int check_frames(const hkv_shape* shape, int32_t fmt, const hkv_records* frames, Geometry* g,
                 RecordView* v, int64_t* rb) {
  int st;
  if (!valid_format(fmt)) return HKV_ERR_INVALID_ARG;
  if ((st = check_shape(shape, g)) != HKV_OK) return st;
  if (shape->block_tokens > 65535 || shape->n_kv_heads > 65535) return HKV_ERR_UNSUPPORTED;
  if (!frames || !frames->base || !aligned16(frames->base)) return HKV_ERR_INVALID_ARG;
  if (frames->layer_stride_bytes < 0 || frames->block_stride_bytes < 0 ||
      frames->layer_stride_bytes % 16 != 0 || frames->block_stride_bytes % 16 != 0)
    return HKV_ERR_INVALID_ARG;
  *rb = hkv_record_bytes(fmt, shape->block_tokens, shape->n_kv_heads, shape->head_dim);
  const int64_t fb = *rb + hkv::kFrameHeaderBytes;
  if (shape->n_blocks > 1 && frames->block_stride_bytes < fb) return HKV_ERR_INVALID_ARG;
  if (shape->n_layers > 1 && frames->layer_stride_bytes < fb) return HKV_ERR_INVALID_ARG;
  if (*rb > (int64_t{1} << 30)) return HKV_ERR_UNSUPPORTED;
  if (!span_ok({{shape->n_layers, frames->layer_stride_bytes},
                {shape->n_blocks, frames->block_stride_bytes}},
               fb))
    return HKV_ERR_INVALID_ARG;
  v->base = static_cast<uint8_t*>(frames->base);
  v->layer = frames->layer_stride_bytes;
  v->block = frames->block_stride_bytes;
  return HKV_OK;
}

int quant_common(int32_t fmt, const hkv_shape* shape, const hkv_pages* src, int32_t src_dtype,
                 const int32_t* block_table, const hkv_records* dst, hipStream_t stream) {
  Geometry g;
  PageView pv;
  RecordView rv;
  int st;
  if ((st = check_shape(shape, &g)) != HKV_OK) return st;
  if ((st = check_pages(src, src_dtype, shape, &pv)) != HKV_OK) return st;
  if ((st = check_records(dst, fmt, shape, &rv)) != HKV_OK) return st;
  if (!block_table && g.n_blocks > 0) return HKV_ERR_INVALID_ARG;
  if (g.n_layers == 0 || g.n_blocks == 0) return HKV_OK;
  return to_status(hkv::launch_quant(fmt, src_dtype, g, pv, block_table, rv, stream));
}

int64_t quant_crc_workspace(const Geometry& g, int64_t rb) {
  if (g.vecs % 64 != 0) return 0;                 // runs the put and the CRC kernel
  return static_cast<int64_t>(g.n_layers) * g.n_blocks * (rb / 128) * 4;
}

// Argument checks of the fused put + CRC, everything but the workspace.
int quant_crc_check(int32_t fmt, const hkv_shape* shape, const hkv_pages* src,
                    int32_t src_dtype, const int32_t* block_table, const hkv_records* dst,
                    const uint32_t* crc_out, Geometry* g, PageView* pv, RecordView* rv,
                    int64_t* rb, int64_t* need) {
  int st;
  if ((st = check_shape(shape, g)) != HKV_OK) return st;
  if ((st = check_pages(src, src_dtype, shape, pv)) != HKV_OK) return st;
  if ((st = check_records(dst, fmt, shape, rv)) != HKV_OK) return st;
  if (!block_table && g->n_blocks > 0) return HKV_ERR_INVALID_ARG;
  if (!crc_out && g->n_layers > 0 && g->n_blocks > 0) return HKV_ERR_INVALID_ARG;
  *rb = hkv_record_bytes(fmt, shape->block_tokens, shape->n_kv_heads, shape->head_dim);
  if (*rb > (int64_t{1} << 30)) return HKV_ERR_UNSUPPORTED;
  *need = quant_crc_workspace(*g, *rb);
  return HKV_OK;
}

// Records the caller's records_ready event, if any, on the call's stream.
int record_ready(hipEvent_t records_ready, hipStream_t stream) {
  if (records_ready && hipEventRecord(records_ready, stream) != hipSuccess) {
    (void)hipGetLastError();
    return HKV_ERR_HIP;
  }
  return HKV_OK;
}

int quant_crc_common(int32_t fmt, const hkv_shape* shape, const hkv_pages* src,
                     int32_t src_dtype, const int32_t* block_table, const hkv_records* dst,
                     uint32_t* crc_out, void* workspace, int64_t workspace_bytes,
                     hipStream_t stream, hipEvent_t records_ready) {
  Geometry g;
  PageView pv;
  RecordView rv;
  int64_t rb, need;
  const int st = quant_crc_check(fmt, shape, src, src_dtype, block_table, dst, crc_out, &g, &pv,
                                 &rv, &rb, &need);
  if (st != HKV_OK) return st;
  if (need > 0 && (!workspace || !aligned16(workspace) || workspace_bytes < need))
    return HKV_ERR_INVALID_ARG;
  if (g.n_layers == 0 || g.n_blocks == 0) return record_ready(records_ready, stream);
  if (need == 0) {
    const hipError_t e = hkv::launch_quant(fmt, src_dtype, g, pv, block_table, rv, stream);
    if (e != hipSuccess) return HKV_ERR_HIP;
    const int st_ready = record_ready(records_ready, stream);
    if (st_ready != HKV_OK) return st_ready;
    // the CRCs of skipped blocks stay unchanged, as on the one-pass path
    return to_status(hkv::launch_crc32(g, rb, rv, block_table, pv.num_pages, crc_out, stream));
  }
  uint32_t* partials = static_cast<uint32_t*>(workspace);
  const hipError_t e = hkv::launch_quant_crc_units(fmt, src_dtype, g, pv, block_table, rv, rb,
                                                   partials, stream);
  if (e != hipSuccess) return HKV_ERR_HIP;
  const int st_ready = record_ready(records_ready, stream);
  if (st_ready != HKV_OK) return st_ready;
  return to_status(hkv::launch_crc32_merge(g, rb, rv, block_table, pv.num_pages, partials,
                                           crc_out, stream));
}

int fetch_common(const hkv_shape* shape, int32_t fmt, const hkv_records* src,
                 const int32_t* block_table, const int32_t* delta_m, bool per_token,
                 const int32_t* visit_order, double rope_base, int32_t pairs,
                 const hkv_pages* dst, int32_t dst_dtype, hipStream_t stream) {
  hkv::FetchViews f;
  const int st = hkv::fetch_check(shape, fmt, src, block_table, delta_m, rope_base, pairs, dst,
                                  dst_dtype, &f);
  if (st != HKV_OK) return st;
  if (f.g.n_layers == 0 || f.g.n_blocks == 0) return HKV_OK;
  return to_status(hkv::launch_fetch(fmt, dst_dtype, pairs, f.g, f.rv, block_table, delta_m,
                                     per_token, visit_order, rope_base, f.pv, stream));
}


}  // namespace

namespace hkv {

bool span_ok(std::initializer_list<Extent> dims, int64_t tail) {
  if (tail < 0 || tail > kMaxSpan) return false;
  int64_t total = tail;
  for (const Extent& d : dims) {
    if (d.count <= 1 || d.stride == 0) continue;
    const int64_t n = d.count - 1;
    if (d.stride < 0 || d.stride > (kMaxSpan - total) / n) return false;
    total += n * d.stride;
  }
  return true;
}

int fetch_check(const hkv_shape* shape, int32_t fmt, const hkv_records* src,
                const int32_t* block_table, const int32_t* delta_m, double rope_base,
                int32_t pairs, const hkv_pages* dst, int32_t dst_dtype, FetchViews* f) {
  int st;
  if (!valid_format(fmt)) return HKV_ERR_INVALID_ARG;
  if ((st = check_shape(shape, &f->g)) != HKV_OK) return st;
  if ((st = check_records(src, fmt, shape, &f->rv)) != HKV_OK) return st;
  if ((st = check_pages(dst, dst_dtype, shape, &f->pv)) != HKV_OK) return st;
  if (pairs != HKV_ROPE_INTERLEAVED && pairs != HKV_ROPE_HALF_SPLIT) return HKV_ERR_INVALID_ARG;
  if (!(rope_base > 0.0) || !isfinite(rope_base)) return HKV_ERR_INVALID_ARG;
  if ((!block_table || !delta_m) && f->g.n_blocks > 0) return HKV_ERR_INVALID_ARG;
  return HKV_OK;
}

int quant_crc_validate(int32_t fmt, const hkv_shape* shape, const hkv_pages* src,
                       int32_t src_dtype, const int32_t* block_table, const hkv_records* dst,
                       const uint32_t* crc_out, int64_t* workspace_bytes) {
  Geometry g;
  PageView pv;
  RecordView rv;
  int64_t rb;
  return quant_crc_check(fmt, shape, src, src_dtype, block_table, dst, crc_out, &g, &pv, &rv,
                         &rb, workspace_bytes);
}

}  // namespace hkv

extern "C" {

int64_t hkv_record_bytes(int32_t fmt, int32_t block_tokens, int32_t n_kv_heads,
                         int32_t head_dim) {
  if (!valid_format(fmt) || block_tokens < 1 || n_kv_heads < 1 || head_dim != HKV_HEAD_DIM)
    return -1;
  const int64_t n = static_cast<int64_t>(block_tokens) * n_kv_heads;
  return 2 * n * code_bytes(fmt) + 4 * n;
}

const char* hkv_status_string(int32_t status) {
  switch (status) {
    case HKV_OK: return "ok";
    case HKV_ERR_INVALID_ARG: return "invalid argument";
    case HKV_ERR_UNSUPPORTED: return "unsupported request";
    case HKV_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

int hkv_quant_fp8(const hkv_shape* shape, const hkv_pages* src, int32_t src_dtype,
                  const int32_t* block_table, const hkv_records* dst, hipStream_t stream) {
  return quant_common(HKV_FP8_E4M3, shape, src, src_dtype, block_table, dst, stream);
}

int hkv_quant_int4(const hkv_shape* shape, const hkv_pages* src, int32_t src_dtype,
                   const int32_t* block_table, const hkv_records* dst, hipStream_t stream) {
  return quant_common(HKV_INT4, shape, src, src_dtype, block_table, dst, stream);
}


int64_t hkv_quant_crc_workspace_bytes(const hkv_shape* shape, int32_t fmt) {
  Geometry g;
  if (!valid_format(fmt) || check_shape(shape, &g) != HKV_OK) return -1;
  const int64_t rb = hkv_record_bytes(fmt, shape->block_tokens, shape->n_kv_heads,
                                      shape->head_dim);
  return quant_crc_workspace(g, rb);
}

int hkv_quant_fp8_crc(const hkv_shape* shape, const hkv_pages* src, int32_t src_dtype,
                      const int32_t* block_table, const hkv_records* dst, uint32_t* crc_out,
                      void* workspace, int64_t workspace_bytes, hipStream_t stream,
                      hipEvent_t records_ready) {
  return quant_crc_common(HKV_FP8_E4M3, shape, src, src_dtype, block_table, dst, crc_out,
                          workspace, workspace_bytes, stream, records_ready);
}

int hkv_quant_int4_crc(const hkv_shape* shape, const hkv_pages* src, int32_t src_dtype,
                       const int32_t* block_table, const hkv_records* dst, uint32_t* crc_out,
                       void* workspace, int64_t workspace_bytes, hipStream_t stream,
                       hipEvent_t records_ready) {
  return quant_crc_common(HKV_INT4, shape, src, src_dtype, block_table, dst, crc_out,
                          workspace, workspace_bytes, stream, records_ready);
}

int hkv_fetch_dequant_rope_shift(const hkv_shape* shape, int32_t fmt, const hkv_records* src,
                                 const int32_t* block_table, const int32_t* delta_m,
                                 const int32_t* visit_order, double rope_base, int32_t pairs,
                                 const hkv_pages* dst, int32_t dst_dtype, hipStream_t stream) {
  return fetch_common(shape, fmt, src, block_table, delta_m, false, visit_order, rope_base,
                      pairs, dst, dst_dtype, stream);
}

int hkv_fetch_dequant_rope_shift_tokens(const hkv_shape* shape, int32_t fmt,
                                        const hkv_records* src, const int32_t* block_table,
                                        const int32_t* delta_m_tokens,
                                        const int32_t* visit_order, double rope_base,
                                        int32_t pairs, const hkv_pages* dst, int32_t dst_dtype,
                                        hipStream_t stream) {
  return fetch_common(shape, fmt, src, block_table, delta_m_tokens, true, visit_order,
                      rope_base, pairs, dst, dst_dtype, stream);
}

int hkv_page_visit_order(const int32_t* block_table, int32_t n_blocks, int32_t num_pages,
                         int32_t* order_out, hipStream_t stream) {
  if (n_blocks < 0 || num_pages < 0) return HKV_ERR_INVALID_ARG;
  if (n_blocks > kMaxOrderBlocks) return HKV_ERR_UNSUPPORTED;
  if (n_blocks == 0) return HKV_OK;
  if (!block_table || !order_out) return HKV_ERR_INVALID_ARG;
  return to_status(hkv::launch_page_order(block_table, n_blocks, num_pages, order_out, stream));
}

int hkv_crc32_blocks(const hkv_shape* shape, int32_t fmt, const hkv_records* src,
                     uint32_t* crc_out, hipStream_t stream) {
  Geometry g;
  RecordView rv;
  int st;
  if (!valid_format(fmt)) return HKV_ERR_INVALID_ARG;
  if ((st = check_shape(shape, &g)) != HKV_OK) return st;
  if ((st = check_records(src, fmt, shape, &rv)) != HKV_OK) return st;
  if (!crc_out && g.n_layers > 0 && g.n_blocks > 0) return HKV_ERR_INVALID_ARG;
  if (g.n_layers == 0 || g.n_blocks == 0) return HKV_OK;
  const int64_t rb = hkv_record_bytes(fmt, shape->block_tokens, shape->n_kv_heads,
                                      shape->head_dim);
  if (rb > (int64_t{1} << 30)) return HKV_ERR_UNSUPPORTED;
  return to_status(hkv::launch_crc32(g, rb, rv, nullptr, 0, crc_out, stream));
}

int hkv_frame_headers(const hkv_shape* shape, int32_t fmt, const hkv_records* frames,
                      const uint32_t* crc, const int32_t* m_old, int32_t layer_base,
                      hipStream_t stream) {
  Geometry g;
  RecordView v;
  int64_t rb;
  int st;
  if ((st = check_frames(shape, fmt, frames, &g, &v, &rb)) != HKV_OK) return st;
  if (layer_base < 0) return HKV_ERR_INVALID_ARG;
  if (g.n_layers == 0 || g.n_blocks == 0) return HKV_OK;
  if (!crc || !m_old) return HKV_ERR_INVALID_ARG;
  return to_status(hkv::launch_frame_headers(fmt, g, v, rb, layer_base, crc, m_old, stream));
}

int hkv_frame_verify(const hkv_shape* shape, int32_t fmt, const hkv_records* frames,
                     int32_t layer_base, uint32_t* status_out, hipStream_t stream) {
  Geometry g;
  RecordView v;
  int64_t rb;
  int st;
  if ((st = check_frames(shape, fmt, frames, &g, &v, &rb)) != HKV_OK) return st;
  if (layer_base < 0) return HKV_ERR_INVALID_ARG;
  if (g.n_layers == 0 || g.n_blocks == 0) return HKV_OK;
  if (!status_out) return HKV_ERR_INVALID_ARG;
  return to_status(hkv::launch_frame_verify(fmt, g, v, rb, layer_base, status_out, stream));
}

int hkv_frame_delta_m(const hkv_shape* shape, int32_t fmt, const hkv_records* frames,
                      const int32_t* m_new, int32_t* delta_out, hipStream_t stream) {
  Geometry g;
  RecordView v;
  int64_t rb;
  int st;
  if ((st = check_frames(shape, fmt, frames, &g, &v, &rb)) != HKV_OK) return st;
  if (g.n_layers == 0 || g.n_blocks == 0) return HKV_OK;
  if (!m_new || !delta_out) return HKV_ERR_INVALID_ARG;
  return to_status(hkv::launch_frame_delta(g, v, m_new, delta_out, stream));
}

int hkv_token_drift(const void* h_cached, const void* h_fresh, int32_t n_tokens,
                    int32_t d_model, int64_t row_stride, int32_t dtype, float* drift_out,
                    hipStream_t stream) {
  const int es = elem_size(dtype);
  if (es == 0 || n_tokens < 0 || d_model < 0 || row_stride < 0) return HKV_ERR_INVALID_ARG;
  if (n_tokens == 0) return HKV_OK;
  if (!drift_out || ((!h_cached || !h_fresh) && d_model > 0)) return HKV_ERR_INVALID_ARG;
  if (!aligned16(h_cached) || !aligned16(h_fresh)) return HKV_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(drift_out) & 3u) != 0) return HKV_ERR_INVALID_ARG;
  if (row_stride > INT64_MAX / 8 || (row_stride * es) % 16 != 0) return HKV_ERR_INVALID_ARG;
  if (n_tokens > 1 && row_stride < d_model) return HKV_ERR_INVALID_ARG;
  if (!span_ok({{n_tokens, row_stride * es}}, int64_t{d_model} * es)) return HKV_ERR_INVALID_ARG;
  return to_status(hkv::launch_drift(dtype, h_cached, h_fresh, n_tokens, d_model,
                                     row_stride * es, drift_out, stream));
}

int hkv_stream_probe(const void* src, void* dst, int64_t bytes_read, hipStream_t stream) {
  if (bytes_read < 0 || bytes_read % 128 != 0) return HKV_ERR_INVALID_ARG;
  if (bytes_read == 0) return HKV_OK;
  if (!src || !dst || !aligned16(src) || !aligned16(dst)) return HKV_ERR_INVALID_ARG;
  return to_status(hkv::launch_stream_expand(src, dst, bytes_read / 16, stream));
}

int hkv_stream_probe_put(const void* src, void* dst, int64_t bytes_written, hipStream_t stream) {
  if (bytes_written < 0 || bytes_written % 128 != 0) return HKV_ERR_INVALID_ARG;
  if (bytes_written / 128 > INT32_MAX / 8) return HKV_ERR_UNSUPPORTED;   // grid of rows * 8 threads
  if (bytes_written == 0) return HKV_OK;
  if (!src || !dst || !aligned16(src) || !aligned16(dst)) return HKV_ERR_INVALID_ARG;
  return to_status(hkv::launch_stream_squeeze(src, dst, bytes_written / 128, stream));
}

int64_t hkv_select_workspace_bytes(int32_t n_tokens) {
  if (n_tokens < 0 || n_tokens > kMaxSelectTokens) return -1;
  return hkv::select_workspace_bytes(n_tokens);
}

int hkv_select_top_tokens(const float* drift, int32_t n_tokens, int32_t k,
                          int32_t* selected_out, void* workspace, int64_t workspace_bytes,
                          hipStream_t stream) {
  if (n_tokens < 0 || k < 0 || k > n_tokens) return HKV_ERR_INVALID_ARG;
  if (n_tokens > kMaxSelectTokens) return HKV_ERR_UNSUPPORTED;
  if (workspace && (!aligned16(workspace) ||
                    workspace_bytes < hkv::select_workspace_bytes(n_tokens)))
    return HKV_ERR_INVALID_ARG;
  if (k == 0) return HKV_OK;
  if (!drift || !selected_out) return HKV_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(drift) & 3u) != 0 ||
      (reinterpret_cast<uintptr_t>(selected_out) & 3u) != 0)
    return HKV_ERR_INVALID_ARG;
  return to_status(hkv::launch_topk(drift, n_tokens, k, selected_out, workspace, stream));
}

}  // extern "C"
