// Layer-wise staged fetch: records held in host memory are brought into two
// device staging buffers one layer at a time and fetched from there.
//
// The HyperCache post ("HyperCache – Distributed KV-cache quantization and
// relative RoPE reuse"), Core Design, layer-wise transfer paragraph: while
// the GPU computes the suffix tokens of layer l, layer l+1 is already being
// brought into a staging buffer, so the transfer hides behind compute.  Here
// the transfer is a DMA copy from pinned host memory (the stand-in for the
// wire or disk tier) on `copy_stream`; the fetch kernel of each layer runs on
// `fetch_stream` once its copy has landed, and the caller's compute for layer
// l waits on the event recorded after that layer's fetch.
//
// Buffer discipline (two buffers, layer l in buffer l mod 2):
//   copy_stream:  wait(freed[l mod 2]); copy layer l; record(copied[l mod 2])
//   fetch_stream: wait(copied[l mod 2]); fetch layer l; record(freed[l mod 2]);
//                 record(layer_ready[l])
// A stream waits on the most recent record of an event made before the wait
// is enqueued, so the copy of layer l + 2 cannot start before the fetch of
// layer l has read the buffer, and the fetch of layer l cannot start before
// its own copy.  Both freed events are first recorded on fetch_stream, so the
// first two copies also wait for fetch-stream work enqueued before the call
// (a previous call's fetches may still be reading the buffers).
#include "hkv.h"

#include <stdint.h>

#include "hkv_launch.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Events {
  hipEvent_t e[4] = {nullptr, nullptr, nullptr, nullptr};   // copied[0..1], freed[0..1]
  ~Events() {
    // Destroying an event whose record has not completed is allowed: its
    // resources are released once it completes.
    for (hipEvent_t x : e)
      if (x) (void)hipEventDestroy(x);
  }
};

}  // namespace

extern "C" int hkv_fetch_staged(const hkv_shape* shape, int32_t fmt, const hkv_host_records* src,
                                void* staging0, void* staging1, int64_t staging_bytes,
                                const int32_t* block_table, const int32_t* delta_m,
                                const int32_t* visit_order, double rope_base, int32_t pairs,
                                const hkv_pages* dst, int32_t dst_dtype, hipStream_t copy_stream,
                                hipStream_t fetch_stream, hipEvent_t* layer_ready) {
  if (!shape || !src || !src->host_base || !staging0 || !staging1 || staging0 == staging1)
    return HKV_ERR_INVALID_ARG;
  if (!aligned16(src->host_base) || !aligned16(staging0) || !aligned16(staging1))
    return HKV_ERR_INVALID_ARG;
  if (src->layer_stride_bytes < 0 || src->block_stride_bytes < 0 ||
      src->layer_stride_bytes % 16 != 0 || src->block_stride_bytes % 16 != 0)
    return HKV_ERR_INVALID_ARG;
  const int64_t rb = hkv_record_bytes(fmt, shape->block_tokens, shape->n_kv_heads,
                                      shape->head_dim);
  if (rb < 0 || shape->n_layers < 0 || shape->n_blocks < 0) return HKV_ERR_INVALID_ARG;
  // one layer of records as the fetch reads it from a staging buffer
  const hkv_shape one = {1, shape->n_blocks, shape->block_tokens, shape->n_kv_heads,
                         shape->head_dim};
  const hkv_records stage_view = {staging0, 0, src->block_stride_bytes};
  hkv::FetchViews f;
  int st = hkv::fetch_check(&one, fmt, &stage_view, block_table, delta_m, rope_base, pairs, dst,
                            dst_dtype, &f);
  if (st != HKV_OK) return st;
  if (shape->n_layers > 65535) return HKV_ERR_UNSUPPORTED;
  // the pages of every layer and the host records of every layer (the
  // check above saw one layer)
  const int64_t vec_bytes = int64_t{HKV_HEAD_DIM} * (dst_dtype == HKV_F32 ? 4 : 2);
  if (!hkv::span_ok({{shape->n_layers, f.pv.layer}, {dst->num_pages, f.pv.page},
                     {shape->block_tokens, f.pv.token}, {shape->n_kv_heads, f.pv.head}},
                    vec_bytes) ||
      !hkv::span_ok({{shape->n_layers, src->layer_stride_bytes},
                     {shape->n_blocks, src->block_stride_bytes}},
                    rb))
    return HKV_ERR_INVALID_ARG;
  if (shape->n_layers == 0 || shape->n_blocks == 0) return HKV_OK;
  const int64_t extent = (static_cast<int64_t>(shape->n_blocks) - 1) * src->block_stride_bytes + rb;
  if (staging_bytes < extent) return HKV_ERR_INVALID_ARG;
  if (shape->n_layers > 1 && src->layer_stride_bytes < extent) return HKV_ERR_INVALID_ARG;

  Events ev;
  for (hipEvent_t& e : ev.e)
    if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) {
      e = nullptr;
      (void)hipGetLastError();
      return HKV_ERR_HIP;
    }
  hipEvent_t* copied = ev.e;
  hipEvent_t* freed = ev.e + 2;
  void* const staging[2] = {staging0, staging1};
  const char* host = static_cast<const char*>(src->host_base);
  if (hipEventRecord(freed[0], fetch_stream) != hipSuccess ||
      hipEventRecord(freed[1], fetch_stream) != hipSuccess)
    return HKV_ERR_HIP;
  for (int32_t l = 0; l < shape->n_layers; ++l) {
    const int b = l & 1;
    if (hipStreamWaitEvent(copy_stream, freed[b], 0) != hipSuccess) return HKV_ERR_HIP;
    if (hipMemcpyAsync(staging[b], host + l * src->layer_stride_bytes, static_cast<size_t>(extent),
                       hipMemcpyHostToDevice, copy_stream) != hipSuccess)
      return HKV_ERR_HIP;
    if (hipEventRecord(copied[b], copy_stream) != hipSuccess) return HKV_ERR_HIP;
    if (hipStreamWaitEvent(fetch_stream, copied[b], 0) != hipSuccess) return HKV_ERR_HIP;
    hkv::RecordView rv = {static_cast<uint8_t*>(staging[b]), 0, src->block_stride_bytes};
    hkv::PageView pv = f.pv;
    pv.k += l * pv.layer;
    pv.v += l * pv.layer;
    if (hkv::launch_fetch(fmt, dst_dtype, pairs, f.g, rv, block_table, delta_m, false, visit_order,
                          rope_base, pv, fetch_stream) != hipSuccess)
      return HKV_ERR_HIP;
    if (hipEventRecord(freed[b], fetch_stream) != hipSuccess) return HKV_ERR_HIP;
    if (layer_ready && layer_ready[l] && hipEventRecord(layer_ready[l], fetch_stream) != hipSuccess)
      return HKV_ERR_HIP;
  }
  return HKV_OK;
}
