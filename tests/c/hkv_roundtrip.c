/* A plain C client of libhkv: device buffers from hipMalloc, one stream from
 * hipStreamCreate, no torch.  It shows that the C ABI in include/hkv.h is all a
 * caller needs, and lets a GPU test check this path against the CPU oracle.
 *
 *   hkv_roundtrip DIR
 *
 * DIR holds the inputs, written by the test:
 *   params.txt      n_layers n_blocks block_tokens n_kv_heads num_pages
 *                   src_dtype fmt pairs dst_dtype rope_base
 *                   (dtypes and enums as in hkv.h)
 *   k_src.bin, v_src.bin   source pages [L][num_pages][T][H][128], src_dtype
 *   put_table.bin, fetch_table.bin, delta.bin   int32 [n_blocks]
 * and receives the outputs:
 *   records.bin        hkv_quant_fp8 / hkv_quant_int4, [L][n_blocks][record bytes]
 *   crc.bin            hkv_crc32_blocks over those records, uint32 [L][n_blocks]
 *   records_fused.bin, crc_fused.bin   hkv_quant_*_crc (put and CRC in one pass)
 *   k_out.bin, v_out.bin   hkv_fetch_dequant_rope_shift of records.bin into
 *                   pages [L][num_pages][T][H][128] of dst_dtype
 * Record buffers start as 0xA5 bytes and output pages as 0xEE bytes, so the
 * test can see what the calls left untouched.  Exit status: 0 on success, 2
 * for bad usage or files, 3 for a HIP error, 4 for a libhkv error status, 5
 * when an argument check did not reject a bad request. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "hkv.h"

#define CHECK_HIP(call)                                                     \
  do {                                                                      \
    hipError_t e_ = (call);                                                 \
    if (e_ != hipSuccess) {                                                 \
      fprintf(stderr, "%s: %s\n", #call, hipGetErrorString(e_));            \
      exit(3);                                                              \
    }                                                                       \
  } while (0)

#define CHECK_HKV(call)                                                     \
  do {                                                                      \
    int s_ = (call);                                                        \
    if (s_ != HKV_OK) {                                                     \
      fprintf(stderr, "%s: %s (%d)\n", #call, hkv_status_string(s_), s_);   \
      exit(4);                                                              \
    }                                                                       \
  } while (0)

static char path_buf[4096];

static const char* path_of(const char* dir, const char* name) {
  snprintf(path_buf, sizeof path_buf, "%s/%s", dir, name);
  return path_buf;
}

static void* read_exact(const char* dir, const char* name, size_t bytes) {
  FILE* f = fopen(path_of(dir, name), "rb");
  if (!f) {
    fprintf(stderr, "cannot open %s\n", path_buf);
    exit(2);
  }
  void* p = malloc(bytes ? bytes : 1);
  if (!p || fread(p, 1, bytes, f) != bytes || fgetc(f) != EOF) {
    fprintf(stderr, "%s does not hold exactly %zu bytes\n", path_buf, bytes);
    exit(2);
  }
  fclose(f);
  return p;
}

static void write_all(const char* dir, const char* name, const void* p, size_t bytes) {
  FILE* f = fopen(path_of(dir, name), "wb");
  if (!f || fwrite(p, 1, bytes, f) != bytes || fclose(f) != 0) {
    fprintf(stderr, "cannot write %s\n", path_buf);
    exit(2);
  }
}

static void* device_copy(const void* host, size_t bytes) {
  void* d = NULL;
  CHECK_HIP(hipMalloc(&d, bytes ? bytes : 16));
  if (bytes) CHECK_HIP(hipMemcpy(d, host, bytes, hipMemcpyHostToDevice));
  return d;
}

static void* device_filled(size_t bytes, int byte) {
  void* d = NULL;
  CHECK_HIP(hipMalloc(&d, bytes ? bytes : 16));
  CHECK_HIP(hipMemset(d, byte, bytes ? bytes : 16));
  return d;
}

/* Records (l, b) at l * n_blocks * stride + b * stride, copied back densely. */
static void save_records(const char* dir, const char* name, const void* dev, int32_t n_layers,
                         int32_t n_blocks, int64_t stride, int64_t record_bytes) {
  const size_t total = (size_t)n_layers * (size_t)n_blocks * (size_t)stride;
  uint8_t* host = (uint8_t*)malloc(total ? total : 1);
  uint8_t* dense = (uint8_t*)malloc(total ? total : 1);
  if (!host || !dense) exit(2);
  if (total) CHECK_HIP(hipMemcpy(host, dev, total, hipMemcpyDeviceToHost));
  for (size_t r = 0; r < (size_t)n_layers * (size_t)n_blocks; ++r)
    memcpy(dense + r * (size_t)record_bytes, host + r * (size_t)stride, (size_t)record_bytes);
  write_all(dir, name, dense, (size_t)n_layers * (size_t)n_blocks * (size_t)record_bytes);
  free(host);
  free(dense);
}

static void save_device(const char* dir, const char* name, const void* dev, size_t bytes) {
  void* host = malloc(bytes ? bytes : 1);
  if (!host) exit(2);
  if (bytes) CHECK_HIP(hipMemcpy(host, dev, bytes, hipMemcpyDeviceToHost));
  write_all(dir, name, host, bytes);
  free(host);
}

static int64_t elem_size(int32_t dtype) { return dtype == HKV_F32 ? 4 : 2; }

int main(int argc, char** argv) {
  if (argc != 2) {
    fprintf(stderr, "usage: %s DIR\n", argv[0]);
    return 2;
  }
  const char* dir = argv[1];
  int32_t L, nb, tb, H, P, src_dtype, fmt, pairs, dst_dtype;
  double rope_base;
  FILE* pf = fopen(path_of(dir, "params.txt"), "r");
  if (!pf || fscanf(pf, "%d %d %d %d %d %d %d %d %d %lf", &L, &nb, &tb, &H, &P, &src_dtype,
                    &fmt, &pairs, &dst_dtype, &rope_base) != 10) {
    fprintf(stderr, "cannot read %s\n", path_buf);
    return 2;
  }
  fclose(pf);

  const hkv_shape shape = {L, nb, tb, H, HKV_HEAD_DIM};
  const int64_t rb = hkv_record_bytes(fmt, tb, H, HKV_HEAD_DIM);
  if (rb <= 0) {
    fprintf(stderr, "hkv_record_bytes rejected the shape\n");
    return 2;
  }
  const int64_t stride = (rb + 15) / 16 * 16;
  const int64_t head = HKV_HEAD_DIM, token = (int64_t)H * head, page = (int64_t)tb * token;
  const int64_t layer = (int64_t)P * page;
  const size_t src_bytes = (size_t)(L * layer * elem_size(src_dtype));
  const size_t dst_bytes = (size_t)(L * layer * elem_size(dst_dtype));
  const size_t tab_bytes = (size_t)nb * sizeof(int32_t);
  const size_t rec_bytes = (size_t)L * (size_t)nb * (size_t)stride;
  const size_t crc_bytes = (size_t)L * (size_t)nb * sizeof(uint32_t);

  void* h_k = read_exact(dir, "k_src.bin", src_bytes);
  void* h_v = read_exact(dir, "v_src.bin", src_bytes);
  void* h_put = read_exact(dir, "put_table.bin", tab_bytes);
  void* h_fetch = read_exact(dir, "fetch_table.bin", tab_bytes);
  void* h_delta = read_exact(dir, "delta.bin", tab_bytes);

  hipStream_t stream;
  CHECK_HIP(hipStreamCreate(&stream));
  void* d_k = device_copy(h_k, src_bytes);
  void* d_v = device_copy(h_v, src_bytes);
  int32_t* d_put = (int32_t*)device_copy(h_put, tab_bytes);
  int32_t* d_fetch = (int32_t*)device_copy(h_fetch, tab_bytes);
  int32_t* d_delta = (int32_t*)device_copy(h_delta, tab_bytes);
  void* d_rec = device_filled(rec_bytes, 0xA5);
  void* d_rec2 = device_filled(rec_bytes, 0xA5);
  uint32_t* d_crc = (uint32_t*)device_filled(crc_bytes, 0);
  uint32_t* d_crc2 = (uint32_t*)device_filled(crc_bytes, 0);
  void* d_ko = device_filled(dst_bytes, 0xEE);
  void* d_vo = device_filled(dst_bytes, 0xEE);

  const hkv_pages src = {d_k, d_v, layer, page, token, head, P};
  const hkv_pages dst = {d_ko, d_vo, layer, page, token, head, P};
  const hkv_records rec = {d_rec, (int64_t)nb * stride, stride};
  const hkv_records rec2 = {d_rec2, (int64_t)nb * stride, stride};

  /* Argument checks run on the host and launch nothing. */
  const hkv_shape bad = {L, nb, tb, H, 64};
  if (hkv_fetch_dequant_rope_shift(&bad, fmt, &rec, d_fetch, d_delta, NULL, rope_base, pairs,
                                   &dst, dst_dtype, stream) != HKV_ERR_INVALID_ARG ||
      hkv_fetch_dequant_rope_shift(&shape, fmt, &rec, d_fetch, d_delta, NULL, -1.0, pairs, &dst,
                                   dst_dtype, stream) != HKV_ERR_INVALID_ARG) {
    fprintf(stderr, "a bad fetch request was not rejected\n");
    return 5;
  }

  /* Put, then the CRC of the records, then the fetch of those records. */
  if (fmt == HKV_FP8_E4M3)
    CHECK_HKV(hkv_quant_fp8(&shape, &src, src_dtype, d_put, &rec, stream));
  else
    CHECK_HKV(hkv_quant_int4(&shape, &src, src_dtype, d_put, &rec, stream));
  CHECK_HKV(hkv_crc32_blocks(&shape, fmt, &rec, d_crc, stream));
  CHECK_HKV(hkv_fetch_dequant_rope_shift(&shape, fmt, &rec, d_fetch, d_delta, NULL, rope_base,
                                         pairs, &dst, dst_dtype, stream));

  /* The same put with its CRC in one pass, into a second record buffer. */
  const int64_t ws_bytes = hkv_quant_crc_workspace_bytes(&shape, fmt);
  if (ws_bytes < 0) {
    fprintf(stderr, "hkv_quant_crc_workspace_bytes rejected the shape\n");
    return 4;
  }
  void* d_ws = device_filled((size_t)ws_bytes, 0x5A);
  hipEvent_t records_ready;
  CHECK_HIP(hipEventCreateWithFlags(&records_ready, hipEventDisableTiming));
  if (fmt == HKV_FP8_E4M3)
    CHECK_HKV(hkv_quant_fp8_crc(&shape, &src, src_dtype, d_put, &rec2, d_crc2, d_ws, ws_bytes,
                                stream, records_ready));
  else
    CHECK_HKV(hkv_quant_int4_crc(&shape, &src, src_dtype, d_put, &rec2, d_crc2, d_ws, ws_bytes,
                                 stream, records_ready));
  CHECK_HIP(hipStreamSynchronize(stream));
  /* recorded by the call, so complete once the stream is */
  CHECK_HIP(hipEventQuery(records_ready));
  CHECK_HIP(hipEventDestroy(records_ready));

  save_records(dir, "records.bin", d_rec, L, nb, stride, rb);
  save_records(dir, "records_fused.bin", d_rec2, L, nb, stride, rb);
  save_device(dir, "crc.bin", d_crc, crc_bytes);
  save_device(dir, "crc_fused.bin", d_crc2, crc_bytes);
  save_device(dir, "k_out.bin", d_ko, dst_bytes);
  save_device(dir, "v_out.bin", d_vo, dst_bytes);

  void* bufs[] = {d_k, d_v, d_put, d_fetch, d_delta, d_rec, d_rec2, d_crc, d_crc2, d_ko, d_vo, d_ws};
  for (size_t i = 0; i < sizeof bufs / sizeof bufs[0]; ++i) CHECK_HIP(hipFree(bufs[i]));
  CHECK_HIP(hipStreamDestroy(stream));
  free(h_k);
  free(h_v);
  free(h_put);
  free(h_fetch);
  free(h_delta);
  printf("hkv_roundtrip: %d layers x %d blocks x %d tokens x %d heads done\n", L, nb, tb, H);
  return 0;
}
