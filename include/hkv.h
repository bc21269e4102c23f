/*
 * hkv.h - C ABI of libhkv, a KV-cache block codec for AMD MI355X (gfx950).
 *
 * libhkv moves cached key/value blocks of a transformer into and out of a
 * compressed record form and re-uses them at a new token position:
 *
 *   put    quantize post-RoPE K and V head vectors of 128 elements to FP8
 *          E4M3 or to INT4, one fp16 scale per vector (hkv_quant_fp8,
 *          hkv_quant_int4);
 *   check  CRC-32 of each record (hkv_crc32_blocks; fused with the put:
 *          hkv_quant_fp8_crc, hkv_quant_int4_crc);
 *   fetch  dequantize, rotate every key pair by the block's position delta
 *          dm = m_new - m_old, leave values unrotated, and scatter into a
 *          paged KV buffer through a block table
 *          (hkv_fetch_dequant_rope_shift; one delta per token:
 *          hkv_fetch_dequant_rope_shift_tokens; a destination-ordered visit
 *          list: hkv_page_visit_order; layer by layer from host memory
 *          through two staging buffers: hkv_fetch_staged);
 *   frame  a self-describing header in front of each record, its
 *          verification, and dm from the stored position (hkv_frame_*);
 *   select the tokens to recompute after a chunk reorder: per-token drift
 *          of the layer-0 hidden state and the top k (hkv_token_drift,
 *          hkv_select_top_tokens);
 *   overlap two compute-unit-partitioned streams for a fetch running beside
 *          compute (hkv_stream_pair_create).
 *
 * The operations follow two web pages:
 *   "HyperCache – Distributed KV-cache quantization and relative RoPE reuse"
 *   (the HyperCache post): Core Design, relative-RoPE paragraph with the SO(2)
 *   identity R(m_new th_i) = R(dm th_i) R(m_old th_i); the compression
 *   paragraph and the Part B benchmark printout (FP8 E4M3 wire records,
 *   INT4 grouped disk records with CRC32).
 *   "Модуль 13: KV-хэндофф: передача кеша между моделями и узлами" of the
 *   LLM Inference Systems course (the KV-handoff module): the module13.py
 *   listing's rope_cache / apply_rope, which fix th_i = 1 / base^(2i/d) and the rotation
 *   (a, b) -> (a cos - b sin, a sin + b cos).
 *
 * Conventions for every call
 * --------------------------
 * - All array pointers are DEVICE pointers owned by the caller; the structs
 *   themselves are read from host memory during the call only.
 * - Calls are asynchronous on `stream` (0 = the default stream), allocate
 *   no memory (hkv_stream_pair_create aside, which creates two streams;
 *   hkv_fetch_staged creates four events for the duration of the call),
 *   keep no state between calls and may be called from several host
 *   threads at once; hkv_quant_fp8_crc_noalloc is the one exception to the
 *   last two: it works in a scratch array the library keeps per GPU.
 * - Return value: HKV_OK (0) or a negative hkv_status.  Argument errors are
 *   detected on the host before anything is launched; nothing throws across
 *   the ABI.  A launch failure is reported as HKV_ERR_HIP.
 * - head_dim must be 128 (the group of one scale).
 * - Zero layers or zero blocks is a valid empty call that launches nothing.
 * - Every view (pages, records, frames, hidden-state rows) must address no
 *   byte offset at or beyond 2^47 from its base, counting (count - 1) *
 *   stride over each of its dimensions plus the last element: more than a
 *   device can address, refused with HKV_ERR_INVALID_ARG.
 * - Block tables are int32 [n_blocks]: logical block -> page.  A negative
 *   entry means "skip this block"; an entry >= num_pages is skipped as well
 *   (it is never dereferenced).  The tables given to one call must not map
 *   two blocks to the same page (the writes would race).
 */
#ifndef HKV_H
#define HKV_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HKV_OK = 0,
  HKV_ERR_INVALID_ARG = -1,  /* null pointer, bad size, misalignment, bad enum */
  HKV_ERR_UNSUPPORTED = -2,  /* a well-formed request the library does not do */
  HKV_ERR_HIP = -3           /* the HIP runtime reported a launch error        */
} hkv_status;

typedef enum { HKV_F32 = 0, HKV_F16 = 1, HKV_BF16 = 2 } hkv_dtype;
typedef enum { HKV_FP8_E4M3 = 0, HKV_INT4 = 1 } hkv_format;
typedef enum { HKV_ROPE_INTERLEAVED = 0, HKV_ROPE_HALF_SPLIT = 1 } hkv_rope_pairs;

#define HKV_HEAD_DIM 128

/* Geometry shared by all calls.  A "vector" is one (layer, K|V, token, head)
 * row of head_dim elements.  Calls return HKV_ERR_UNSUPPORTED for shapes
 * beyond the launch grids: n_layers > 65535, block_tokens * n_kv_heads >
 * 2^24, n_layers * n_blocks > 2^31 - 1, or n_blocks * 2 *
 * ceil(block_tokens * n_kv_heads / 16) > 2^31 - 1. */
typedef struct {
  int32_t n_layers;      /* >= 0 */
  int32_t n_blocks;      /* >= 0, logical blocks per layer */
  int32_t block_tokens;  /* >= 1, tokens per block (= tokens per page) */
  int32_t n_kv_heads;    /* >= 1 */
  int32_t head_dim;      /* must be 128 */
} hkv_shape;

/* An engine's paged KV buffer: separate K and V arrays of one dtype.
 * Element (layer l, page p, token t, head h, dim j) of K is at
 *   k + l*layer_stride + p*page_stride + t*token_stride + h*head_stride + j
 * (strides in ELEMENTS, non-negative; the head_dim elements of a vector are
 * contiguous).  k, v and every stride times the element size must be
 * multiples of 16 bytes. */
typedef struct {
  void* k;
  void* v;
  int64_t layer_stride;
  int64_t page_stride;
  int64_t token_stride;
  int64_t head_stride;
  int32_t num_pages;     /* pages per layer; table entries >= this are skipped */
} hkv_pages;

/* Compressed records, one per (layer, logical block), record (l, b) at
 *   base + l*layer_stride_bytes + b*block_stride_bytes.
 * Record layout (N = block_tokens * n_kv_heads vectors, C = 128 code bytes
 * for FP8 or 64 for INT4):
 *   [K codes N*C][V codes N*C][K scales N*2][V scales N*2]
 * codes ordered token-major, then head, then element; scales are IEEE fp16,
 * little endian, in the same vector order.  INT4 packs element 2k in the
 * low nibble and 2k+1 in the high nibble of byte k, two's complement.
 * base and both strides must be multiples of 16 bytes and the block stride
 * at least hkv_record_bytes(). */
typedef struct {
  void* base;
  int64_t layer_stride_bytes;
  int64_t block_stride_bytes;
} hkv_records;

/* Put, FP8 (HyperCache post: compression paragraph; Part B, the FP8 E4M3
 * wire line, 1.97x against fp16).
 * For every vector x of logical block b (read from page block_table[b] of
 * `src`, dtype src_dtype):
 *   amax = max_j |x_j|                       (exact, fp32)
 *   s    = fp16_RNE(amax / 448)              (IEEE fp32 division)
 *          with s = 2^-24 if that rounds to 0 while amax > 0, and
 *          s = 65504 if it exceeds the fp16 range; s = 0 if amax = 0
 *   c_j  = E4M3FN_RNE(x_j / s), saturating at +-448, sign of zero kept
 *          (x_j itself, a signed zero, when s = 0)
 * and writes codes and s to record (l, b) of `dst`.  Records of skipped
 * blocks are not written. */
int hkv_quant_fp8(const hkv_shape* shape, const hkv_pages* src, int32_t src_dtype,
                  const int32_t* block_table, const hkv_records* dst,
                  hipStream_t stream);

/* Put, INT4 grouped symmetric (HyperCache post: Part B, the grouped INT4
 * L3-disk line, 3.88x against fp16).  As hkv_quant_fp8 with
 *   s   = fp16_RNE(amax / 7) (same edge cases),
 *   q_j = clamp(round_half_even(x_j / s), -7, 7). */
int hkv_quant_int4(const hkv_shape* shape, const hkv_pages* src, int32_t src_dtype,
                   const int32_t* block_table, const hkv_records* dst,
                   hipStream_t stream);

/* Put and CRC in one pass (HyperCache post: Part B, the L3-disk line: INT4
 * records written with their CRC32).  Writes the same records as
 * hkv_quant_fp8 / hkv_quant_int4 and to crc_out (uint32 [n_layers *
 * n_blocks], device, layer-major) the CRC-32 of every record the put wrote,
 * equal to what hkv_crc32_blocks computes over them.  Entries of skipped
 * blocks are left unchanged (on both paths below).  The put kernel
 * stages each workgroup's codes in LDS and stores the raw CRC of every
 * 128-byte unit of the record's codes to `workspace`; a second kernel reads
 * each record's scales back and merges both into the record's CRC.  The
 * workspace's contents on entry do not matter and are left undefined.
 * workspace: 16-byte aligned device memory of at least
 * hkv_quant_crc_workspace_bytes() bytes (4 bytes per 128 bytes of records);
 * when block_tokens * n_kv_heads is not a multiple of 64 that is 0, no
 * workspace is needed and the call runs the put and then the CRC kernel.
 * records_ready: NULL, or an event (created by the caller) that the call
 * records on `stream` once the put has written the records and before the
 * CRC work that follows it: work that needs only the records (a fetch on
 * another stream) can wait on it instead of on the whole call, so the
 * merge of the CRCs overlaps it.  The CRCs are complete when `stream`
 * reaches the end of the call.  An event with timing enabled times the put
 * phase. */
int hkv_quant_fp8_crc(const hkv_shape* shape, const hkv_pages* src, int32_t src_dtype,
                      const int32_t* block_table, const hkv_records* dst, uint32_t* crc_out,
                      void* workspace, int64_t workspace_bytes, hipStream_t stream,
                      hipEvent_t records_ready);
int hkv_quant_int4_crc(const hkv_shape* shape, const hkv_pages* src, int32_t src_dtype,
                       const int32_t* block_table, const hkv_records* dst, uint32_t* crc_out,
                       void* workspace, int64_t workspace_bytes, hipStream_t stream,
                       hipEvent_t records_ready);

/* Workspace bytes for hkv_quant_*_crc with this shape and format; -1 on bad
 * arguments. */
int64_t hkv_quant_crc_workspace_bytes(const hkv_shape* shape, int32_t fmt);

/* hkv_quant_fp8_crc for callers that cannot allocate device memory (code
 * under HIP graph capture, serving loops that never call the allocator,
 * harnesses that forbid it).  Same arguments, records and CRCs as
 * hkv_quant_fp8_crc, without the workspace (and records no records_ready
 * event): the call uses a scratch array
 * of HKV_NOALLOC_SCRATCH_BYTES that the library holds in device memory, one
 * per GPU it runs on, for the life of the process, and calls no allocator.
 * A shape whose hkv_quant_crc_workspace_bytes(shape, HKV_FP8_E4M3) exceeds
 * HKV_NOALLOC_SCRATCH_BYTES (about 1 GiB of records; one Llama-3-70B-shaped
 * layer needs 4.3 MB) returns HKV_ERR_UNSUPPORTED before anything runs:
 * split it into several calls.  The scratch belongs to the device of
 * `stream`; its contents between calls do not matter.  All calls on one GPU
 * share that GPU's scratch, so calls that overlap in time on one GPU (on
 * different streams, or from several host threads without ordering) race
 * and must not be made. */
#define HKV_NOALLOC_SCRATCH_BYTES (32LL * 1024 * 1024)
int hkv_quant_fp8_crc_noalloc(const hkv_shape* shape, const hkv_pages* src, int32_t src_dtype,
                              const int32_t* block_table, const hkv_records* dst,
                              uint32_t* crc_out, hipStream_t stream);

/* Fetch (HyperCache post: Core Design, relative-RoPE paragraph; Part B, the
 * socket-fetch line with RoPE applied on the fly).
 * For every layer l and logical block b with 0 <= block_table[b] < num_pages:
 *   y = code * s                                      (exact in fp32)
 *   V: y unchanged.
 *   K: each pair i = 0..63 - elements (2i, 2i+1) for HKV_ROPE_INTERLEAVED,
 *      (i, i+64) for HKV_ROPE_HALF_SPLIT - is rotated by
 *      phi = delta_m[b] * th_i, th_i = 1 / rope_base^(2i/128):
 *        (a, b) -> (a cos phi - b sin phi, a sin phi + b cos phi),
 *      with phi, cos and sin evaluated in double precision (full range
 *      reduction) and rounded to fp32 once per (block, i); a block with
 *      delta_m[b] = 0 is passed through unrotated.
 *   The result is rounded to nearest even to dst_dtype and stored at page
 *   block_table[b] of `dst`, token t, head h.
 * delta_m: int32 [n_blocks] device array, any sign.
 * visit_order: NULL, or an int32 [n_blocks] device array holding a
 *   permutation of 0..n_blocks-1: the order in which blocks are processed.
 *   The result does not depend on it.  Listing blocks by increasing
 *   destination page (hkv_page_visit_order) keeps concurrent writes close
 *   together in HBM; entries outside [0, n_blocks) are skipped.
 * rope_base: finite and > 0. */
int hkv_fetch_dequant_rope_shift(const hkv_shape* shape, int32_t fmt,
                                 const hkv_records* src, const int32_t* block_table,
                                 const int32_t* delta_m, const int32_t* visit_order,
                                 double rope_base, int32_t pairs, const hkv_pages* dst,
                                 int32_t dst_dtype, hipStream_t stream);

/* Fetch with one delta per token: as hkv_fetch_dequant_rope_shift, but
 * delta_m_tokens is an int32 [n_blocks][block_tokens] device array and each
 * key vector is rotated by its own token's delta (for example -m to strip
 * the cached positions' phase, as the KV-handoff module's strip_rope does,
 * or a per-token re-layout).  phi = delta * theta_i and its reduction
 * modulo pi/2 are computed in double (accurate for |phi| < 2^31); cos and sin
 * of the reduced argument in fp32.  The tolerance is the same as for the
 * per-block fetch. */
int hkv_fetch_dequant_rope_shift_tokens(const hkv_shape* shape, int32_t fmt,
                                        const hkv_records* src, const int32_t* block_table,
                                        const int32_t* delta_m_tokens,
                                        const int32_t* visit_order, double rope_base,
                                        int32_t pairs, const hkv_pages* dst, int32_t dst_dtype,
                                        hipStream_t stream);

/* Records in host memory, one per (layer, logical block): record (l, b) at
 *   host_base + l*layer_stride_bytes + b*block_stride_bytes
 * (layout as hkv_records).  host_base and both strides: multiples of 16. */
typedef struct {
  const void* host_base;
  int64_t layer_stride_bytes;
  int64_t block_stride_bytes;
} hkv_host_records;

/* Layer-wise staged fetch (HyperCache post, Core Design, layer-wise transfer
 * paragraph: layer l+1 is brought into a staging buffer while the GPU
 * computes the suffix tokens of layer l).  For l = 0 .. n_layers-1: copies
 * layer l's records, the bytes [0, (n_blocks-1)*block_stride_bytes +
 * hkv_record_bytes()) of the layer, from host memory into staging buffer
 * l mod 2 on copy_stream (DMA), then runs hkv_fetch_dequant_rope_shift on
 * that one layer on fetch_stream into layer l of `dst`, with the same
 * table, deltas, visit order, base and pairs for every layer.  A layer's
 * fetch waits for its copy; a buffer is refilled only after the fetch that
 * read it has run (and, for the first two copies, after the work enqueued on
 * fetch_stream before the call).  layer_ready: NULL, or n_layers events
 * created by the caller (NULL entries are skipped); event l is recorded on
 * fetch_stream after layer l's fetch, so a compute stream that waits on it
 * sees layer l's pages.  The call creates four events for its own use and
 * allocates no memory.
 * src: host memory the copies read until fetch_stream has passed the last
 * layer; pinned (hipHostMalloc) for the copies to run asynchronously.
 * staging0, staging1: distinct device buffers of staging_bytes >= one
 * layer's extent above, 16-byte aligned, not used by anything else until
 * fetch_stream has passed the last layer.  When that point of fetch_stream
 * completes, every copy and fetch of the call has completed.  copy_stream
 * and fetch_stream may be the same stream (no overlap then). */
int hkv_fetch_staged(const hkv_shape* shape, int32_t fmt, const hkv_host_records* src,
                     void* staging0, void* staging1, int64_t staging_bytes,
                     const int32_t* block_table, const int32_t* delta_m,
                     const int32_t* visit_order, double rope_base, int32_t pairs,
                     const hkv_pages* dst, int32_t dst_dtype, hipStream_t copy_stream,
                     hipStream_t fetch_stream, hipEvent_t* layer_ready);

/* Visiting order for hkv_fetch_dequant_rope_shift: writes to order_out
 * (int32 [n_blocks], device) the logical blocks sorted by destination page
 * block_table[b]; blocks whose entry is negative or >= num_pages come last,
 * in index order (ties, which the fetch contract excludes, by index).  This
 * is a scheduling aid, not a step of the method; O(n_blocks^2) work, meant
 * for tables of up to a few thousand blocks; n_blocks above 65,536 returns
 * HKV_ERR_UNSUPPORTED. */
int hkv_page_visit_order(const int32_t* block_table, int32_t n_blocks, int32_t num_pages,
                         int32_t* order_out, hipStream_t stream);

/* CRC-32 of every record (HyperCache post: Part B, the L3-disk line with its
 * per-file CRC32, and the tamper-detection tests of its test-suite section).  The common zlib variant:
 * reflected polynomial 0xEDB88320, initial value and final xor 0xFFFFFFFF,
 * over the hkv_record_bytes() bytes of each record.
 * crc_out: uint32 [n_layers * n_blocks] device array, layer-major. */
int hkv_crc32_blocks(const hkv_shape* shape, int32_t fmt, const hkv_records* src,
                     uint32_t* crc_out, hipStream_t stream);

/* Layer-wise overlap (HyperCache post, Core Design, layer-wise transfer
 * paragraph: layer l+1 is fetched while layer l computes).  Creates two
 * streams on the current device that split its compute units: the first
 * fetch_cus of them for *fetch_stream, all others for *compute_stream.  Kernels on the two streams then run side by side
 * instead of the fetch waiting for gaps in a compute kernel that holds every
 * CU.  Both streams have the default priority; release them with
 * hkv_stream_destroy.  HKV_ERR_INVALID_ARG unless 1 <= fetch_cus < CU count. */
int hkv_stream_pair_create(int32_t fetch_cus, hipStream_t* fetch_stream,
                           hipStream_t* compute_stream);
int hkv_stream_destroy(hipStream_t stream);

/* Self-describing frames (HyperCache post: Part B, the FP8 wire frame and
 * the INT4 disk file, both a header around the payload; the post prints
 * their sizes but not their layout, so the header is this library's own).
 * A frame is a 64-byte header followed by the record of one (layer, block);
 * `frames` describes the frames as hkv_records does records (the record of
 * frame (l, b) starts HKV_FRAME_HEADER_BYTES after it, so the same buffer
 * serves put, CRC and fetch through a records view at base + 64).  Each
 * frame must hold header + record: block and layer strides >= 64 +
 * hkv_record_bytes() (when there is more than one), multiples of 16.
 * block_tokens and n_kv_heads must fit 16 bits (else HKV_ERR_UNSUPPORTED).
 * Header, little endian:
 *    0 u32 magic 0x46564B48 ("HKVF")  4 u16 version 1  6 u16 header bytes 64
 *    8 u8 format (0 FP8, 1 INT4)  9 u8 0  10 u16 head_dim
 *   12 u16 block_tokens  14 u16 n_kv_heads  16 u32 layer  20 u32 block
 *   24 i32 m_old (cached position of the block's first token)
 *   28 u32 record bytes  32 u32 record CRC-32  36..59 zero
 *   60 u32 CRC-32 of bytes 0..59 (zlib variant, as hkv_crc32_blocks) */
#define HKV_FRAME_HEADER_BYTES 64

/* Flags written by hkv_frame_verify (0 = intact and in its place). */
#define HKV_FRAME_BAD_MAGIC 1u        /* magic, version or header size     */
#define HKV_FRAME_BAD_HEADER_CRC 2u   /* header bytes 0..59 vs their CRC   */
#define HKV_FRAME_BAD_GEOMETRY 4u     /* format, head_dim, block_tokens,
                                         n_kv_heads or record bytes differ
                                         from the call's                   */
#define HKV_FRAME_BAD_INDEX 8u        /* layer or block field is not the
                                         frame's slot                      */
#define HKV_FRAME_BAD_PAYLOAD_CRC 16u /* record bytes vs the stored CRC    */

/* Writes the header of every frame (l, b): layer = layer_base + l, block =
 * b, m_old[b] (int32 [n_blocks], device, shared by the layers), the record's
 * CRC crc[l * n_blocks + b] (uint32, device, as hkv_crc32_blocks writes it
 * for the records view).  Record bytes are not touched. */
int hkv_frame_headers(const hkv_shape* shape, int32_t fmt, const hkv_records* frames,
                      const uint32_t* crc, const int32_t* m_old, int32_t layer_base,
                      hipStream_t stream);

/* Checks every frame against the call's shape and format and its slot
 * (layer_base + l, b): recomputes the record's CRC-32 and the header's, and
 * writes the HKV_FRAME_BAD_* flags to status_out (uint32 [n_layers *
 * n_blocks], device, layer-major). */
int hkv_frame_verify(const hkv_shape* shape, int32_t fmt, const hkv_records* frames,
                     int32_t layer_base, uint32_t* status_out, hipStream_t stream);

/* delta_out[b] = m_new[b] - m_old of frame (0, b), clamped to the int32
 * range: the per-block delta for hkv_fetch_dequant_rope_shift (HyperCache
 * post, relative-RoPE paragraph: dm = m_new - m_old).  m_new, delta_out:
 * int32 [n_blocks], device.  Reads only the first layer's headers. */
int hkv_frame_delta_m(const hkv_shape* shape, int32_t fmt, const hkv_records* frames,
                      const int32_t* m_new, int32_t* delta_out, hipStream_t stream);

/* Recompute selection after a chunk reorder (HyperCache post, Core Design,
 * recompute paragraph; Part A, the "15% CacheBlend" line): the layer-0 KV
 * is exact after the rotation, and the tokens whose layer-0 hidden state
 * moved the most between the cached and the fresh context are the ones
 * recomputed through the deeper layers.
 *
 * Step 1, drift.  For t < n_tokens:
 *   drift_out[t] = sqrt( sum_j (h_fresh[t][j] - h_cached[t][j])^2 ),
 * j < d_model, element (t, j) at h + t*row_stride + j (row_stride in
 * ELEMENTS, shared by both arrays; dtype HKV_F32/F16/BF16).  Differences,
 * squares and the sum are fp32 (one accumulator per lane over
 * d_model/64 elements, then a 64-way tree), so the relative error is at most
 * about (d_model/64 + 10) * 2^-24.  h_cached, h_fresh: device, 16-byte
 * aligned, row_stride * element size a multiple of 16 and >= d_model when
 * n_tokens > 1.  drift_out: float [n_tokens], device.  n_tokens = 0 is an
 * empty call; d_model = 0 gives zeros (the row pointers may then be NULL). */
int hkv_token_drift(const void* h_cached, const void* h_fresh, int32_t n_tokens,
                    int32_t d_model, int64_t row_stride, int32_t dtype, float* drift_out,
                    hipStream_t stream);

/* Step 2, selection.  Writes to selected_out (int32 [k], device) the indices
 * of the k largest values of drift (float [n_tokens], device) in increasing
 * index order.  Order: a larger value first; NaN above every number; equal
 * values (+0 and -0 are equal) by lower index, so the result is unique.
 * 0 <= k <= n_tokens <= 2^30 (k = 0 writes nothing; more tokens:
 * HKV_ERR_UNSUPPORTED).  The caller picks k; the post recomputes about 15%
 * of the tokens.
 * workspace: NULL, or 16-byte aligned device memory of at least
 * hkv_select_workspace_bytes(n_tokens) bytes (workspace_bytes says how many).
 * Without it one workgroup makes four passes over drift (fine for a few
 * thousand tokens, ~2 ns per token beyond); with it the passes are spread
 * over up to 64 workgroups in five launches.  The workspace holds no state
 * between calls; calls that share one must not overlap. */
int hkv_select_top_tokens(const float* drift, int32_t n_tokens, int32_t k,
                          int32_t* selected_out, void* workspace, int64_t workspace_bytes,
                          hipStream_t stream);

/* Workspace bytes for hkv_select_top_tokens over n_tokens values (about
 * 24 KiB per 4,096 tokens up to 64k tokens, at most 1.6 MB); -1 if n_tokens
 * is negative or above 2^30. */
int64_t hkv_select_workspace_bytes(int32_t n_tokens);

/* Measurement aid, not a step of the method: a plain streaming kernel with
 * the fetch's byte mix.  Reads bytes_read bytes of src and writes 2 *
 * bytes_read bytes to dst (each 16 bytes twice, as two non-temporal 16-byte
 * stores 128 bytes apart), so a benchmark can state the fetch as a fraction
 * of what a kernel that only moves bytes in that ratio reaches.  bytes_read:
 * a multiple of 128; src, dst: device, 16-byte aligned, not overlapping. */
int hkv_stream_probe(const void* src, void* dst, int64_t bytes_read, hipStream_t stream);

/* Measurement aid, not a step of the method: a plain streaming kernel with
 * the put's byte mix.  Reads 2 * bytes_written bytes of src and writes
 * bytes_written bytes to dst: every 256-byte row of src becomes one 128-byte
 * row of dst, eight threads per row, each loading 16 bytes at offsets 16s and
 * 128 + 16s of the source row and storing two 8-byte words (xor mixes of
 * what it loaded) at offsets 8s and 64 + 8s of the output row, non-temporal,
 * like the put's loads of one bf16 vector and stores of its FP8 codes.
 * Output word pair of thread s in row r, with x, y the two loaded 16-byte
 * values as four 32-bit words each: dst[r][8s..] = {x0^y1, x2^y3},
 * dst[r][64+8s..] = {x1^y0, x3^y2}.  bytes_written: a multiple of 128, at most
 * 128 * (2^31 - 1) / 8 (HKV_ERR_UNSUPPORTED beyond); src, dst: device,
 * 16-byte aligned, not overlapping. */
int hkv_stream_probe_put(const void* src, void* dst, int64_t bytes_written, hipStream_t stream);

/* Host-only helpers. */

/* Bytes of one record: 2*N*C + 4*N (see hkv_records); -1 on bad arguments. */
int64_t hkv_record_bytes(int32_t fmt, int32_t block_tokens, int32_t n_kv_heads,
                         int32_t head_dim);

/* Static, NUL-terminated description of a status code. */
const char* hkv_status_string(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* HKV_H */
