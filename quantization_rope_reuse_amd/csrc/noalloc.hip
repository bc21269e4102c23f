// hkv_quant_fp8_crc_noalloc: the fused FP8 put + CRC-32 for callers that
// cannot allocate device memory (code under HIP graph capture, serving loops
// that never call the allocator, harnesses that forbid it).
//
// The fused put + CRC needs scratch memory for the raw CRCs of the records'
// 128-byte code units.  Here it is a file-scope device array, `scratch`, of
// HKV_NOALLOC_SCRATCH_BYTES.  Every GPU that runs this library holds its own
// copy of the array at its own address until the process ends.  In host code
// the name `scratch` is only a host-side stand-in, so its device address is
// looked up once per device with hipGetSymbolAddress (with that device
// current) and that address is what the kernels receive.
//
// The put writes every scratch slot the merge reads before the merge reads
// it, so no part of the array has to start at zero and nothing is cleared;
// calls that overlap on one GPU share the array and race.
#include "hkv.h"

#include <stdint.h>

#include <mutex>

#include "hkv_launch.h"

namespace {

constexpr int64_t kScratchBytes = HKV_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_lock;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` per device, once known

// Device address of this device's `scratch`, looked up on first use with the
// device current.  The previously current device is restored.
int scratch_address(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return HKV_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> guard(g_lock);
  if (!g_scratch_ptr[dev]) {
    int prev = 0;
    if (hipGetDevice(&prev) != hipSuccess) return HKV_ERR_HIP;
    if (prev != dev && hipSetDevice(dev) != hipSuccess) return HKV_ERR_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (prev != dev) (void)hipSetDevice(prev);
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      return HKV_ERR_HIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return HKV_OK;
}

}  // namespace

extern "C" int hkv_quant_fp8_crc_noalloc(const hkv_shape* shape, const hkv_pages* src,
                                         int32_t src_dtype, const int32_t* block_table,
                                         const hkv_records* dst, uint32_t* crc_out,
                                         hipStream_t stream) {
  int64_t need = 0;
  const int st0 = hkv::quant_crc_validate(HKV_FP8_E4M3, shape, src, src_dtype, block_table, dst,
                                          crc_out, &need);
  if (st0 != HKV_OK) return st0;
  if (need > kScratchBytes) return HKV_ERR_UNSUPPORTED;
  void* ws = nullptr;
  if (need > 0) {
    // the device the stream belongs to (the current one for the null stream)
    int dev = 0;
    if (hipStreamGetDevice(stream, &dev) != hipSuccess) {
      (void)hipGetLastError();
      return HKV_ERR_HIP;
    }
    const int st = scratch_address(dev, &ws);
    if (st != HKV_OK) return st;
  }
  return hkv_quant_fp8_crc(shape, src, src_dtype, block_table, dst, crc_out, ws,
                           ws ? kScratchBytes : 0, stream, nullptr);
}
