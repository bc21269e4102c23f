// Stream pair that splits the device's compute units between the fetch and
// the caller's compute, for the layer-wise overlap the HyperCache post
// describes (layer-wise transfer paragraph: fetch layer l+1 while the GPU
// computes layer l).  On one GPU the fetch is itself an HBM-bound kernel: if
// the compute kernel holds every CU, the fetch runs only in its gaps.  Giving
// the fetch its own CUs lets both run at once.  The fetch gets the first
// fetch_cus CUs of the device and the compute the rest: masks that pick CUs
// sparsely (every k-th CU) were refused by the runtime on MI355X, contiguous
// ranges are accepted, and a streaming kernel's bandwidth grows about
// linearly with the range (measured ~55 GB/s per CU).  Streams keep the
// default priority.
#include "hkv.h"

#include <stdint.h>

#include <vector>

extern "C" {

int hkv_stream_pair_create(int32_t fetch_cus, hipStream_t* fetch_stream,
                           hipStream_t* compute_stream) {
  if (!fetch_stream || !compute_stream) return HKV_ERR_INVALID_ARG;
  int dev = 0, n_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return HKV_ERR_HIP;
  if (hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return HKV_ERR_HIP;
  if (fetch_cus < 1 || fetch_cus >= n_cu) return HKV_ERR_INVALID_ARG;
  const int words = (n_cu + 31) / 32;
  std::vector<uint32_t> fetch_mask(words, 0u), compute_mask(words, 0u);
  for (int i = 0; i < n_cu; ++i) {
    std::vector<uint32_t>& m = i < fetch_cus ? fetch_mask : compute_mask;
    m[i / 32] |= 1u << (i % 32);
  }
  // A failed creation leaves an error that the runtime would otherwise report
  // at the caller's next, unrelated call: read it back (which clears it).
  hipStream_t f = nullptr, c = nullptr;
  if (hipExtStreamCreateWithCUMask(&f, static_cast<uint32_t>(words), fetch_mask.data()) !=
      hipSuccess) {
    (void)hipGetLastError();
    return HKV_ERR_HIP;
  }
  if (hipExtStreamCreateWithCUMask(&c, static_cast<uint32_t>(words), compute_mask.data()) !=
      hipSuccess) {
    (void)hipGetLastError();
    (void)hipStreamDestroy(f);
    return HKV_ERR_HIP;
  }
  *fetch_stream = f;
  *compute_stream = c;
  return HKV_OK;
}

int hkv_stream_destroy(hipStream_t stream) {
  if (!stream) return HKV_ERR_INVALID_ARG;
  return hipStreamDestroy(stream) == hipSuccess ? HKV_OK : HKV_ERR_HIP;
}

}  // extern "C"
