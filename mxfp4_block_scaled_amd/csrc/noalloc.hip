// The routed linear without any allocation: mxfp4_moe_linear_ex on a scratch
// array that the library owns, one per device, in device memory that the
// code object brings with it. For callers that cannot allocate (code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The array is a file-scope __device__ symbol. In host code its name is a
// host-side stand-in, not a device address, so the host never passes it to
// a kernel: the first call on a device looks up that device's copy with
// hipGetSymbolAddress (with the device current) and keeps the address; every
// later call on the device uses the kept address.
#include <hip/hip_runtime.h>

#include <mutex>

#include "mxfp4_moe.h"

namespace {

constexpr size_t kScratchBytes = size_t(MXFP4_NOALLOC_SCRATCH_BYTES);
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::once_flag g_once[kMaxDevices];
void* g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];

// this device's copy of the scratch array (null and an error when the lookup failed)
void* device_scratch(int dev, hipError_t* err) {
  std::call_once(g_once[dev], [dev] {
    void* p = nullptr;
    g_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_ptr[dev] = g_err[dev] == hipSuccess ? p : nullptr;
  });
  *err = g_err[dev];
  return g_ptr[dev];
}

}  // namespace

extern "C" int mxfp4_moe_linear_noalloc(const void* x, const uint8_t* packed, const uint8_t* scales,
                                        const int32_t* sel, const float* p, const void* shared, void* y, int64_t T,
                                        int64_t E, int64_t O, int64_t G, int64_t K, int dtype, uint32_t flags,
                                        hipStream_t stream) {
  size_t need = 0;
  int st = mxfp4_moe_workspace_size(T, E, O, G, K, dtype, flags, &need);
  if (st != MXFP4_OK) return st;
  if (need > kScratchBytes) return MXFP4_ERR_WORKSPACE_TOO_SMALL;
  if (T == 0) return mxfp4_moe_linear_ex(x, packed, scales, sel, p, shared, y, T, E, O, G, K, dtype, flags, nullptr,
                                         0, stream);
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MXFP4_ERR_HIP;
  hipError_t err = hipSuccess;
  void* ws = device_scratch(dev, &err);
  if (err != hipSuccess || !ws) return MXFP4_ERR_HIP;
  return mxfp4_moe_linear_ex(x, packed, scales, sel, p, shared, y, T, E, O, G, K, dtype, flags, ws, kScratchBytes,
                             stream);
}
