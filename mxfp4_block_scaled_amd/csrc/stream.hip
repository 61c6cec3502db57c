// Plain streaming read of a device buffer: the practical HBM read ceiling
// that the decode-shaped kernels are compared with (a measurement helper,
// not a step of the layer). Every thread reads 16-byte pieces in a
// grid-stride loop, four in flight; the values are folded together and
// stored only if they equal a constant that no real data produces in
// practice, so that no load can be dropped and nothing is written.
#include <algorithm>

#include "device_common.h"
#include "launch.h"

namespace mxfp4 {
namespace {

__global__ void __launch_bounds__(256) stream_read_kernel(const u32x4* __restrict__ buf, int64_t n16,
                                                          uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  u32x4 acc = u32x4{0u, 0u, 0u, 0u};
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = buf[i], b = buf[i + stride], c = buf[i + 2 * stride], d = buf[i + 3 * stride];
    acc ^= a ^ b ^ c ^ d;
  }
  for (; i < n16; i += stride) acc ^= buf[i];
  const uint32_t v = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (v == 0x9E3779B9u && threadIdx.x == 0) sink[blockIdx.x] = v;
}

}  // namespace

hipError_t launch_stream_read(const void* buf, int64_t bytes, int blocks, uint32_t* sink, hipStream_t stream) {
  const int64_t n16 = bytes / 16;
  if (n16 <= 0) return hipSuccess;
  int64_t nb = blocks > 0 ? blocks : std::min<int64_t>((n16 + 255) / 256, 2048);
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)nb), dim3(256), 0, stream, static_cast<const u32x4*>(buf), n16,
                     sink);
  return hipGetLastError();
}

}  // namespace mxfp4
