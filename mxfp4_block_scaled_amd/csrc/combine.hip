// Combine of the prefill-shaped path and the exported row decode.
//
// Combine (page "MXFP4 Routed Expert Linear", "Route, weight, and add the
// shared path" and "Implementation order"):
//     y[t, o] = round(shared[t, o] + (sum over k = 0..K-1, in order, of p[t,k] * part[slot(t,k), o]))
// One thread per output element, fp32 fused multiply-adds in slot order,
// one rounding to y's dtype; no atomics, so the result is deterministic.
#include "device_common.h"
#include "launch.h"

namespace mxfp4 {
namespace {

template <bool BF16>
__global__ void __launch_bounds__(256) combine_kernel(const float* __restrict__ part,
                                                      const int32_t* __restrict__ slot_of_pair,
                                                      const float* __restrict__ p, const void* shared, void* y, int T,
                                                      int K, int O) {
  for (int t = blockIdx.y; t < T; t += gridDim.y) {
    for (int o = blockIdx.x * 256 + threadIdx.x; o < O; o += gridDim.x * 256) {
      float a = 0.f;
      for (int k = 0; k < K; k++) {
        const int sp = slot_of_pair[t * K + k];
        if (sp >= 0) a = fmaf(p[t * K + k], part[(int64_t)sp * O + o], a);
      }
      const int64_t yo = (int64_t)t * O + o;
      if constexpr (BF16) {
        const uint16_t sh = static_cast<const uint16_t*>(shared)[yo];
        static_cast<uint16_t*>(y)[yo] = f32_to_bf16_rne(bf16_to_f32(sh) + a);
      } else {
        const float sh = static_cast<const float*>(shared)[yo];
        static_cast<float*>(y)[yo] = sh + a;
      }
    }
  }
}

// Exact decode of whole rows: one thread per 16-byte group.
__global__ void __launch_bounds__(256) decode_rows_kernel(const uint8_t* __restrict__ packed_rows,
                                                          const uint8_t* __restrict__ scales_rows, int64_t nrows,
                                                          int64_t G, int dtype, void* out) {
  const int64_t n = nrows * G;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < n; idx += (int64_t)gridDim.x * 256) {
    const u32x4 wv = *reinterpret_cast<const u32x4*>(packed_rows + idx * 16);
    const uint32_t s = scales_rows[idx];
    if (dtype == 0) {
      // unscaled table values, then the exact power-of-two scaling
      float v[32];
#pragma unroll
      for (int j = 0; j < 4; j++) decode8_f32_unscaled(wv[j], v + 8 * j);
      float4* o = reinterpret_cast<float4*>(static_cast<float*>(out) + idx * 32);
#pragma unroll
      for (int j = 0; j < 8; j++) {
        o[j] = make_float4(__builtin_amdgcn_ldexpf(v[4 * j], (int)s - 127), __builtin_amdgcn_ldexpf(v[4 * j + 1], (int)s - 127),
                           __builtin_amdgcn_ldexpf(v[4 * j + 2], (int)s - 127), __builtin_amdgcn_ldexpf(v[4 * j + 3], (int)s - 127));
      }
    } else {
      uint32_t wd[4][4];
#pragma unroll
      for (int j = 0; j < 4; j++) {
        if (s == 255) decode8_bf16_slow(wv[j], s, wd[j]);
        else decode8_bf16_fast(wv[j], e8m0_operand(s), wd[j]);
      }
      u32x4* o = reinterpret_cast<u32x4*>(static_cast<uint16_t*>(out) + idx * 32);
#pragma unroll
      for (int j = 0; j < 4; j++) o[j] = u32x4{wd[j][0], wd[j][1], wd[j][2], wd[j][3]};
    }
  }
}

}  // namespace

hipError_t launch_combine(const float* part, const int32_t* slot_of_pair, const float* p, const void* shared, void* y,
                          int T, int K, int O, int dtype, hipStream_t stream) {
  const unsigned gx = (unsigned)((O + 255) / 256);
  const unsigned gy = (unsigned)(T < 32768 ? T : 32768);
  if (dtype == 1)
    hipLaunchKernelGGL(combine_kernel<true>, dim3(gx, gy), dim3(256), 0, stream, part, slot_of_pair, p, shared, y, T, K, O);
  else
    hipLaunchKernelGGL(combine_kernel<false>, dim3(gx, gy), dim3(256), 0, stream, part, slot_of_pair, p, shared, y, T, K, O);
  return hipGetLastError();
}

hipError_t launch_decode_rows(const uint8_t* packed_rows, const uint8_t* scales_rows, int64_t nrows, int64_t G,
                              int dtype, void* out, hipStream_t stream) {
  const int64_t n = nrows * G;
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(decode_rows_kernel, dim3((unsigned)(blocks < 65536 ? blocks : 65536)), dim3(256), 0, stream,
                     packed_rows, scales_rows, nrows, G, dtype, out);
  return hipGetLastError();
}

}  // namespace mxfp4
