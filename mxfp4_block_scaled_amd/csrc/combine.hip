// Combine of the prefill-shaped path and the exported row decode.
//
// Combine (page "MXFP4 Routed Expert Linear", "Route, weight, and add the
// shared path" and "Implementation order"):
//     y[t, o] = round(shared[t, o] + (sum over k = 0..K-1, in order, of p[t,k] * part[slot(t,k), o]))
// One thread per output element (or four, with 16-byte loads), fp32 fused
// multiply-adds in slot order, one rounding to y's dtype; no atomics, so the
// result is deterministic and the same in both forms.
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

// The same, four outputs per thread with 16-byte loads of the partial rows
// (O % 4 == 0, so every row start is 16-byte aligned). Each slot's partial
// row is read through a buffer resource of its own (a dropped slot gets an
// empty resource: zeros, no traffic, weight 0), so the KT loads of an output
// quad are issued back to back and waited for once, instead of one load and
// one wait per slot behind a branch. KT = K at compile time for the common
// K; KT = 0 takes K at run time (up to kCombMaxK).
constexpr int kCombMaxK = 16;
constexpr int kRsrcFlags = 0x00020000;
// cache policy of the partial-row loads (gfx950: 2 = nt, non-temporal):
// each partial row is read once, here
constexpr int kPartLoadPolicy = 2;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
// the output rows are written once and not read again by this pass, so
// they are stored non-temporally too (global_store ... nt)
template <bool BF16, int KT>
__global__ void __launch_bounds__(256) combine4_kernel(const float* __restrict__ part,
                                                       const int32_t* __restrict__ slot_of_pair,
                                                       const float* __restrict__ p, const void* shared, void* y, int T,
                                                       int K, int O) {
  constexpr int KM = KT > 0 ? KT : kCombMaxK;
  if constexpr (KT > 0) K = KT;
  const int O4 = O >> 2;
  for (int t = blockIdx.y; t < T; t += gridDim.y) {
    __amdgpu_buffer_rsrc_t rk[KM];
    float pk[KM];
#pragma unroll
    for (int k = 0; k < KM; k++) {
      const int sp = k < K ? slot_of_pair[t * K + k] : -1;
      pk[k] = sp >= 0 ? p[t * K + k] : 0.f;
      rk[k] = __builtin_amdgcn_make_buffer_rsrc((void*)(part + (int64_t)(sp >= 0 ? sp : 0) * O), (short)0,
                                                sp >= 0 ? O * 4 : 0, kRsrcFlags);
    }
    for (int o4 = blockIdx.x * 256 + threadIdx.x; o4 < O4; o4 += gridDim.x * 256) {
      f32x4 v[KM];
#pragma unroll
      for (int k = 0; k < KM; k++) v[k] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rk[k], 16 * o4, 0, kPartLoadPolicy));
      f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < KM; k++)
#pragma unroll
        for (int i = 0; i < 4; i++) a[i] = fmaf(pk[k], v[k][i], a[i]);
      const int64_t yo = (int64_t)t * O + 4 * o4;
      if constexpr (BF16) {
        const uint2 sh = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(shared) + yo);
        const uint32_t r0 = f32_to_bf16_rne(bf16_to_f32((uint16_t)sh.x) + a[0]);
        const uint32_t r1 = f32_to_bf16_rne(bf16_to_f32((uint16_t)(sh.x >> 16)) + a[1]);
        const uint32_t r2 = f32_to_bf16_rne(bf16_to_f32((uint16_t)sh.y) + a[2]);
        const uint32_t r3 = f32_to_bf16_rne(bf16_to_f32((uint16_t)(sh.y >> 16)) + a[3]);
        __builtin_nontemporal_store(u32x2{r0 | (r1 << 16), r2 | (r3 << 16)},
                                    reinterpret_cast<u32x2*>(static_cast<uint16_t*>(y) + yo));
      } else {
        const f32x4 sh = *reinterpret_cast<const f32x4*>(static_cast<const float*>(shared) + yo);
        f32x4 r;
#pragma unroll
        for (int i = 0; i < 4; i++) r[i] = sh[i] + a[i];
        __builtin_nontemporal_store(r, reinterpret_cast<f32x4*>(static_cast<float*>(y) + yo));
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

template <int KT>
void launch_combine4(dim3 grid, const float* part, const int32_t* slot_of_pair, const float* p, const void* shared,
                     void* y, int T, int K, int O, int dtype, hipStream_t stream) {
  if (dtype == 1)
    hipLaunchKernelGGL((combine4_kernel<true, KT>), grid, dim3(256), 0, stream, part, slot_of_pair, p, shared, y, T, K, O);
  else
    hipLaunchKernelGGL((combine4_kernel<false, KT>), grid, dim3(256), 0, stream, part, slot_of_pair, p, shared, y, T, K,
                       O);
}

hipError_t launch_combine(const float* part, const int32_t* slot_of_pair, const float* p, const void* shared, void* y,
                          int T, int K, int O, int dtype, hipStream_t stream) {
  const unsigned gy = (unsigned)(T < 32768 ? T : 32768);
  const bool vec = O % 4 == 0 && K <= kCombMaxK && reinterpret_cast<uintptr_t>(part) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(shared) % 16 == 0 && reinterpret_cast<uintptr_t>(y) % 16 == 0;
  if (vec) {
    const dim3 grid((unsigned)((O / 4 + 255) / 256), gy);
    switch (K) {
      case 1: launch_combine4<1>(grid, part, slot_of_pair, p, shared, y, T, K, O, dtype, stream); break;
      case 2: launch_combine4<2>(grid, part, slot_of_pair, p, shared, y, T, K, O, dtype, stream); break;
      case 4: launch_combine4<4>(grid, part, slot_of_pair, p, shared, y, T, K, O, dtype, stream); break;
      case 8: launch_combine4<8>(grid, part, slot_of_pair, p, shared, y, T, K, O, dtype, stream); break;
      default: launch_combine4<0>(grid, part, slot_of_pair, p, shared, y, T, K, O, dtype, stream); break;
    }
    return hipGetLastError();
  }
  const unsigned gx = (unsigned)((O + 255) / 256);
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
