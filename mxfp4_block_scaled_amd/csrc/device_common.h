// Device-side building blocks shared by the gfx950 kernels: MXFP4 group
// decode, wave64 reductions, bf16 rounding, the small in-workgroup bucketing.
//
// MXFP4 decode (page "MXFP4 Routed Expert Linear", sections "What is stored
// in one group" and "Apply the shared group scale"; page "MXFP4 Dequant",
// "How it works"): byte j of a 16-byte group holds code 2j in its low
// nibble and code 2j+1 in its high nibble; code n means E2M1[n] and the
// group's scale byte s multiplies every value by 2^(s-127).
//
// gfx950 has scaled FP4 converts (v_cvt_scalef32_pk_{f32,bf16}_fp4) that
// turn one byte (two codes, low nibble first) into two values times a
// power of two taken from the exponent field of an fp32 operand. Measured on
// MI355X over every byte and scale: the result equals E2M1[n] * 2^(s-127)
// bit for bit for s = 0..254; for s = 255 the instruction returns NaN
// (E8M0's NaN code), whereas the layer reads 255 as 2^128 like every other
// byte. Decoders therefore take a slow exact path for s = 255 under a
// wave-uniform branch that is never taken on ordinary data.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxfp4 {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kGroupBytes = 16;
constexpr int kGroupValues = 32;

// Cache-policy argument of the decode kernels' buffer loads of weight codes
// (gfx950: 2 = nt, non-temporal). Each code byte is read once. These kernels
// are bound by the vector L1's outstanding misses times their latency
// (counters on the T = 8 decode shape: the L1 waits on pending L2 data
// about 63% of its cycles); marked nt, the same number of L1-to-L2 requests
// came back about 8% sooner on average, and the kernels ran about 6%
// faster. The grouped GEMMs re-read weight lines (the other half of a line
// in the next chunk, an expert's weights again for its partial M-tile) and
// keep the default policy: nt made them slower.
constexpr int kCodeLoadPolicy = 2;

// fp32 operand whose exponent field is the E8M0 byte s: the scaled converts
// multiply by 2^(s-127).
__device__ __forceinline__ float e8m0_operand(uint32_t s) { return __uint_as_float(s << 23); }

// Two fp32 values E2M1[lo] * 2^(s-127), E2M1[hi] * 2^(s-127) of byte BYTE
// of w (s < 255). BYTE is a compile-time byte index 0..3.
template <int BYTE>
__device__ __forceinline__ f32x2 cvt_fp4x2_f32(uint32_t w, float scale_operand) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, scale_operand, BYTE);
}

// The same into a pair of bf16 (low half = low nibble's value). Written as
// inline assembly: the builtin's second element is lost by this compiler
// (it rebuilds the pair from the low half), while the instruction itself
// returns both values in one 32-bit register.
template <int BYTE>
__device__ __forceinline__ uint32_t cvt_fp4x2_bf16(uint32_t w, float scale_operand) {
  uint32_t r;
  if constexpr (BYTE == 0)
    asm("v_cvt_scalef32_pk_bf16_fp4 %0, %1, %2" : "=v"(r) : "v"(w), "v"(scale_operand));
  else if constexpr (BYTE == 1)
    asm("v_cvt_scalef32_pk_bf16_fp4 %0, %1, %2 op_sel:[1,0,0]" : "=v"(r) : "v"(w), "v"(scale_operand));
  else if constexpr (BYTE == 2)
    asm("v_cvt_scalef32_pk_bf16_fp4 %0, %1, %2 op_sel:[0,1,0]" : "=v"(r) : "v"(w), "v"(scale_operand));
  else
    asm("v_cvt_scalef32_pk_bf16_fp4 %0, %1, %2 op_sel:[1,1,0]" : "=v"(r) : "v"(w), "v"(scale_operand));
  return r;
}

// c + a.lo * b.lo + a.hi * b.hi for two bf16 pairs, fp32 accumulate
// (v_dot2c_f32_bf16). The operands go through memcpy: with this compiler a
// bit cast of the 32-bit elements of a vector makes the builtin reuse one
// element for all of them. (Not inline assembly: the compiler must see the
// instruction to add the wait states its result needs.)
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  bf16x2 av, bv;
  __builtin_memcpy(&av, &a, 4);
  __builtin_memcpy(&bv, &b, 4);
  return __builtin_amdgcn_fdot2_f32_bf16(av, bv, c, false);
}

// Round-to-nearest-even fp32 -> bf16 bits (NaN stays a quiet NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Exact fp32 value of E2M1 code n times 2^(s-127) for any s (slow path).
__device__ __forceinline__ float e2m1_scaled_exact(uint32_t n, uint32_t s) {
  // E2M1: sign bit 3, exponent bits 2..1, mantissa bit 0; magnitudes
  // 0, .5, 1, 1.5, 2, 3, 4, 6 = (m ? 1.5 : 1) * 2^(e-1) for e > 0, m * 0.5 for e = 0.
  uint32_t mag = n & 7u, e = mag >> 1, m = mag & 1u;
  float v = (e == 0) ? (m ? 0.5f : 0.0f) : ((m ? 1.5f : 1.0f) * (float)(1u << (e - 1)));
  v = __builtin_amdgcn_ldexpf(v, (int)s - 127);
  return (n & 8u) ? -v : v;
}

// Decode the 4 bytes of w (8 codes, low nibble first) at scale byte s into
// 8 bf16 (as 4 packed 32-bit words, element 2i in the low half of word i).
__device__ __forceinline__ void decode8_bf16_slow(uint32_t w, uint32_t s, uint32_t out[4]) {
#pragma unroll
  for (int b = 0; b < 4; b++) {
    uint32_t byte = (w >> (8 * b)) & 0xffu;
    uint16_t lo = f32_to_bf16_rne(e2m1_scaled_exact(byte & 15u, s));
    uint16_t hi = f32_to_bf16_rne(e2m1_scaled_exact(byte >> 4, s));
    out[b] = (uint32_t)lo | ((uint32_t)hi << 16);
  }
}

// Scale byte 255 (2^128): decode at 2^127 in fp32 (exact), double (exact,
// overflowing to +-inf where the value does), keep the bf16 high halves
// (exact: every such value is a bf16 value or an infinity).
__device__ __forceinline__ void decode8_bf16_s255(uint32_t w, uint32_t out[4]) {
  const float sc = e8m0_operand(254);
  f32x2 v[4];
  v[0] = cvt_fp4x2_f32<0>(w, sc);
  v[1] = cvt_fp4x2_f32<1>(w, sc);
  v[2] = cvt_fp4x2_f32<2>(w, sc);
  v[3] = cvt_fp4x2_f32<3>(w, sc);
#pragma unroll
  for (int b = 0; b < 4; b++) {
    const float lo = v[b].x * 2.0f, hi = v[b].y * 2.0f;
    out[b] = (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xffff0000u);
  }
}

__device__ __forceinline__ void decode8_bf16_fast(uint32_t w, float sc, uint32_t out[4]) {
  out[0] = cvt_fp4x2_bf16<0>(w, sc);
  out[1] = cvt_fp4x2_bf16<1>(w, sc);
  out[2] = cvt_fp4x2_bf16<2>(w, sc);
  out[3] = cvt_fp4x2_bf16<3>(w, sc);
}

// The same 8 values as an MFMA operand. Built from the builtin's vector
// elements, which this compiler keeps intact (unlike a bit cast of the pair
// to 32 bits): the four converts then write the operand registers directly,
// with no copies.
__device__ __forceinline__ bf16x8 decode8_bf16x8(uint32_t w, float sc) {
  const bf16x2 r0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0);
  const bf16x2 r1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1);
  const bf16x2 r2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2);
  const bf16x2 r3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3);
  return bf16x8{r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]};
}

// Unscaled E2M1 values of the 8 codes of w as fp32 (exact).
__device__ __forceinline__ void decode8_f32_unscaled(uint32_t w, float out[8]) {
  f32x2 a = cvt_fp4x2_f32<0>(w, 1.0f), b = cvt_fp4x2_f32<1>(w, 1.0f);
  f32x2 c = cvt_fp4x2_f32<2>(w, 1.0f), d = cvt_fp4x2_f32<3>(w, 1.0f);
  out[0] = a.x; out[1] = a.y; out[2] = b.x; out[3] = b.y;
  out[4] = c.x; out[5] = c.y; out[6] = d.x; out[7] = d.y;
}

// fp32 -> three bf16 (bit patterns) with f = x0 + x1 + x2 exactly: each
// piece keeps the top 8 significant bits of what is left, and the
// subtractions are exact (both operands share sign and exponent range).
__device__ __forceinline__ void split3(float f, uint32_t& b0, uint32_t& b1, uint32_t& b2) {
  const uint32_t u = __float_as_uint(f);
  const float r1 = f - __uint_as_float(u & 0xffff0000u);
  const uint32_t u1 = __float_as_uint(r1);
  const float r2 = r1 - __uint_as_float(u1 & 0xffff0000u);
  b0 = u >> 16;
  b1 = u1 >> 16;
  b2 = __float_as_uint(r2) >> 16;
}

// Sum over the 64 lanes of a wave in a fixed butterfly order. Every lane
// gets the same bits, so the result is deterministic.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

}  // namespace mxfp4
