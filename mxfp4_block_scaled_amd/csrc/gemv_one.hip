// Decode-shaped path for one token (T = 1): routing, dequant-GEMV and
// combine in one launch, on the vector ALUs, with the token's activations
// held in registers.
//
//     y[o] = shared[o] + sum_{k<K} p[k] * (W_{sel[k]} x)[o]
//
// (page "MXFP4 Routed Expert Linear", "Route, weight, and add the shared
// path"; each output coordinate is a row of W_e dotted with the token,
// "Reconstruct the matrix in the right orientation").
//
// Lane layout. A wave covers RPW = 64 / LPR consecutive output rows at a
// time, LPR lanes per row; lane j of a row owns the groups j, j + LPR, ...,
// j + (NG - 1) LPR of every row it ever touches (NG * LPR >= G). So one
// wave-wide 16-byte load reads LPR consecutive groups (16 LPR contiguous
// bytes) of each of its RPW rows, and the lane's activations - 32 values
// per owned group - never change: they are read once from LDS into
// registers and serve every row and every expert of the call. There is no
// activation traffic per weight byte at all.
//
// Work. The rows are cut into row sets of RPW rows, and every wave takes a
// contiguous range of row sets. A slot is (row set, k): the RPW rows of
// expert sel[k]. Slots run k-minor, with kRing slots of loads in flight in
// registers (every slot issues the same loads; a group past G, a row past
// O or an expert index outside [0, E) reads beyond its buffer resource:
// zeros, no memory traffic).
//
// Arithmetic (page "MXFP4 Dequant", "How it works": code n is E2M1[n]
// times 2^(s-127)). A lane takes the dot product of a group's exact E2M1
// values with its activations in fp32 (fp32 activations: fp32 FMA; bf16
// activations: v_dot2_f32_bf16), multiplies it by 2^(s-127) with ldexp
// (exact, so no decoded weight can overflow, whatever the scale byte), adds
// its groups, and accumulates p[k] times that into its row sum, k in order.
// When a row set's K slots are done, the LPR lanes of each row are summed
// by a fixed butterfly, and one lane writes y = shared + sum, rounded once.
// The order of every sum is fixed, so results are deterministic.
#include "device_common.h"
#include "launch.h"

namespace mxfp4 {
namespace {

constexpr int kWaves = 4;
// group offset beyond any expert's resource (O * G < 2^27): loads return zero
constexpr uint32_t kOobGroup = 0x08000000u;
constexpr uint32_t kOobByte = 0x80000000u;
constexpr int kRsrcFlags = 0x00020000;  // raw buffer, 32-bit data format
#ifndef MXFP4_DECODE1_RING
#define MXFP4_DECODE1_RING 1
#endif
#ifndef MXFP4_DECODE1_WG_PER_CU
#define MXFP4_DECODE1_WG_PER_CU 4
#endif
#ifndef MXFP4_DECODE1_MIN_WAVES
#define MXFP4_DECODE1_MIN_WAVES 2
#endif
constexpr int kRing = MXFP4_DECODE1_RING;  // slots whose loads a wave keeps in flight
#ifndef MXFP4_DECODE1_MAX_NG
#define MXFP4_DECODE1_MAX_NG 4
#endif
constexpr int kMaxNG = MXFP4_DECODE1_MAX_NG;  // groups per lane (activation registers: 32 NG fp32)
constexpr int kMaxG = 64 * kMaxNG;
constexpr int kXPre = kMaxG * 8 / (kWaves * 64);  // 16-byte activation chunks per thread, at most

template <bool XF32, int NG>
__global__ void __launch_bounds__(kWaves * 64, MXFP4_DECODE1_MIN_WAVES) gemv_one_kernel(
    const void* __restrict__ xv, const uint8_t* __restrict__ packed, const uint8_t* __restrict__ scales,
    const int32_t* __restrict__ sel, const float* __restrict__ p, const void* shared, void* y, int E, int O, int G,
    int K, int lpr_log2, int n_rs, int32_t* __restrict__ n_invalid) {
  constexpr int CH = XF32 ? 8 : 4;  // 16-byte activation chunks per group
  constexpr int GS = CH * 16 + 16;  // LDS bytes per group (padded: 16 lanes read 16 groups conflict-free)
  constexpr int es = XF32 ? 4 : 2;  // bytes per activation / output element
  extern __shared__ __attribute__((aligned(16))) uint8_t xs[];  // [G][GS]
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int LPR = 1 << lpr_log2, RPW = 64 >> lpr_log2;
  const int h = lane >> lpr_log2, jl = lane & (LPR - 1);

  // ---- routing input (lane k: slot k), then the activations, before anything
  // waits. Every load is unconditional (clamped indices), so that no branch
  // joins force a wait for all loads in flight.
  const int sel_raw = sel[lane < K ? lane : 0];
  const float p_raw = p[lane < K ? lane : 0];
  const int nch = G * CH;
  // activations through a buffer resource: a chunk past the row reads zeros, no traffic
  const __amdgpu_buffer_rsrc_t rx =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(xv), (short)0, nch * 16, kRsrcFlags);
  u32x4 xr[kXPre];
#pragma unroll
  for (int i = 0; i < kXPre; i++)
    xr[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, (tid + i * kWaves * 64) * 16, 0, 0));
  const int sel_l = lane < K ? sel_raw : -1;
  const float p_l = lane < K ? p_raw : 0.f;

  // ---- this wave's row sets and slots
  const int64_t nwt = (int64_t)gridDim.x * kWaves, gw = (int64_t)blockIdx.x * kWaves + w;
  const int rs0 = (int)(gw * n_rs / nwt), rs1 = (int)((gw + 1) * n_rs / nwt);
  const int nslot = (rs1 - rs0) * K;
  const uint32_t wbytes = (uint32_t)O * (uint32_t)G * 16u, sbytes = (uint32_t)O * (uint32_t)G;
  const __amdgpu_buffer_rsrc_t rsh =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(shared), (short)0, (int)((uint32_t)O * es), kRsrcFlags);

  // ---- issue cursor: slot i_q = (row set i_rs, slot i_k)
  int i_q = 0, i_rs = rs0, i_k = 0;
  u32x4 wq[kRing][NG];
  uint32_t sq[kRing][NG];
  float shq[kRing];
  auto issue = [&](int pos) {
    const bool live = i_q < nslot;
    const int e = live ? __builtin_amdgcn_readlane(sel_l, i_k) : -1;
    const bool ok = e >= 0 && e < E;
    const int eo = ok ? e : 0;
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(packed + (int64_t)eo * wbytes), (short)0, ok ? (int)wbytes : 0, kRsrcFlags);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(scales + (int64_t)eo * sbytes), (short)0, ok ? (int)sbytes : 0, kRsrcFlags);
    const int row = i_rs * RPW + h;
    // a row past O: the sign bit of O - 1 - row moves the offset past the resource
    const uint32_t row_out = (uint32_t)(O - 1 - row) >> 31;
#pragma unroll
    for (int j = 0; j < NG; j++) {
      const int g = jl + (j << lpr_log2);
      const uint32_t out = row_out | ((uint32_t)(G - 1 - g) >> 31);
      const uint32_t off = (uint32_t)(row * G + g) | (out * kOobGroup);
      wq[pos][j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, (int)(off * 16u), 0, kCodeLoadPolicy));
      // the scale bytes non-temporal too: decode 9.44-9.51 -> 9.35-9.39 us (the
      // row-contiguous kernel's decode8 measured slower with them: 112.8 -> 119.7 us)
      sq[pos][j] = __builtin_amdgcn_raw_buffer_load_b8(rs, (int)off, 0, kCodeLoadPolicy);
    }
    // the shared output of the row, with the row set's last slot (a wave-uniform test)
    const uint32_t last = (live && i_k == K - 1) ? 0u : 1u;
    const uint32_t so = ((uint32_t)row * es) | ((row_out | last) * kOobByte);
    if constexpr (XF32) {
      shq[pos] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsh, (int)so, 0, 0));
    } else {
      shq[pos] = bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(rsh, (int)so, 0, 0));
    }
    if (live) {
      i_q++;
      if (++i_k == K) i_k = 0, i_rs++;
    }
  };
#pragma unroll
  for (int s = 0; s < kRing; s++) issue(s);
  __builtin_amdgcn_sched_barrier(0);  // every load is out before the first wait

  // ---- activations -> LDS (group g at g * GS), then this lane's groups -> registers
#pragma unroll
  for (int i = 0; i < kXPre; i++) {
    const int c = tid + i * kWaves * 64;
    if (c < nch) *reinterpret_cast<u32x4*>(xs + (c / CH) * GS + (c % CH) * 16) = xr[i];
  }
  __syncthreads();
  u32x4 xg[NG][CH];
#pragma unroll
  for (int j = 0; j < NG; j++) {
    const int g = jl + (j << lpr_log2);
#pragma unroll
    for (int c = 0; c < CH; c++)
      xg[j][c] = g < G ? *reinterpret_cast<const u32x4*>(xs + g * GS + c * 16) : u32x4{0u, 0u, 0u, 0u};
  }
  if (blockIdx.x == 0 && w == 0 && n_invalid) {
    const uint64_t bad = __ballot(lane < K && (sel_l < 0 || sel_l >= E));
    if (lane == 0) n_invalid[0] = __popcll(bad);
  }

  // ---- compute cursor
  int c_q = 0, c_rs = rs0, c_k = 0;
  float yacc = 0.f;
  const float one = e8m0_operand(127u);
  auto consume = [&](int pos) {
    if (c_q >= nslot) return;
    const int e = __builtin_amdgcn_readlane(sel_l, c_k);
    const float pk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(p_l), c_k));
    float part = 0.f;
#pragma unroll
    for (int j = 0; j < NG; j++) {
      float a = 0.f;
      if constexpr (XF32) {
#pragma unroll
        for (int d = 0; d < 4; d++) {
          const uint32_t wd = wq[pos][j][d];
          const f32x2 v0 = cvt_fp4x2_f32<0>(wd, one), v1 = cvt_fp4x2_f32<1>(wd, one);
          const f32x2 v2 = cvt_fp4x2_f32<2>(wd, one), v3 = cvt_fp4x2_f32<3>(wd, one);
          const u32x4 xa = xg[j][2 * d], xb = xg[j][2 * d + 1];
          a = fmaf(v0.x, __uint_as_float(xa[0]), a);
          a = fmaf(v0.y, __uint_as_float(xa[1]), a);
          a = fmaf(v1.x, __uint_as_float(xa[2]), a);
          a = fmaf(v1.y, __uint_as_float(xa[3]), a);
          a = fmaf(v2.x, __uint_as_float(xb[0]), a);
          a = fmaf(v2.y, __uint_as_float(xb[1]), a);
          a = fmaf(v3.x, __uint_as_float(xb[2]), a);
          a = fmaf(v3.y, __uint_as_float(xb[3]), a);
        }
      } else {
#pragma unroll
        for (int d = 0; d < 4; d++) {
          uint32_t wd[4];
          decode8_bf16_fast(wq[pos][j][d], one, wd);
#pragma unroll
          for (int t = 0; t < 4; t++) a = dot2_bf16(wd[t], xg[j][d][t], a);
        }
      }
      part += __builtin_amdgcn_ldexpf(a, (int)sq[pos][j] - 127);
    }
    if (e >= 0 && e < E) yacc = fmaf(pk, part, yacc);
    if (c_k == K - 1) {
      // the row set is done: sum each row over its LPR lanes, write y
      float v = yacc;
      for (int m = 1; m < LPR; m <<= 1) v += __shfl_xor(v, m, 64);
      const int row = c_rs * RPW + h;
      if (jl == 0 && row < O) {
        const float r = shq[pos] + v;
        if constexpr (XF32) static_cast<float*>(y)[row] = r;
        else static_cast<uint16_t*>(y)[row] = f32_to_bf16_rne(r);
      }
      yacc = 0.f;
    }
    c_q++;
    if (++c_k == K) c_k = 0, c_rs++;
  };

  for (int base = 0; base < nslot; base += kRing) {
#pragma unroll
    for (int s = 0; s < kRing; s++) {
      __builtin_amdgcn_sched_barrier(0);
      consume(s);
      issue(s);
    }
  }
}

// Lanes per row (as log2) and groups per lane for G groups: the layout with
// the fewest idle lane-groups among NG <= kMaxNG, the narrower rows (more
// rows per wave) on a tie; -1 when G is too large.
struct OnePlan {
  int lpr_log2, ng;
};
OnePlan one_plan(int G) {
  OnePlan best{-1, 0};
  int best_waste = 1 << 30;
  for (int l2 = 6; l2 >= 0; l2--) {
    const int lpr = 1 << l2, ng = (G + lpr - 1) / lpr;
    if (ng > kMaxNG) continue;
    const int waste = ng * lpr - G;
    if (waste <= best_waste) best = OnePlan{l2, ng}, best_waste = waste;
  }
  return best;
}

template <bool XF32, int NG>
hipError_t launch_ng(const OnePlan& pl, const void* x, const uint8_t* packed, const uint8_t* scales,
                     const int32_t* sel, const float* p, const void* shared, void* y, int E, int O, int G, int K,
                     int32_t* n_invalid, int n_cu, hipStream_t stream) {
  const int rpw = 64 >> pl.lpr_log2;
  const int n_rs = (O + rpw - 1) / rpw;
  const int64_t want = (n_rs + kWaves - 1) / kWaves;
  const int64_t cap = (int64_t)n_cu * MXFP4_DECODE1_WG_PER_CU;
  const int nwg = (int)(want < cap ? want : cap);
  const size_t lds = (size_t)G * ((XF32 ? 8 : 4) * 16 + 16);
  hipLaunchKernelGGL((gemv_one_kernel<XF32, NG>), dim3(nwg), dim3(kWaves * 64), lds, stream, x, packed, scales, sel,
                     p, shared, y, E, O, G, K, pl.lpr_log2, n_rs, n_invalid);
  return hipGetLastError();
}

template <bool XF32>
hipError_t launch_dt(const OnePlan& pl, const void* x, const uint8_t* packed, const uint8_t* scales,
                     const int32_t* sel, const float* p, const void* shared, void* y, int E, int O, int G, int K,
                     int32_t* n_invalid, int n_cu, hipStream_t stream) {
  switch (pl.ng) {
    case 1: return launch_ng<XF32, 1>(pl, x, packed, scales, sel, p, shared, y, E, O, G, K, n_invalid, n_cu, stream);
    case 2: return launch_ng<XF32, 2>(pl, x, packed, scales, sel, p, shared, y, E, O, G, K, n_invalid, n_cu, stream);
    case 3: return launch_ng<XF32, 3>(pl, x, packed, scales, sel, p, shared, y, E, O, G, K, n_invalid, n_cu, stream);
    default: return launch_ng<XF32, 4>(pl, x, packed, scales, sel, p, shared, y, E, O, G, K, n_invalid, n_cu, stream);
  }
}

}  // namespace

bool gemv_one_supported(int O, int G, int K) {
  return K <= kMaxFusedPairs && one_plan(G).lpr_log2 >= 0 && (int64_t)O * G * 16 < ((int64_t)1 << 31);
}

hipError_t launch_gemv_one(const void* x, const uint8_t* packed, const uint8_t* scales, const int32_t* sel,
                           const float* p, const void* shared, void* y, int E, int O, int G, int K, int dtype,
                           int32_t* n_invalid, int n_cu, hipStream_t stream) {
  if (!gemv_one_supported(O, G, K) || n_cu < 1) return hipErrorInvalidValue;
  const OnePlan pl = one_plan(G);
  return dtype == 0 ? launch_dt<true>(pl, x, packed, scales, sel, p, shared, y, E, O, G, K, n_invalid, n_cu, stream)
                    : launch_dt<false>(pl, x, packed, scales, sel, p, shared, y, E, O, G, K, n_invalid, n_cu, stream);
}

}  // namespace mxfp4
