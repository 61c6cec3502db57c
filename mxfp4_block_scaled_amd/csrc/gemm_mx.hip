// Block-scaled variant of the prefill-shaped path: the activations are
// quantised to MXFP8 (E4M3 codes, one E8M0 scale byte per token and block of
// 32 inputs) and gfx950's v_mfma_scale_f32_16x16x128_f8f6f4 multiplies them
// by the packed E2M1 weights and their E8M0 scale bytes exactly as stored:
// no weight is decoded by the vector ALUs. MXFP4 and MXFP8 are members of
// the OCP Microscaling family, blocks of 32 codes sharing one E8M0 scale
// (page "MXFP4 Dequant", "Overview"); the activation readings (E4M3 with
// bias 7 and 448 as largest value, the smallest power-of-two scale that fits
// the block maximum, round to nearest even, the block = weight group's 32
// inputs) are the oracle's.
//
// Quantisation (quant_mxfp8_kernel): 8 lanes per block of 32, four inputs a
// lane, the block maximum by three DPP steps; every step is exact in fp32
// (power-of-two scaling, a round-to-nearest-even to the E4M3 grid, bit
// assembly of the code), so the codes equal the oracle's bit for bit.
//
// Grouped GEMM (gemm_mx_kernel): the M-tiles of the bucketing (<= 128 pairs
// of one expert) x N-tiles of 128 features; 2 x 2 waves of 64 x 64. MFMA
// operand A = weights: lane (r, c) = (lane & 15, lane >> 4) holds the 16
// packed bytes of group 4q + c of weight row r of its 16-row fragment (one
// 16-byte load straight from memory into the operand registers) and that
// group's scale byte. Operand B = activations: lane (p, c) holds E4M3 codes
// 16c .. 16c+15 and 64+16c .. 64+16c+15 of the chunk for pair p, and the
// scale byte of block 4q + c (the hardware applies the scale of lane group c
// to inputs 32c .. 32c+31 of both operands). Activation rows are gathered
// (row = perm / K; each wave-wide request reads eight whole 128-byte row
// pieces) into LDS once per workgroup and chunk (144-byte rows:
// conflict-free 16-byte reads), double-buffered with one barrier a chunk
// and fetched two chunks ahead (held a chunk in registers before the LDS
// store); weights and their scales are loaded three chunks ahead into a
// ring of four register slots. Groups
// past G and rows past O read through an offset beyond the buffer resource
// (zeros). Output: fp32 rows of `part` at sorted positions, as the bf16 GEMM.
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace mxfp4 {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kRsrcFlags = 0x00020000;
constexpr uint32_t kOob = 0x80000000u;
constexpr int MT = kGemmTileM;  // 128 pairs
constexpr int NT = 128;         // features
constexpr int KC = 128;         // inputs per chunk
constexpr int kPitch = KC + 16; // bytes per LDS activation row
constexpr int kWRing = 4;       // weight chunks held in registers: three in flight while one is used

// ---- quantisation

__device__ __forceinline__ uint32_t e4m3_code(float v) {
  // v = x / 2^X with |v| <= 448 by the choice of X
  const float a = fabsf(v);
  const int ea = (int)(__float_as_uint(a) >> 23) - 127;  // floor(log2 a); -127 for 0 and subnormals
  const int eq = ea > -6 ? ea : -6;
  const float n = rintf(a * __uint_as_float((uint32_t)(127 + 3 - eq) << 23));  // nearest, ties to even
  float aq = n * __uint_as_float((uint32_t)(127 + eq - 3) << 23);
  aq = fminf(aq, 448.0f);
  const uint32_t b = __float_as_uint(aq);
  const uint32_t code = aq < 0.015625f ? (uint32_t)(aq * 512.0f) : ((((b >> 23) - 120u) << 3) | ((b >> 20) & 7u));
  return code;
}

__global__ void __launch_bounds__(256) quant_mxfp8_kernel(const uint16_t* __restrict__ x, int T, int I, int Kp,
                                                          uint8_t* __restrict__ codes, uint8_t* __restrict__ sb) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int nb = Kp / 32;                 // blocks per row
  const int64_t blk = gid >> 3;           // (token, block)
  const int sub = (int)(gid & 7);         // four inputs 4 sub .. 4 sub + 3 of the block
  if (blk >= (int64_t)T * nb) return;     // whole 8-lane groups leave together
  const int t = (int)(blk / nb), jb = (int)(blk - (int64_t)t * nb);
  const int k0 = 32 * jb + 4 * sub;
  uint2 raw = make_uint2(0u, 0u);
  if (32 * jb < I) raw = *reinterpret_cast<const uint2*>(x + (int64_t)t * I + k0);  // I % 32 == 0: whole blocks
  const uint32_t h[4] = {raw.x & 0xFFFFu, raw.x >> 16, raw.y & 0xFFFFu, raw.y >> 16};
  uint32_t amax = 0;  // |x| as bits: bf16 magnitudes order like their bit patterns
#pragma unroll
  for (int i = 0; i < 4; i++) amax = max(amax, h[i] & 0x7FFFu);
  // maximum over the 8 lanes of the block: xor 1, xor 2, then mirror within 8
  amax = max(amax, (uint32_t)__builtin_amdgcn_mov_dpp((int)amax, 0xB1, 0xF, 0xF, false));
  amax = max(amax, (uint32_t)__builtin_amdgcn_mov_dpp((int)amax, 0x4E, 0xF, 0xF, false));
  amax = max(amax, (uint32_t)__builtin_amdgcn_mov_dpp((int)amax, 0x141, 0xF, 0xF, false));
  // X: the smallest exponent with amax <= 448 * 2^X (448 = 1.75 * 2^8), clamped to [-127, 127]
  const uint32_t ab = amax << 16;  // fp32 bits of amax
  const int e = (int)(ab >> 23) - 127;
  int X = (ab & 0x7FFFFFu) <= 0x600000u ? e - 8 : e - 7;
  if ((ab >> 23) == 0) X = -127;  // zero or subnormal block
  X = X < -127 ? -127 : (X > 127 ? 127 : X);
  const float inv = __uint_as_float((uint32_t)(127 - X) << 23);  // 2^-X, X in [-127, 120]
  uint32_t word = 0;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const float v = __uint_as_float(h[i] << 16) * inv;
    word |= (e4m3_code(v) | ((h[i] >> 8) & 0x80u)) << (8 * i);
  }
  *reinterpret_cast<uint32_t*>(codes + (int64_t)t * Kp + k0) = word;
  if (sub == 0) sb[(int64_t)t * nb + jb] = (uint8_t)(X + 127);
}

// ---- grouped GEMM

// PREP: the weights come in the prepared layout of prepare_mx_kernel (one
// contiguous 1 KB block per 16-row fragment and chunk, and a 64-byte block of
// its scales) instead of the canonical [E, O, G, 16] / [E, O, G].
template <bool PREP>
__global__ void __launch_bounds__(256, 2) gemm_mx_kernel(const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs,
                                                         const uint8_t* __restrict__ packed,
                                                         const uint8_t* __restrict__ scales,
                                                         const int32_t* __restrict__ perm,
                                                         const GemmTile* __restrict__ tiles,
                                                         const int32_t* __restrict__ n_tiles, float* __restrict__ part,
                                                         int K, int O, int G, int Kp, int n_ntiles, uint32_t xq_bytes,
                                                         uint32_t xs_bytes) {
  const int ti = blockIdx.x / n_ntiles;
  const int nt = blockIdx.x - ti * n_ntiles;
  if (ti >= n_tiles[0]) return;
  const GemmTile tl = tiles[ti];
  const int f0 = nt * NT;

  __shared__ __attribute__((aligned(16))) uint8_t Xs[2][MT * kPitch];
  __shared__ uint32_t Ss[2][MT];

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int wm = w >> 1, wn = w & 1;
  const int lr = lane & 15, lc = lane >> 4;

  // activation loader: wave w, request j covers pair rows 32 w + 8 j .. +7,
  // eight lanes a row, 16 bytes a lane (the row's 128 bytes of the chunk)
  const int ld_ch = lane & 7;
  uint32_t x_off[4], s_off[4];
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const int m = 32 * w + 8 * j + (lane >> 3);
    const int tok = m < tl.mlen ? perm[tl.row0 + m] / K : -1;
    x_off[j] = tok >= 0 ? (uint32_t)tok * (uint32_t)Kp + 16u * ld_ch : kOob;
    s_off[j] = tok >= 0 ? (uint32_t)tok * (uint32_t)(Kp / 32) : kOob;
  }
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc((void*)xq, (short)0, (int)xq_bytes, kRsrcFlags);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)xs, (short)0, (int)xs_bytes, kRsrcFlags);

  // weight fragments: rows f0 + 64 wn + 16 i + lr, group 4 q + lc
  const int nq = Kp / KC;
  const int64_t ebase = (int64_t)tl.e * O * G;                   // canonical layout
  const int64_t pbase = (int64_t)tl.e * n_ntiles * nq * 512;     // prepared layout: groups before expert e
  const __amdgpu_buffer_rsrc_t rw = PREP
      ? __builtin_amdgcn_make_buffer_rsrc((void*)(packed + pbase * 16), (short)0, n_ntiles * nq * 8192, kRsrcFlags)
      : __builtin_amdgcn_make_buffer_rsrc((void*)(packed + ebase * 16), (short)0, O * G * 16, kRsrcFlags);
  const __amdgpu_buffer_rsrc_t rsc = PREP
      ? __builtin_amdgcn_make_buffer_rsrc((void*)(scales + pbase), (short)0, n_ntiles * nq * 512, kRsrcFlags)
      : __builtin_amdgcn_make_buffer_rsrc((void*)(scales + ebase), (short)0, O * G, kRsrcFlags);
  // a wave whose 64 pairs are all past the tile's end multiplies nothing:
  // its weight requests go past the resource (no memory traffic)
  const bool w_live = 64 * wm < tl.mlen;
  uint32_t w_grp[4];  // canonical: group index (row * G + lc) of chunk 0; prepared: group slot of chunk 0; or kOob
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int f = f0 + 64 * wn + 16 * i + lr;
    if constexpr (PREP)
      w_grp[i] = w_live ? (uint32_t)((nt * nq * 8 + 4 * wn + i) * 64 + lane) : kOob;
    else
      w_grp[i] = (f < O && w_live) ? (uint32_t)f * (uint32_t)G + (uint32_t)lc : kOob;
  }

  u32x4 xa[4];
  uint32_t xsc[4];
  u32x4 wf[kWRing][4];
  uint32_t wsc[kWRing][4];
  auto load_x = [&](int q) {
#pragma unroll
    for (int j = 0; j < 4; j++) {
      xa[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, (int)(x_off[j] + 128u * q), 0, 0));
      xsc[j] = __builtin_amdgcn_raw_buffer_load_b32(rs, (int)(s_off[j] + 4u * q), 0, 0);
    }
  };
  auto load_w = [&](int q, int slot) {
    // canonical: a group past G moves the offset past the resource (the sign
    // bit of G - 1 - group); prepared: padding groups hold zeros, chunk q is
    // 8 fragments x 64 group slots further on
    const uint32_t past = PREP ? 0u : (uint32_t)(G - 1 - (4 * q + lc)) >> 31 << 31;
    const uint32_t step_q = PREP ? 512u : 4u;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const uint32_t g = (w_grp[i] + step_q * q) | past;  // kOob stays past the resource
      wf[slot][i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, (int)(g << 4 | (g & kOob)), 0, 0));
      wsc[slot][i] = __builtin_amdgcn_raw_buffer_load_b8(rsc, (int)g, 0, 0);
    }
  };
  auto store_x = [&](int buf) {
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int m = 32 * w + 8 * j + (lane >> 3);
      *reinterpret_cast<u32x4*>(&Xs[buf][m * kPitch + 16 * ld_ch]) = xa[j];
      Ss[buf][m] = xsc[j];  // the eight lanes of a row write the same dword: no branch
    }
  };

  v4f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // One chunk q; W = q mod 4 (compile-time) is its weight register slot and
  // W mod 2 its LDS buffer, so no register array is indexed at run time.
  // The activations of chunk q + 1 (loaded during chunk q - 1) go to the
  // other LDS buffer first, then chunk q + 2's activations and chunk q + 3's
  // weights are requested (the weights stream from HBM: three chunks in
  // flight cover its latency), then chunk q is multiplied. Past the last
  // chunk the same requests repeat the last chunk (harmless, never read), so
  // that no load or store in the steady state sits behind a branch and the
  // compiler's wait counts stay exact.
  auto step = [&](int q, auto slot) {
    constexpr int W = decltype(slot)::value, S = W & 1;
    store_x(S ^ 1);
    load_x(min(q + 2, nq - 1));
    load_w(min(q + 3, nq - 1), (W + 3) % kWRing);
    __builtin_amdgcn_sched_barrier(0);  // keep the requests ahead of the MFMAs
#pragma unroll
    for (int j = 0; j < 4; j++) {
      if (64 * wm + 16 * j >= tl.mlen) break;  // 16-pair fragments past the tile's end (wave-uniform)
      const int p = 64 * wm + 16 * j + lr;
      const u32x4 lo = *reinterpret_cast<const u32x4*>(&Xs[S][p * kPitch + 16 * lc]);
      const u32x4 hi = *reinterpret_cast<const u32x4*>(&Xs[S][p * kPitch + 64 + 16 * lc]);
      const v8i bf = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      const int bs = (int)((Ss[S][p] >> (8 * lc)) & 0xFFu);
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const v8i a = v8i{(int)wf[W][i][0], (int)wf[W][i][1], (int)wf[W][i][2], (int)wf[W][i][3], 0, 0, 0, 0};
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, bf, acc[i][j], 4, 0, 0, (int)wsc[W][i], 0, bs);
      }
    }
    __syncthreads();
  };
  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;
  using C2 = std::integral_constant<int, 2>;
  using C3 = std::integral_constant<int, 3>;
  load_w(0, 0);
  load_w(min(1, nq - 1), 1);
  load_w(min(2, nq - 1), 2);
  load_x(0);
  store_x(0);
  load_x(min(1, nq - 1));
  __syncthreads();
  int q = 0;
  for (; q + 3 < nq; q += 4) {
    step(q, C0{});
    step(q + 1, C1{});
    step(q + 2, C2{});
    step(q + 3, C3{});
  }
  if (q < nq) step(q, C0{});
  if (q + 1 < nq) step(q + 1, C1{});
  if (q + 2 < nq) step(q + 2, C2{});

  // lane (lr, lc) of fragment (i, j): pair 64 wm + 16 j + lr, features 64 wn + 16 i + 4 lc .. +3
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const int p = 64 * wm + 16 * j + lr;
    if (p >= tl.mlen) continue;
    float* row = part + (int64_t)(tl.row0 + p) * O;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int f = f0 + 64 * wn + 16 * i + 4 * lc;
      if (f < O) *reinterpret_cast<v4f*>(row + f) = acc[i][j];
    }
  }
}

// Prepared layout, per expert e, N-tile n (128 rows), chunk q (4 groups) and
// 16-row fragment f: 64 group slots of 16 bytes (slot l = row 16 f + (l & 15)
// of the tile, group 4 q + (l >> 4): exactly what lane l of the MFMA's A
// operand takes) and, in a second array, their 64 scale bytes in the same
// order. Rows past O and groups past G are zero. One thread per group slot.
__global__ void __launch_bounds__(256) prepare_mx_kernel(const uint8_t* __restrict__ packed,
                                                         const uint8_t* __restrict__ scales, int64_t n_slots, int O,
                                                         int G, int n_ntiles, int nq, uint8_t* __restrict__ pp,
                                                         uint8_t* __restrict__ ps) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= n_slots) return;
  const int l = (int)(idx & 63), fr = (int)((idx >> 6) & 7);
  const int64_t rest = idx >> 9;  // (e * n_ntiles + n) * nq + q
  const int q = (int)(rest % nq);
  const int64_t en = rest / nq;
  const int n = (int)(en % n_ntiles);
  const int64_t e = en / n_ntiles;
  const int row = 128 * n + 16 * fr + (l & 15), g = 4 * q + (l >> 4);
  u32x4 v = u32x4{0u, 0u, 0u, 0u};
  uint8_t sc = 0;
  if (row < O && g < G) {
    const int64_t src = (e * O + row) * G + g;
    v = *reinterpret_cast<const u32x4*>(packed + src * 16);
    sc = scales[src];
  }
  *reinterpret_cast<u32x4*>(pp + idx * 16) = v;
  ps[idx] = sc;
}

}  // namespace

size_t mx_prepared_bytes(int64_t E, int64_t O, int64_t G) {
  const int64_t slots = E * ((O + NT - 1) / NT) * (mx_row_bytes(32 * G) / KC) * 512;
  return (size_t)slots * 17;
}

hipError_t launch_prepare_mx(const uint8_t* packed, const uint8_t* scales, int64_t E, int O, int G, uint8_t* prepared,
                             hipStream_t stream) {
  const int n_ntiles = (O + NT - 1) / NT, nq = mx_row_bytes(32 * (int64_t)G) / KC;
  const int64_t slots = E * n_ntiles * nq * 512;
  if (slots == 0) return hipSuccess;
  hipLaunchKernelGGL(prepare_mx_kernel, dim3((unsigned)((slots + 255) / 256)), dim3(256), 0, stream, packed, scales,
                     slots, O, G, n_ntiles, nq, prepared, prepared + slots * 16);
  return hipGetLastError();
}

int mx_row_bytes(int64_t I) { return (int)(KC * ((I + KC - 1) / KC)); }

bool gemm_mx_supported(int64_t T, int64_t O, int64_t G) {
  const int64_t Kp = mx_row_bytes(32 * G);
  const int64_t per_expert_prepared = ((O + NT - 1) / NT) * (Kp / KC) * 8192;
  return O % 4 == 0 && T * Kp < (int64_t(1) << 31) && O * G * 16 < (int64_t(1) << 31) &&
         per_expert_prepared < (int64_t(1) << 31);
}

hipError_t launch_quant_mxfp8(const uint16_t* x, int T, int I, int Kp, uint8_t* codes, uint8_t* sb,
                              hipStream_t stream) {
  if (I % 32 || Kp % 32 || Kp < I) return hipErrorInvalidValue;
  const int64_t threads = (int64_t)T * (Kp / 32) * 8;
  if (threads == 0) return hipSuccess;
  hipLaunchKernelGGL(quant_mxfp8_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, x, T, I, Kp,
                     codes, sb);
  return hipGetLastError();
}

hipError_t launch_gemm_mx(const uint8_t* xq, const uint8_t* xs, const uint8_t* packed, const uint8_t* scales,
                          const int32_t* perm, const GemmTile* tiles, const int32_t* n_tiles, int64_t max_tiles,
                          float* part, int T, int K, int O, int G, hipStream_t stream, bool prepared) {
  const int Kp = mx_row_bytes(32 * (int64_t)G);
  const int n_ntiles = (O + NT - 1) / NT;
  const int64_t nblk = max_tiles * n_ntiles;
  if (nblk == 0) return hipSuccess;
  const uint32_t xq_bytes = (uint32_t)((int64_t)T * Kp), xs_bytes = (uint32_t)((int64_t)T * Kp / 32);
  if (prepared)
    hipLaunchKernelGGL(gemm_mx_kernel<true>, dim3((unsigned)nblk), dim3(256), 0, stream, xq, xs, packed, scales, perm,
                       tiles, n_tiles, part, K, O, G, Kp, n_ntiles, xq_bytes, xs_bytes);
  else
    hipLaunchKernelGGL(gemm_mx_kernel<false>, dim3((unsigned)nblk), dim3(256), 0, stream, xq, xs, packed, scales, perm,
                       tiles, n_tiles, part, K, O, G, Kp, n_ntiles, xq_bytes, xs_bytes);
  return hipGetLastError();
}

}  // namespace mxfp4
