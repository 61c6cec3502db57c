// Prefill-shaped path: grouped GEMM over the expert segments made by the
// bucketing, on bf16 MFMA with fp32 accumulation.
//
// For an M-tile of expert e (sorted positions row0 .. row0+mlen-1) and an
// N-tile of output features n0 .. n0+127, the workgroup computes
//     part[row0 + m, n] = sum_i x[token(perm[row0 + m]), i] * W_e[n, i]
// (page "MXFP4 Routed Expert Linear", "Reconstruct the matrix in the right
// orientation": each output coordinate is a row of W_e dotted with the
// token). Per K-stage of two groups (64 inputs) the workgroup stages in LDS
// the gathered bf16 token rows (128 x 64) and the raw packed bytes and scale
// bytes of its 128 weight rows; every wave then decodes its own weight
// fragments from LDS straight into MFMA operand registers (exact in bf16:
// every E2M1 value times a power of two up to 2^127 is a bf16 value), so no
// decoded weight is ever stored, in LDS or in HBM.
//
// MFMA: v_mfma_f32_32x32x16_bf16, A = token rows (m), B = weights (n).
// Lane (m, q) = (lane & 31, lane >> 5) of MFMA j supplies the 8 inputs
// 32q + 8j .. 32q + 8j + 7 of the stage (group q of the stage, dword j),
// for both operands; this permutes the order of k inside the stage, which
// leaves every product x_i * w_i paired correctly.
// Waves are 2 x 2 over the 128 x 128 tile; each owns 64 x 64 = 2 x 2 MFMA
// tiles (a 32-row sub-tile past the segment's end is skipped). Loads of the
// next stage overlap the MFMAs of the current one.
#include "device_common.h"
#include "launch.h"

namespace mxfp4 {
namespace {

constexpr int MT = kGemmTileM;
constexpr int NT = kGemmTileN;
constexpr int A_LD = 64 + 8;  // bf16 elements per LDS row (144 B: conflict-free 16-B reads)
constexpr int B_LD = 48;      // bytes per LDS row of packed weights (32 used)

__global__ void __launch_bounds__(256, 2) gemm_bf16_kernel(const uint16_t* __restrict__ x,
                                                           const uint8_t* __restrict__ packed,
                                                           const uint8_t* __restrict__ scales,
                                                           const int32_t* __restrict__ perm,
                                                           const GemmTile* __restrict__ tiles,
                                                           const int32_t* __restrict__ n_tiles, float* __restrict__ part,
                                                           int K, int O, int G, int n_ntiles) {
  const int ti = blockIdx.x / n_ntiles;
  const int nt = blockIdx.x - ti * n_ntiles;
  if (ti >= n_tiles[0]) return;
  const GemmTile tl = tiles[ti];
  const int n0 = nt * NT;
  const int64_t I = 32 * (int64_t)G;

  __shared__ __attribute__((aligned(16))) uint16_t As[2][MT * A_LD];
  __shared__ __attribute__((aligned(16))) uint8_t Bs[2][NT * B_LD];
  __shared__ uint8_t Ss[2][NT * 2];

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int lm = lane & 31, lq = lane >> 5;
  const int wm = w >> 1, wn = w & 1;

  // A loader: rows (tid >> 3) + 32 i, 16-byte column tid & 7 of the stage slice
  const uint16_t* arow[4];
  bool aok[4];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int m = (tid >> 3) + 32 * i;
    aok[i] = m < tl.mlen;
    const int pr = aok[i] ? perm[tl.row0 + m] : 0;
    arow[i] = x + (int64_t)(pr / K) * I + (tid & 7) * 8;
  }
  // B loader: row tid >> 1, group (tid & 1) of the stage
  const int bn = n0 + (tid >> 1);
  const bool bok = bn < O;
  const uint8_t* brow = packed + ((int64_t)tl.e * O + (bok ? bn : 0)) * (int64_t)G * 16 + (tid & 1) * 16;
  const uint8_t* srow = scales + ((int64_t)tl.e * O + (bok ? bn : 0)) * (int64_t)G + (tid & 1);

  u32x4 ra[4], rb;
  uint32_t rs;
  auto gload = [&](int st) {
    const int g0 = 2 * st;
    const bool ag = g0 + ((tid & 7) >> 2) < G;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      ra[i] = u32x4{0u, 0u, 0u, 0u};
      if (aok[i] && ag) ra[i] = *reinterpret_cast<const u32x4*>(arow[i] + 64 * (int64_t)st);
    }
    const bool bg = g0 + (tid & 1) < G;
    rb = u32x4{0u, 0u, 0u, 0u};
    rs = 127;
    if (bok && bg) {
      rb = *reinterpret_cast<const u32x4*>(brow + (int64_t)g0 * 16);
      rs = srow[g0];
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; i++)
      *reinterpret_cast<u32x4*>(&As[buf][((tid >> 3) + 32 * i) * A_LD + (tid & 7) * 8]) = ra[i];
    *reinterpret_cast<u32x4*>(&Bs[buf][(tid >> 1) * B_LD + (tid & 1) * 16]) = rb;
    Ss[buf][(tid >> 1) * 2 + (tid & 1)] = (uint8_t)rs;
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; a++)
#pragma unroll
    for (int b = 0; b < 2; b++) acc[a][b] = f32x16{};

  const int nst = (G + 1) / 2;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int st = 0; st < nst; st++) {
    const int buf = st & 1;
    if (st + 1 < nst) gload(st + 1);
    uint32_t bw[2][4][4];
#pragma unroll
    for (int nj = 0; nj < 2; nj++) {
      const int nl = 64 * wn + 32 * nj + lm;
      const u32x4 wv = *reinterpret_cast<const u32x4*>(&Bs[buf][nl * B_LD + lq * 16]);
      const uint32_t s = Ss[buf][nl * 2 + lq];
      if (__builtin_expect(__ballot(s == 255) != 0, 0)) {
#pragma unroll
        for (int j = 0; j < 4; j++) {
          if (s == 255) decode8_bf16_slow(wv[j], s, bw[nj][j]);
          else decode8_bf16_fast(wv[j], e8m0_operand(s), bw[nj][j]);
        }
      } else {
        const float sc = e8m0_operand(s);
#pragma unroll
        for (int j = 0; j < 4; j++) decode8_bf16_fast(wv[j], sc, bw[nj][j]);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; j++) {
#pragma unroll
      for (int mi = 0; mi < 2; mi++) {
        if (64 * wm + 32 * mi >= tl.mlen) continue;  // a 32-row sub-tile past the segment
        const int ml = 64 * wm + 32 * mi + lm;
        const u32x4 av = *reinterpret_cast<const u32x4*>(&As[buf][ml * A_LD + lq * 32 + j * 8]);
#pragma unroll
        for (int nj = 0; nj < 2; nj++) {
          const u32x4 bv = {bw[nj][j][0], bw[nj][j][1], bw[nj][j][2], bw[nj][j][3]};
          acc[mi][nj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av),
                                                                __builtin_bit_cast(bf16x8, bv), acc[mi][nj], 0, 0, 0);
        }
      }
    }
    if (st + 1 < nst) sstore(buf ^ 1);
    __syncthreads();
  }
  // D layout of the 32x32 MFMA: element i of lane l is row 8(i/4) + 4(l/32) + i%4, column l%32.
#pragma unroll
  for (int mi = 0; mi < 2; mi++) {
#pragma unroll
    for (int nj = 0; nj < 2; nj++) {
      const int n = n0 + 64 * wn + 32 * nj + lm;
      if (n >= O) continue;
#pragma unroll
      for (int i = 0; i < 16; i++) {
        const int m = 64 * wm + 32 * mi + 8 * (i >> 2) + 4 * lq + (i & 3);
        if (m < tl.mlen) part[(int64_t)(tl.row0 + m) * O + n] = acc[mi][nj][i];
      }
    }
  }
}


}  // namespace

hipError_t launch_gemm_bf16(const uint16_t* x, const uint8_t* packed, const uint8_t* scales, const int32_t* perm,
                            const GemmTile* tiles, const int32_t* n_tiles, int64_t max_tiles, float* part, int T, int K,
                            int O, int G, hipStream_t stream) {
  (void)T;
  const int n_ntiles = (O + NT - 1) / NT;
  const int64_t nblk = max_tiles * n_ntiles;
  if (nblk <= 0) return hipSuccess;
  hipLaunchKernelGGL(gemm_bf16_kernel, dim3((unsigned)nblk), dim3(256), 0, stream, x, packed, scales, perm, tiles,
                     n_tiles, part, K, O, G, n_ntiles);
  return hipGetLastError();
}

}  // namespace mxfp4
