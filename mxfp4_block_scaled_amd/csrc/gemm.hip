// Prefill-shaped path: grouped GEMM over the expert segments made by the
// bucketing, on bf16 MFMA with fp32 accumulation.
//
// For an M-tile of expert e (sorted positions row0 .. row0+mlen-1) and an
// N-tile of output features n0 .. n0+127, the workgroup computes
//     part[row0 + m, n] = sum_i x[token(perm[row0 + m]), i] * W_e[n, i]
// (page "MXFP4 Routed Expert Linear", "Reconstruct the matrix in the right
// orientation": each output coordinate is a row of W_e dotted with the
// token). Per K-stage of two groups (64 inputs) the workgroup stages in LDS
// the gathered bf16 token rows (128 x 64) and the raw packed bytes of its
// 128 weight rows. Scale bytes go to LDS in chunks of 16 groups (8 stages),
// each row's 16 bytes with a few dword loads, prefetched a chunk ahead
// (one byte per lane per stage would touch a cache line per row per stage);
// every wave then decodes its own weight
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
// tiles. A wave whose 64 rows hold no pair skips its MFMAs; otherwise both
// of its 32-row sub-tiles run, so the stage body has no branch and its LDS
// reads (one k-step ahead), converts and MFMAs interleave. Loads of the
// next stage overlap the MFMAs of the current one.
//
// fp32 activations (NP = 3): the host splits every value exactly into three
// bf16 pieces, x = x0 + x1 + x2 (each piece the top 8 significant bits of
// what is left), stored as three planes of the activation array. The kernel
// stages all three and multiplies each decoded weight fragment by each piece
// into one fp32 accumulator: every product is exact. To keep the fp32 sum
// of I = 32G products within the fp32 bar for outputs near zero, the MFMA
// accumulator holds only the sum of one chunk of 128 inputs (two stages) and
// is then added into a running (hi, lo) pair with an error-free TwoSum
// (Knuth: s = hi + a, e = (hi - (s - (s - hi))) + (a - (s - hi))), so the
// error is that of the short chunk sums.
//
// Large scale bytes. E2M1 * 2^(s-127) exceeds the bf16 range for s >= 253
// (|code value| >= 4 at 253, >= 2 at 254, >= 1 at 255), while the layer's
// value stays finite. A wave that meets such a scale byte (a wave-uniform
// test, never true on ordinary data) switches for the rest of its tile to
// decoding every group at scale byte s - 3 (0 for s < 3) and multiplies its
// accumulators by 2^-3 once; at the end it multiplies them by 2^3. Power of
// two scaling commutes with the exact products and the fp32 sums, so the
// result is the exact layer's up to fp32 rounding, as on the decode-shaped
// path; the only approximation is in a tile that mixes such bytes with scale
// bytes 0..2, whose weights (below 2^-121 in magnitude) are read at 2^-124.
#include <algorithm>

#include "device_common.h"
#include "launch.h"

namespace mxfp4 {
namespace {

constexpr int MT = kGemmTileM;
constexpr int NT = kGemmTileN;
constexpr int A_LD = 64 + 8;  // bf16 elements per LDS row (144 B: conflict-free 16-B reads)
constexpr int B_LD = 48;      // bytes per LDS row of packed weights (32 used)
constexpr int kRsrcFlags = 0x00020000;        // raw buffer, 32-bit data format
constexpr uint32_t kOobByte = 0x80000000u;    // byte offset past the activation and weight resources
constexpr int kScGroups = 16;                   // scale bytes per row and chunk
constexpr int kScStages = kScGroups / 2;        // stages per chunk
constexpr int kScPitch = 5;                     // dwords per LDS row of a chunk (16 bytes at offset 0..3)
constexpr int kScSlots = (kGemmTileN * kScPitch + 255) / 256;
constexpr uint32_t kShiftFrom = 253;  // scale bytes whose decoded weights may overflow bf16
constexpr uint32_t kShift = 3;        // scale-byte shift of a wave that met one
static_assert(kGemmTileN * kScPitch <= 1020, "q / 5 by multiply-shift");

// What the kernel's rows and columns are:
//  kGather: A rows are the tokens of the tile's pairs (perm / K), the
//           128 columns are weight rows n0 .. n0+127, output fp32 part rows.
//  kSwiGLU: A rows as kGather; the weight matrix stacks gate (rows [0, F))
//           over up (rows [F, 2F)), and the tile's 128 columns are the gate
//           and up rows of 64 features f0 .. f0+63 arranged so that each
//           lane's two 32-column MFMA tiles hold the gate and the up value
//           of the same feature; the epilogue writes bf16
//           h[row, f] = silu(gate) * up (page "MoE Expert Kernels: Grouped
//           Prefill and Mixed-Quant Compact Experts", section 1).
//  kDirect: A rows are the sorted positions themselves (rows of h), output
//           fp32 part rows.
enum GemmMode { kGather = 0, kSwiGLU = 1, kDirect = 2 };

template <int MODE, int NP>
__global__ void __launch_bounds__(256, NP == 1 ? 3 : 1) gemm_bf16_kernel(const uint16_t* __restrict__ x,
                                                           const uint8_t* __restrict__ packed,
                                                           const uint8_t* __restrict__ scales,
                                                           const int32_t* __restrict__ perm,
                                                           const GemmTile* __restrict__ tiles,
                                                           const int32_t* __restrict__ n_tiles, void* __restrict__ out,
                                                           int K, int O, int G, int n_ntiles, uint32_t x_bytes, int F,
                                                           uint32_t plane_bytes) {
  const int ti = blockIdx.x / n_ntiles;
  const int nt = blockIdx.x - ti * n_ntiles;
  if (ti >= n_tiles[0]) return;
  const GemmTile tl = tiles[ti];
  const int n0 = nt * NT;           // kGather / kDirect: first weight row of the tile
  const int f0 = nt * (NT / 2);     // kSwiGLU: first feature of the tile
  // weight row of LDS row r of the tile (-1: none)
  auto wrow = [&](int r) -> int {
    if constexpr (MODE == kSwiGLU) {
      const int f = f0 + 32 * (r >> 6) + (r & 31);
      return f < F ? (((r >> 5) & 1) ? F + f : f) : -1;
    } else {
      return n0 + r < O ? n0 + r : -1;
    }
  };

  __shared__ __attribute__((aligned(16))) uint16_t As[2][NP][MT * A_LD];
  __shared__ __attribute__((aligned(16))) uint8_t Bs[2][NT * B_LD];
  __shared__ __attribute__((aligned(16))) uint32_t Sc[NT * kScPitch];  // scale chunk: row r at dword kScPitch r

  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int lm = lane & 31, lq = lane >> 5;
  const int wm = w >> 1, wn = w & 1;

  // A loader: rows (tid >> 3) + 32 i, 16-byte column tid & 7 of the stage slice
  // activations through a buffer resource: 32-bit byte offsets, an invalid
  // row gets an offset past the resource (zeros, no memory traffic)
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc((void*)x, (short)0, (int)x_bytes, kRsrcFlags);
  uint32_t a_off[4];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int m = (tid >> 3) + 32 * i;
    const int arow = m < tl.mlen ? (MODE == kDirect ? tl.row0 + m : perm[tl.row0 + m] / K) : -1;
    a_off[i] = arow >= 0 ? (uint32_t)arow * (uint32_t)(64 * G) + 16u * (tid & 7) : kOobByte;
  }
  // B loader: LDS row tid >> 1, group (tid & 1) of the stage
  const int bn = wrow(tid >> 1);
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(packed + (int64_t)tl.e * O * G * 16), (short)0, O * G * 16, kRsrcFlags);
  const uint32_t b_off = bn >= 0 ? ((uint32_t)bn * (uint32_t)G + (uint32_t)(tid & 1)) * 16u : kOobByte;
  // Scale chunk loader: thread slot i covers (LDS row, dword) = ((tid + 256 i) / 5, (tid + 256 i) % 5)
  // of the chunk; the 16 bytes of chunk c of weight row w start at byte w G + 16 c of the expert's
  // scales and are read from the dword boundary below (the first byte sits at offset (w G) & 3 of
  // the LDS row, counted from that boundary).
  const uintptr_t s_first = reinterpret_cast<uintptr_t>(scales) + (uintptr_t)((int64_t)tl.e * O * G);
  const uint32_t* s_al = reinterpret_cast<const uint32_t*>(s_first & ~(uintptr_t)3);  // wave-uniform
  const int s_mis = (int)(s_first & 3);
  // the expert's scale bytes from the dword boundary below them, whole dwords
  const __amdgpu_buffer_rsrc_t rsa =
      __builtin_amdgcn_make_buffer_rsrc((void*)s_al, (short)0, (s_mis + O * G + 3) & ~3, kRsrcFlags);
  const int nchunk = (G + kScGroups - 1) / kScGroups;
  uint32_t sreg[kScSlots];
  auto sc_load = [&](int c) {
    const int len = min(kScGroups, G - kScGroups * c);
#pragma unroll
    for (int i = 0; i < kScSlots; i++) {
      const int q = tid + 256 * i, r = (q * 205) >> 10, k = q - r * kScPitch;  // q / 5 for q < 1020
      const int w = q < NT * kScPitch ? wrow(r) : -1;
      const int a = s_mis + w * G + kScGroups * c;  // byte offset from s_al
      // a buffer load (not a flat one) so that the compiler's wait counts stay
      // exact; a dword with none of the chunk's bytes reads past the resource
      const bool need = w >= 0 && 4 * k < (a & 3) + len;
      sreg[i] = __builtin_amdgcn_raw_buffer_load_b32(rsa, (int)(need ? (uint32_t)((a >> 2) + k) * 4u : kOobByte), 0,
                                                     0);
    }
  };
  auto sc_store = [&]() {
#pragma unroll
    for (int i = 0; i < kScSlots; i++) {
      const int q = tid + 256 * i;
      if (q < NT * kScPitch) Sc[q] = sreg[i];  // rows without a weight row get zeros (their weights are zero)
    }
  };
  // this lane's two weight rows: first byte offset of their chunk rows in Sc
  int s_row[2];
#pragma unroll
  for (int nj = 0; nj < 2; nj++) {
    const int nl = 64 * wn + 32 * nj + lm;
    const int w = wrow(nl);
    s_row[nj] = 4 * kScPitch * nl + (w >= 0 ? (s_mis + w * G) & 3 : 0);
  }
  const uint8_t* scb = reinterpret_cast<const uint8_t*>(Sc);

  u32x4 ra[NP][4], rb;
  auto gload = [&](int st) {
    const int g0 = 2 * st;
    // past G: the sign bit of G - 1 - group moves the offset past the resource
    const uint32_t past = (uint32_t)(G - 1 - (g0 + ((tid & 7) >> 2))) >> 31 << 31;
#pragma unroll
    for (int pc = 0; pc < NP; pc++)
#pragma unroll
      for (int i = 0; i < 4; i++)
        ra[pc][i] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, (int)((a_off[i] + plane_bytes * pc + 128u * st) | past), 0, 0));
    const uint32_t bpast = (uint32_t)(G - 1 - (g0 + (tid & 1))) >> 31 << 31;
    rb = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, (int)((b_off + 32u * st) | bpast), 0, 0));
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int pc = 0; pc < NP; pc++)
#pragma unroll
      for (int i = 0; i < 4; i++)
        *reinterpret_cast<u32x4*>(&As[buf][pc][((tid >> 3) + 32 * i) * A_LD + (tid & 7) * 8]) = ra[pc][i];
    *reinterpret_cast<u32x4*>(&Bs[buf][(tid >> 1) * B_LD + (tid & 1) * 16]) = rb;
  };

  f32x16 acc[2][2];
  f32x16 hi[NP == 3 ? 2 : 1][2], lo[NP == 3 ? 2 : 1][2];  // fp32 activations: the compensated total
#pragma unroll
  for (int a = 0; a < 2; a++)
#pragma unroll
    for (int b = 0; b < 2; b++) acc[a][b] = f32x16{};
  if constexpr (NP == 3) {
#pragma unroll
    for (int a = 0; a < 2; a++)
#pragma unroll
      for (int b = 0; b < 2; b++) hi[a][b] = lo[a][b] = f32x16{};
  }
  // fp32 activations: add the chunk sums to (hi, lo) without rounding error, restart the chunk
  auto fold = [&]() {
    if constexpr (NP == 3) {
#pragma unroll
      for (int a = 0; a < 2; a++)
#pragma unroll
        for (int b = 0; b < 2; b++) {
          const f32x16 sum = hi[a][b] + acc[a][b];
          const f32x16 bp = sum - hi[a][b];
          lo[a][b] += (hi[a][b] - (sum - bp)) + (acc[a][b] - bp);
          hi[a][b] = sum;
          acc[a][b] = f32x16{};
        }
    }
  };

  bool shifted = false;  // wave-uniform: decoding at scale byte s - kShift
  const int nst = (G + 1) / 2;
  gload(0);
  sc_load(0);
  sstore(0);
  sc_store();
  __syncthreads();
  for (int st = 0; st < nst; st++) {
    const int buf = st & 1;
    const int sst = st % kScStages;  // stage within the scale chunk
    if (st + 1 < nst) gload(st + 1);
    if (sst == 0 && st / kScStages + 1 < nchunk) sc_load(st / kScStages + 1);
    u32x4 wv[2];
    uint32_t sb[2];
#pragma unroll
    for (int nj = 0; nj < 2; nj++) {
      const int nl = 64 * wn + 32 * nj + lm;
      wv[nj] = *reinterpret_cast<const u32x4*>(&Bs[buf][nl * B_LD + lq * 16]);
      // a group past G (odd G, last stage) has zero weights; its byte is unused
      sb[nj] = scb[s_row[nj] + 2 * sst + lq];
    }
    // a scale byte from kShiftFrom up anywhere in the wave (never on ordinary data)
    if (!shifted && __ballot(sb[0] >= kShiftFrom || sb[1] >= kShiftFrom) != 0) {
      shifted = true;
#pragma unroll
      for (int a = 0; a < 2; a++)
#pragma unroll
        for (int b = 0; b < 2; b++) {
          acc[a][b] *= 0.125f;
          if constexpr (NP == 3) {
            hi[a][b] *= 0.125f;
            lo[a][b] *= 0.125f;
          }
        }
    }
    float sc[2];
#pragma unroll
    for (int nj = 0; nj < 2; nj++)
      sc[nj] = e8m0_operand(!shifted ? sb[nj] : (sb[nj] > kShift ? sb[nj] - kShift : 0u));
    // A wave whose rows hold no pair skips the MFMAs; otherwise both of its
    // 32-row sub-tiles run (rows past the segment hold zeros), so the body
    // has no branch and its LDS reads, converts and MFMAs interleave: the A
    // fragments are read one k-step ahead, and a scheduling barrier between
    // k-steps keeps the compiler from hoisting the whole stage's reads.
    if (64 * wm < tl.mlen) {
      auto aload = [&](int j, int mi, int pc) {
        const int ml = 64 * wm + 32 * mi + lm;
        return *reinterpret_cast<const u32x4*>(&As[buf][pc][ml * A_LD + lq * 32 + j * 8]);
      };
      u32x4 av[2][2][NP];
#pragma unroll
      for (int mi = 0; mi < 2; mi++)
#pragma unroll
        for (int pc = 0; pc < NP; pc++) av[0][mi][pc] = aload(0, mi, pc);
#pragma unroll
      for (int j = 0; j < 4; j++) {
        if (j + 1 < 4) {
#pragma unroll
          for (int mi = 0; mi < 2; mi++)
#pragma unroll
            for (int pc = 0; pc < NP; pc++) av[(j + 1) & 1][mi][pc] = aload(j + 1, mi, pc);
        }
        bf16x8 bw[2];
#pragma unroll
        for (int nj = 0; nj < 2; nj++) bw[nj] = decode8_bf16x8(wv[nj][j], sc[nj]);
#pragma unroll
        for (int mi = 0; mi < 2; mi++)
#pragma unroll
          for (int pc = 0; pc < NP; pc++)
#pragma unroll
            for (int nj = 0; nj < 2; nj++)
              acc[mi][nj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av[j & 1][mi][pc]),
                                                                    bw[nj], acc[mi][nj], 0, 0, 0);
#ifndef MXFP4_GEMM_NO_SCHED_BARRIER
        __builtin_amdgcn_sched_barrier(0);
#endif
      }
    }
    if (NP == 3 && ((st & 1) || st + 1 == nst)) fold();
    if (st + 1 < nst) sstore(buf ^ 1);
    __syncthreads();
    if (sst == kScStages - 1 && st + 1 < nst) {  // every wave is past the chunk's last stage
      sc_store();
      __syncthreads();
    }
  }
  if constexpr (NP == 3) {
#pragma unroll
    for (int a = 0; a < 2; a++)
#pragma unroll
      for (int b = 0; b < 2; b++) acc[a][b] = hi[a][b] + lo[a][b];
  }
  if (shifted) {
#pragma unroll
    for (int a = 0; a < 2; a++)
#pragma unroll
      for (int b = 0; b < 2; b++) acc[a][b] *= 8.0f;
  }
  // D layout of the 32x32 MFMA: element i of lane l is row 8(i/4) + 4(l/32) + i%4, column l%32.
  if constexpr (MODE == kSwiGLU) {
    // acc[mi][0] holds the gate and acc[mi][1] the up value of feature f, at the same places
    const int f = f0 + 32 * wn + lm;
    if (f < F) {
      uint16_t* h = static_cast<uint16_t*>(out);
#pragma unroll
      for (int mi = 0; mi < 2; mi++) {
#pragma unroll
        for (int i = 0; i < 16; i++) {
          const int m = 64 * wm + 32 * mi + 8 * (i >> 2) + 4 * lq + (i & 3);
          if (m < tl.mlen) {
            const float g = acc[mi][0][i], u = acc[mi][1][i];
            h[(int64_t)(tl.row0 + m) * F + f] = f32_to_bf16_rne(g / (1.0f + __expf(-g)) * u);
          }
        }
      }
    }
  } else {
    float* part = static_cast<float*>(out);
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
}


}  // namespace

bool gemm_supported(int64_t T, int64_t O, int64_t G, int np) {
  // 32-bit byte offsets into the activations (np planes) and into one expert's packed bytes
  return np * T * 64 * G < ((int64_t)1 << 31) && O * G * 16 < ((int64_t)1 << 31);
}

namespace {
template <int MODE, int NP>
hipError_t launch_mode(const uint16_t* x, const uint8_t* packed, const uint8_t* scales, const int32_t* perm,
                       const GemmTile* tiles, const int32_t* n_tiles, int64_t max_tiles, void* out, int64_t x_rows,
                       int K, int O, int G, int F, int n_ntiles, hipStream_t stream) {
  if (!gemm_supported(x_rows, O, G, NP)) return hipErrorInvalidValue;
  const int64_t nblk = max_tiles * n_ntiles;
  if (nblk <= 0) return hipSuccess;
  const uint32_t plane = (uint32_t)(x_rows * 64 * G);
  hipLaunchKernelGGL((gemm_bf16_kernel<MODE, NP>), dim3((unsigned)nblk), dim3(256), 0, stream, x, packed, scales, perm,
                     tiles, n_tiles, out, K, O, G, n_ntiles, NP * plane, F, plane);
  return hipGetLastError();
}

// fp32 activations -> three bf16 planes (plane j holds piece j of every
// value), four values per thread
__global__ void __launch_bounds__(256) split3_kernel(const u32x4* __restrict__ x, uint32_t* __restrict__ xs,
                                                     int64_t n4) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
    const u32x4 v = x[i];
    uint32_t b[3][4];
#pragma unroll
    for (int c = 0; c < 4; c++) split3(__uint_as_float(v[c]), b[0][c], b[1][c], b[2][c]);
#pragma unroll
    for (int pc = 0; pc < 3; pc++) {
      uint32_t* dst = xs + 2 * (pc * n4 + i);
      dst[0] = b[pc][0] | (b[pc][1] << 16);
      dst[1] = b[pc][2] | (b[pc][3] << 16);
    }
  }
}
}  // namespace

hipError_t launch_gemm_bf16(const uint16_t* x, const uint8_t* packed, const uint8_t* scales, const int32_t* perm,
                            const GemmTile* tiles, const int32_t* n_tiles, int64_t max_tiles, float* part, int T, int K,
                            int O, int G, hipStream_t stream) {
  return launch_mode<kGather, 1>(x, packed, scales, perm, tiles, n_tiles, max_tiles, part, T, K, O, G, 0,
                                 (O + NT - 1) / NT, stream);
}

hipError_t launch_split3(const float* x, int64_t n, uint16_t* xs, hipStream_t stream) {
  if (n % 4 != 0) return hipErrorInvalidValue;
  const int64_t n4 = n / 4;
  if (n4 == 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((n4 + 255) / 256, 4096);
  hipLaunchKernelGGL(split3_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, reinterpret_cast<const u32x4*>(x),
                     reinterpret_cast<uint32_t*>(xs), n4);
  return hipGetLastError();
}

hipError_t launch_gemm_f32(const uint16_t* xs, const uint8_t* packed, const uint8_t* scales, const int32_t* perm,
                           const GemmTile* tiles, const int32_t* n_tiles, int64_t max_tiles, float* part, int T, int K,
                           int O, int G, hipStream_t stream) {
  return launch_mode<kGather, 3>(xs, packed, scales, perm, tiles, n_tiles, max_tiles, part, T, K, O, G, 0,
                                 (O + NT - 1) / NT, stream);
}

hipError_t launch_gemm_swiglu(const uint16_t* x, const uint8_t* gu_packed, const uint8_t* gu_scales,
                              const int32_t* perm, const GemmTile* tiles, const int32_t* n_tiles, int64_t max_tiles,
                              uint16_t* h, int T, int K, int F, int G, hipStream_t stream) {
  return launch_mode<kSwiGLU, 1>(x, gu_packed, gu_scales, perm, tiles, n_tiles, max_tiles, h, T, K, 2 * F, G, F,
                                 (F + NT / 2 - 1) / (NT / 2), stream);
}

hipError_t launch_gemm_direct(const uint16_t* h, const uint8_t* packed, const uint8_t* scales, const GemmTile* tiles,
                              const int32_t* n_tiles, int64_t max_tiles, float* part, int64_t P, int O, int G,
                              hipStream_t stream) {
  return launch_mode<kDirect, 1>(h, packed, scales, nullptr, tiles, n_tiles, max_tiles, part, P, 1, O, G, 0,
                                 (O + NT - 1) / NT, stream);
}

}  // namespace mxfp4
