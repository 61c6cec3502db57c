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
// of one expert) x N-tiles of 512 features; the 8 waves split the features
// (each wave: all 128 pairs x 64 features), so no two waves load the same
// weights, and the activations, shared by all eight, come from LDS once per
// 512 features. MFMA
// operand A = weights: lane (r, c) = (lane & 15, lane >> 4) holds the 16
// packed bytes of group 4q + c of weight row r of its 16-row fragment (one
// 16-byte load straight from memory into the operand registers) and that
// group's scale byte. Operand B = activations: lane (p, c) holds E4M3 codes
// 16c .. 16c+15 and 64+16c .. 64+16c+15 of the chunk for pair p, and the
// scale byte of block 4q + c (the hardware applies the scale of lane group c
// to inputs 32c .. 32c+31 of both operands). Activation rows are gathered
// (row = perm / K) by LDS DMA (buffer loads that write LDS directly, no
// registers) into a ring of three chunk slots, two chunks ahead, each
// wave-wide request filling eight whole 128-byte row pieces; the pieces of a
// row sit XOR-swizzled so that the 16-byte fragment reads are conflict-free
// without padding. Weights go to a ring of three register slots, two chunks
// ahead. Their scale bytes: prepared weights, one dword per lane loaded with
// the weights; canonical weights, by DMA into LDS with the activations (each
// row's bytes of the chunk with the dword boundary below them), read at the
// chunk's start (per-lane byte loads had touched 16 rows' lines per
// instruction). Every chunk issues the same number of requests,
// so one counted wait per chunk (this wave's DMA of the next chunk) and a
// bare barrier replace a full fence. Groups past G and rows past O read
// through an offset beyond the buffer resource (zeros). Output: fp32 rows of
// `part` at sorted positions, as the bf16 GEMM.
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
constexpr int NT = 128;         // rows of a prepared weight tile
constexpr int kWaves = 8;       // waves per workgroup
constexpr int kWI = 4;          // weight fragments (16 features each) per wave: the waves split the features
constexpr int NW = 16 * kWI * kWaves;  // features per workgroup (each wave: all 128 pairs x 64 features)
constexpr int KC = 128;         // inputs per chunk
constexpr int kWJ = 8;           // activation fragments (16 pairs each) per wave: every wave covers all 128 pairs
constexpr int kRing = 3;         // chunk slots: activations (LDS) and weights (registers), two in flight
// canonical weights: the chunk's weight scale bytes (4 groups of the
// workgroup's NW rows, each row's bytes with the dword boundary below them:
// 2 dwords, pitch 8 bytes) come into LDS by DMA with the activations, 2
// requests per wave, followed by zero bytes read for groups past G
constexpr int kWsPitch = 8;
constexpr int kWsWin = NW * kWsPitch;
constexpr int kWsDma = kWsWin / (256 * kWaves);
constexpr int kWsZero = 16 * kWsPitch * kWI;
static_assert(kWsDma * 256 * kWaves == kWsWin, "weight scale DMA");
// vector-memory requests per wave and chunk: (canonical: 2 weight-scale DMA)
// 2 activation + 1 activation-scale DMA, then kWI weight loads and
// (prepared) 1 weight-scale dword
template <bool PREP>
constexpr int kWeightLoads = PREP ? kWI + 1 : kWI;
// activation DMA requests per wave and chunk: MXFP8 rows of 128 bytes, two;
// MXFP4 rows of 64 bytes, one
template <bool AF4>
constexpr int kXDma = AF4 ? 1 : 2;
template <bool PREP, bool AF4>
constexpr int kLoadsPerChunk = kXDma<AF4> + 1 + (PREP ? 0 : kWsDma) + kWeightLoads<PREP>;

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

// MXFP4 activations: the same block maximum; X is the smallest exponent with
// amax <= 6 * 2^X (6 = 1.5 * 2^2), each element's magnitude is rounded on
// the E2M1 grid of its range (steps 0.5 below 2, 1 in [2, 4), 2 from 4;
// rintf: ties to the even step, which is the even code) and clamped to 6;
// codes sign << 3 | magnitude index, two to a byte, low nibble first.
__device__ __forceinline__ uint32_t e2m1_code(float v) {
  // v = x / 2^X with |v| <= 6 by the choice of X
  const float a = fabsf(v);
  const int ea = (int)(__float_as_uint(a) >> 23) - 127;  // floor(log2 a); -127 for 0 and subnormals
  const int eq = ea > 0 ? ea : 0;
  const uint32_t n = (uint32_t)rintf(a * __uint_as_float((uint32_t)(127 + 1 - eq) << 23));  // a / 2^(eq - 1)
  const uint32_t code = 2u * (uint32_t)eq + n;
  return code < 7u ? code : 7u;
}

__global__ void __launch_bounds__(256) quant_mxfp4_kernel(const uint16_t* __restrict__ x, int T, int I, int Kp,
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
  amax = max(amax, (uint32_t)__builtin_amdgcn_mov_dpp((int)amax, 0xB1, 0xF, 0xF, false));
  amax = max(amax, (uint32_t)__builtin_amdgcn_mov_dpp((int)amax, 0x4E, 0xF, 0xF, false));
  amax = max(amax, (uint32_t)__builtin_amdgcn_mov_dpp((int)amax, 0x141, 0xF, 0xF, false));
  // X: the smallest exponent with amax <= 6 * 2^X (6 = 1.5 * 2^2), clamped to [-127, 127]
  const uint32_t ab = amax << 16;  // fp32 bits of amax
  const int e = (int)(ab >> 23) - 127;
  int X = (ab & 0x7FFFFFu) <= 0x400000u ? e - 2 : e - 1;
  if ((ab >> 23) == 0) X = -127;  // zero or subnormal block
  X = X < -127 ? -127 : (X > 127 ? 127 : X);
  const float inv = __uint_as_float((uint32_t)(127 - X) << 23);  // 2^-X, X in [-127, 126] for finite bf16
  uint32_t half = 0;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const float v = __uint_as_float(h[i] << 16) * inv;
    half |= (e2m1_code(v) | ((h[i] >> 12) & 0x8u)) << (4 * i);
  }
  *reinterpret_cast<uint16_t*>(codes + (int64_t)t * (Kp / 2) + k0 / 2) = (uint16_t)half;
  if (sub == 0) sb[(int64_t)t * nb + jb] = (uint8_t)(X + 127);
}

// ---- grouped GEMM

// PREP: the weights come in the fragment-major prepared layout of
// prepare_mx_kernel (one contiguous 1 KB block per 16-row fragment and chunk,
// and one scale dword per lane for four fragments) instead of the canonical
// [E, O, G, 16] / [E, O, G].
template <bool PREP, bool AF4>
__global__ void __launch_bounds__(512, 1) gemm_mx_kernel(const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs,
                                                         const uint8_t* __restrict__ packed,
                                                         const uint8_t* __restrict__ scales,
                                                         const int32_t* __restrict__ perm,
                                                         const GemmTile* __restrict__ tiles,
                                                         const int32_t* __restrict__ n_tiles, float* __restrict__ part,
                                                         int K, int O, int G, int Kp, int n_ntiles, int n_wg, uint32_t xq_bytes,
                                                         uint32_t xs_bytes) {
  // Workgroup i runs on XCD i mod 8. Each XCD takes its M-tiles (below) with
  // all their N-tiles back to back, so the N-tiles of an M-tile share its
  // gathered activation rows in one L2 instead of every XCD fetching them,
  // while the pairs of neighbouring M-tiles still spread over all XCDs.
  const int xcd_step = blockIdx.x >> 3;
  // tiles in pairs (2x, 2x + 1, 2x + 16, ...): an expert's partial second
  // M-tile usually runs on the same XCD as its first and finds the weights in L2
  const int jx = xcd_step / n_wg;
  const int ti = 2 * ((blockIdx.x & 7) + 8 * (jx >> 1)) + (jx & 1);
  const int nt = xcd_step % n_wg;  // feature tile of NW features
  if (ti >= n_tiles[0]) return;
  const GemmTile tl = tiles[ti];
  const int f0 = nt * NW;

  // Activation ring: three chunk slots, each 128 rows x 128 bytes with the
  // 16-byte pieces of row m stored at position piece ^ ((m >> 1) & 7): LDS
  // serves a 16-byte read for 16 lanes at a time over 64 banks (256 bytes, two
  // rows), and the 16 rows of a fragment read then land on 16 distinct bank
  // groups without padding; and 4 x 64 scale dwords (wave w's dword
  // l < 32 is row 32 w + l). Three separate arrays, so that the compiler can
  // tell a slot being read from the slots the DMA is filling.
  constexpr int XB = AF4 ? KC / 2 : KC;  // bytes of one activation row and chunk
  __shared__ __attribute__((aligned(16))) uint8_t X0[MT * XB];
  __shared__ __attribute__((aligned(16))) uint8_t X1[MT * XB];
  __shared__ __attribute__((aligned(16))) uint8_t X2[MT * XB];
  __shared__ __attribute__((aligned(16))) uint32_t S0[64 * kWaves];
  __shared__ __attribute__((aligned(16))) uint32_t S1[64 * kWaves];
  __shared__ __attribute__((aligned(16))) uint32_t S2[64 * kWaves];
  // canonical: the chunk's weight scale bytes, three slots with the activations
  __shared__ __attribute__((aligned(16))) uint8_t WS0[PREP ? 16 : kWsWin + kWsZero];
  __shared__ __attribute__((aligned(16))) uint8_t WS1[PREP ? 16 : kWsWin + kWsZero];
  __shared__ __attribute__((aligned(16))) uint8_t WS2[PREP ? 16 : kWsWin + kWsZero];

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int lr = lane & 15, lc = lane >> 4;

  // activation DMA: wave w, request j fills rows 16 w + 8 j .. +7 of a slot
  // (1 KB); lane l lands at row m = 16 w + 8 j + (l >> 3), position l & 7 and
  // so fetches piece (l & 7) ^ ((m >> 1) & 7) of its row. Scale DMA: lane l < 16 fetches the dword of
  // row 16 w + l (blocks 4q .. 4q+3); lanes 16 .. 63 read past the resource
  // and write zeros into the unused part of the wave's 64 dwords.
  // MXFP4 activations (rows of 64 bytes, 4 pieces): wave w's one request
  // fills rows 16 w .. 16 w + 15; lane l lands at row m = 16 w + (l >> 2),
  // position l & 3, and fetches piece (l & 3) ^ ((m >> 2) & 3) of its row.
  uint32_t x_off[kXDma<AF4>];
#pragma unroll
  for (int j = 0; j < kXDma<AF4>; j++) {
    const int m = AF4 ? 16 * w + (lane >> 2) : 16 * w + 8 * j + (lane >> 3);
    const int tok = m < tl.mlen ? perm[tl.row0 + m] / K : -1;
    const int piece = AF4 ? (lane & 3) ^ ((m >> 2) & 3) : (lane & 7) ^ ((m >> 1) & 7);
    x_off[j] = tok >= 0 ? (uint32_t)tok * (uint32_t)(Kp / (AF4 ? 2 : 1)) + 16u * (uint32_t)piece : kOob;
  }
  uint32_t s_off;
  {
    const int m = 16 * w + lane;
    const int tok = (lane < 16 && m < tl.mlen) ? perm[tl.row0 + m] / K : -1;
    s_off = tok >= 0 ? (uint32_t)tok * (uint32_t)(Kp / 32) : kOob;
  }
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc((void*)xq, (short)0, (int)xq_bytes, kRsrcFlags);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)xs, (short)0, (int)xs_bytes, kRsrcFlags);

  // weight fragments: rows f0 + 32 w + 16 i + lr, group 4 q + lc
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
  // prepared: byte offset of this lane's scale dword in chunk 0
  // prepared: this wave's 64 features lie in 128-row tile pt, fragments 4 (w & 1) + i
  const int pt = 4 * nt + (w >> 1);
  const bool pt_live = pt < n_ntiles;  // the second half of the last workgroup may lie past O
  const uint32_t w_sc = pt_live ? (uint32_t)(((pt * nq * 2 + (w & 1)) * 64 + lane) * 4) : kOob;
  uint32_t w_grp[kWI];  // canonical: group index (row * G + lc) of chunk 0; prepared: group slot of chunk 0; or kOob
#pragma unroll
  for (int i = 0; i < kWI; i++) {
    const int f = f0 + 16 * kWI * w + 16 * i + lr;
    if constexpr (PREP)
      w_grp[i] = pt_live ? (uint32_t)((pt * nq * 8 + kWI * (w & 1) + i) * 64 + lane) : kOob;
    else
      w_grp[i] = f < O ? (uint32_t)f * (uint32_t)G + (uint32_t)lc : kOob;
  }

  // canonical weight scales: request m of wave w fills dwords d = 64 (2 w + m) + l
  // of a slot: LDS row R = d / 2 (feature f0 + R), dword d % 2 of the row's
  // bytes from the dword boundary below group 4 q (a dword that holds a valid
  // byte lies in a valid page)
  const uintptr_t s_first = reinterpret_cast<uintptr_t>(scales) + (uintptr_t)ebase;
  const int s_mis = PREP ? 0 : (int)(s_first & 3);
  const __amdgpu_buffer_rsrc_t rsa = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(s_first & ~(uintptr_t)3), (short)0, (s_mis + O * G + 3) & ~3, kRsrcFlags);
  uint32_t ws_off[PREP ? 1 : kWsDma];  // byte offset of this lane's dword in chunk 0 (chunk q: + 4 q)
  int ws_lds = 0;  // byte of fragment 0's row in a slot where group 4 q starts (fragment i: + 16 kWsPitch i)
  if constexpr (!PREP) {
#pragma unroll
    for (int m = 0; m < kWsDma; m++) {
      const int d = 64 * (kWsDma * w + m) + lane, R = d / 2, k = d - 2 * R;
      const int f = f0 + R;
      ws_off[m] = f < O ? (uint32_t)(((s_mis + f * G) >> 2) + k) * 4u : kOob;
    }
    const int f = f0 + 16 * kWI * w + lr;  // rows 16 apart share the offset within the dword
    ws_lds = (16 * kWI * w + lr) * kWsPitch + (f < O ? (s_mis + f * G) & 3 : 0) + lc;
  }

  u32x4 wf[kRing][kWI];
  uint32_t wsp[kRing];     // prepared: the four fragments' scale bytes in one dword
  // exactly kLoadsPerChunk vector-memory requests per chunk, in this order
  auto dma_x = [&](int q, uint8_t* xdst, uint32_t* sdst, uint8_t* wsdst) {
    if constexpr (!PREP) {
#pragma unroll
      for (int m = 0; m < kWsDma; m++)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rsa, (__attribute__((address_space(3))) void*)(wsdst + (kWsDma * w + m) * 256), 4,
            (int)(ws_off[m] + 4u * q), 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < kXDma<AF4>; j++)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (__attribute__((address_space(3))) void*)(xdst + (16 * w + 8 * j) * XB),
                                               16, (int)(x_off[j] + (uint32_t)XB * q), 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(sdst + 64 * w), 4,
                                             (int)(s_off + 4u * q), 0, 0, 0);
  };
  auto load_w = [&](int q, int slot) {
    // canonical: a group past G moves the offset past the resource (the sign
    // bit of G - 1 - group); prepared: padding groups hold zeros, chunk q is
    // 8 fragments x 64 group slots further on
    const uint32_t past = PREP ? 0u : (uint32_t)(G - 1 - (4 * q + lc)) >> 31 << 31;
    const uint32_t step_q = PREP ? 512u : 4u;
#pragma unroll
    for (int i = 0; i < kWI; i++) {
      const uint32_t g = (w_grp[i] + step_q * q) | past;  // kOob stays past the resource
      wf[slot][i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, (int)(g << 4 | (g & kOob)), 0, 0));
    }
    if constexpr (PREP) wsp[slot] = __builtin_amdgcn_raw_buffer_load_b32(rsc, (int)(w_sc + 512u * q), 0, 0);
  };
  // wait until this wave's DMA of the next chunk has landed: it was followed
  // by that chunk's weight requests and by one whole chunk of requests
  auto wait_next_x = [&]() {
    constexpr int n = kWeightLoads<PREP> + kLoadsPerChunk<PREP, AF4>;
    __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | 0x0F70);
  };

  v4f acc[kWI][kWJ];
#pragma unroll
  for (int i = 0; i < kWI; i++)
#pragma unroll
    for (int j = 0; j < kWJ; j++) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // One chunk q in ring slot R = q mod 3 (compile-time: no register array or
  // LDS slot is chosen at run time): request chunk q + 2 (activations by DMA
  // into slot (q + 2) mod 3, read last during chunk q - 1; weights into
  // register slot (q + 2) mod 3), multiply chunk q, wait for this wave's DMA
  // of chunk q + 1, barrier. Past the last chunk the requests repeat the
  // last chunk into a slot nobody reads again, so the number of requests per
  // chunk - and with it every wait count - is fixed.
  auto step = [&](int q, auto slot) {
    constexpr int R = decltype(slot)::value, RN = (R + 2) % kRing;
    uint8_t* xn = RN == 0 ? X0 : (RN == 1 ? X1 : X2);
    uint32_t* sn = RN == 0 ? S0 : (RN == 1 ? S1 : S2);
    uint8_t* wsn = RN == 0 ? WS0 : (RN == 1 ? WS1 : WS2);
    const uint8_t* xc = R == 0 ? X0 : (R == 1 ? X1 : X2);
    const uint32_t* sc = R == 0 ? S0 : (R == 1 ? S1 : S2);
    const uint8_t* wsc = R == 0 ? WS0 : (R == 1 ? WS1 : WS2);
    dma_x(min(q + 2, nq - 1), xn, sn, wsn);
    load_w(min(q + 2, nq - 1), RN);
    __builtin_amdgcn_sched_barrier(0);  // keep the requests ahead of the MFMAs
    // canonical: the fragments' scale bytes of chunk q (a group past G reads
    // the zero bytes after the slot: another row's byte otherwise)
    int as_c[kWI];
    if constexpr (!PREP) {
      const int off = 4 * q + lc < G ? ws_lds : kWsWin;
#pragma unroll
      for (int i = 0; i < kWI; i++) as_c[i] = wsc[off + 16 * kWsPitch * i];
    }
#pragma unroll
    for (int j = 0; j < kWJ; j++) {
      const int p = 16 * j + lr;  // rows past the tile's end hold zeros (their DMA read past the resource)
      v8i bf;
      if constexpr (AF4) {
        // lane (p, c): the 16 bytes of block 4 q + c of pair p, like a weight lane's group
        const u32x4 lo = *reinterpret_cast<const u32x4*>(&xc[p * XB + 16 * (lc ^ (lr >> 2))]);  // (p >> 2) & 3 = lr >> 2
        bf = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], 0, 0, 0, 0};
      } else {
        const u32x4 lo = *reinterpret_cast<const u32x4*>(&xc[p * XB + 16 * (lc ^ (lr >> 1))]);  // (p >> 1) & 7 = lr >> 1
        const u32x4 hi = *reinterpret_cast<const u32x4*>(&xc[p * XB + 16 * ((4 + lc) ^ (lr >> 1))]);
        bf = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      }
      const int bs = (int)((sc[(p >> 4) * 64 + (p & 15)] >> (8 * lc)) & 0xFFu);
#pragma unroll
      for (int i = 0; i < kWI; i++) {
        const v8i a = v8i{(int)wf[R][i][0], (int)wf[R][i][1], (int)wf[R][i][2], (int)wf[R][i][3], 0, 0, 0, 0};
        const int as = PREP ? (int)((wsp[R] >> (8 * i)) & 0xFFu) : as_c[i];
        // A: E2M1 (format 4); B: E4M3 (0) or E2M1 (4)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, bf, acc[i][j], 4, AF4 ? 4 : 0, 0, as, 0, bs);
      }
    }
    // interleave each fragment's LDS reads with its MFMAs, so that only a few
    // activation fragments are live at once (registers; with MXFP4
    // activations, groups of one read keep the canonical instantiation
    // within its registers)
#pragma unroll
    for (int j = 0; j < kWJ; j++) {
      __builtin_amdgcn_sched_group_barrier(0x100, AF4 ? 1 : 3, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, kWI, 0);
    }
    wait_next_x();
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS reads are done
    __builtin_amdgcn_s_barrier();
  };
  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;
  using C2 = std::integral_constant<int, 2>;
  if constexpr (!PREP) {
    if (tid < kWsZero / 16) {
      reinterpret_cast<u32x4*>(WS0 + kWsWin)[tid] = u32x4{0u, 0u, 0u, 0u};
      reinterpret_cast<u32x4*>(WS1 + kWsWin)[tid] = u32x4{0u, 0u, 0u, 0u};
      reinterpret_cast<u32x4*>(WS2 + kWsWin)[tid] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  dma_x(0, X0, S0, WS0);
  load_w(0, 0);
  dma_x(min(1, nq - 1), X1, S1, WS1);
  load_w(min(1, nq - 1), 1);
  wait_next_x();  // chunk 0's DMA: followed by chunk 0's weights and all of chunk 1's requests
  __builtin_amdgcn_s_barrier();
  int q = 0;
  for (; q + 2 < nq; q += 3) {
    step(q, C0{});
    step(q + 1, C1{});
    step(q + 2, C2{});
  }
  if (q < nq) step(q, C0{});
  if (q + 1 < nq) step(q + 1, C1{});
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): no DMA may land in LDS after the workgroup ends

  // lane (lr, lc) of fragment (i, j): pair 16 j + lr, features 32 w + 16 i + 4 lc .. +3
#pragma unroll
  for (int j = 0; j < kWJ; j++) {
    const int p = 16 * j + lr;
    if (p >= tl.mlen) continue;
    float* row = part + (int64_t)(tl.row0 + p) * O;
#pragma unroll
    for (int i = 0; i < kWI; i++) {
      const int f = f0 + 16 * kWI * w + 16 * i + 4 * lc;
      if (f < O) *reinterpret_cast<v4f*>(row + f) = acc[i][j];
    }
  }
}

// Prepared layout, per expert e, N-tile n (128 rows) and chunk q (4 groups):
// group slot (f, l) = row 16 f + (l & 15) of the tile, group 4 q + (l >> 4)
// (exactly what lane l of the MFMA's A operand for 16-row fragment f takes).
// The codes form 8 blocks of 1 KB: fragment-major (block f = the 16-byte
// slots of fragment f in lane order; the block-scaled variant loads one slot
// per lane) or, with `interleaved`, dword-interleaved (block 4 h + s holds at
// bytes 16 l + 4 (f & 3) dword s of slot (f, l) for the fragments f of half h;
// one 16-byte read then gives a lane one bf16 MFMA step's codes of four
// fragments). In a second array, the slots' scale bytes (four fragments to a
// lane's dword). Rows past O and groups past G are zero. One thread per slot.
// F > 0 (SwiGLU order): the source stacks gate rows [0, F) over up rows
// [F, 2F) (O = 2F), and prepared tile n holds gate rows 64 n .. 64 n + 63
// followed by the up rows of the same features, so that one 128-row tile
// carries both halves of 64 features; rows of features past F are zero.
__global__ void __launch_bounds__(256) prepare_mx_kernel(const uint8_t* __restrict__ packed,
                                                         const uint8_t* __restrict__ scales, int64_t n_slots, int O,
                                                         int G, int n_ntiles, int nq, uint8_t* __restrict__ pp,
                                                         uint8_t* __restrict__ ps, int F, bool interleaved) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= n_slots) return;
  const int l = (int)(idx & 63), fr = (int)((idx >> 6) & 7);
  const int64_t rest = idx >> 9;  // (e * n_ntiles + n) * nq + q
  const int q = (int)(rest % nq);
  const int64_t en = rest / nq;
  const int n = (int)(en % n_ntiles);
  const int64_t e = en / n_ntiles;
  const int k = 16 * fr + (l & 15), g = 4 * q + (l >> 4);
  int row = 128 * n + k;
  if (F > 0) {
    const int f = 64 * n + (k & 63);
    row = f < F ? (k < 64 ? f : F + f) : O;
  }
  u32x4 v = u32x4{0u, 0u, 0u, 0u};
  uint8_t sc = 0;
  if (row < O && g < G) {
    const int64_t src = (e * O + row) * G + g;
    v = *reinterpret_cast<const u32x4*>(packed + src * 16);
    sc = scales[src];
  }
  if (interleaved) {
    // dword s of slot (fr, l) goes to block 4 (fr >> 2) + s of the (tile, chunk), lane l, position fr & 3
#pragma unroll
    for (int sd = 0; sd < 4; sd++)
      *reinterpret_cast<uint32_t*>(pp + ((((rest * 2 + (fr >> 2)) * 4 + sd) * 64 + l) * 16 + 4 * (fr & 3))) = v[sd];
  } else {
    *reinterpret_cast<u32x4*>(pp + idx * 16) = v;
  }
  // scales: per (tile, chunk, half of the 8 fragments) 64 lanes x 4 bytes,
  // byte 4 l + (fr & 3): one dword per lane holds its four fragments' scales
  ps[((rest * 2 + (fr >> 2)) * 64 + l) * 4 + (fr & 3)] = sc;
}

}  // namespace

size_t mx_prepared_bytes(int64_t E, int64_t O, int64_t G) {
  const int64_t slots = E * ((O + NT - 1) / NT) * (mx_row_bytes(32 * G) / KC) * 512;
  return (size_t)slots * 17;
}

hipError_t launch_prepare_mx(const uint8_t* packed, const uint8_t* scales, int64_t E, int O, int G, uint8_t* prepared,
                             hipStream_t stream, int swiglu_F, bool interleaved) {
  const int n_ntiles = (O + NT - 1) / NT, nq = mx_row_bytes(32 * (int64_t)G) / KC;
  const int64_t slots = E * n_ntiles * nq * 512;
  if (slots == 0) return hipSuccess;
  hipLaunchKernelGGL(prepare_mx_kernel, dim3((unsigned)((slots + 255) / 256)), dim3(256), 0, stream, packed, scales,
                     slots, O, G, n_ntiles, nq, prepared, prepared + slots * 16, swiglu_F, interleaved);
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

namespace {
template <bool PREP, bool AF4>
void launch_gemm_mx_t(dim3 grid, const uint8_t* xq, const uint8_t* xs, const uint8_t* packed, const uint8_t* scales,
                      const int32_t* perm, const GemmTile* tiles, const int32_t* n_tiles, float* part, int K, int O,
                      int G, int Kp, int n_ntiles, int n_wg, uint32_t xq_bytes, uint32_t xs_bytes, hipStream_t stream) {
  hipLaunchKernelGGL((gemm_mx_kernel<PREP, AF4>), grid, dim3(64 * kWaves), 0, stream, xq, xs, packed, scales, perm,
                     tiles, n_tiles, part, K, O, G, Kp, n_ntiles, n_wg, xq_bytes, xs_bytes);
}
}  // namespace

hipError_t launch_quant_mxfp4(const uint16_t* x, int T, int I, int Kp, uint8_t* codes, uint8_t* sb,
                              hipStream_t stream) {
  if (I % 32 || Kp % 32 || Kp < I) return hipErrorInvalidValue;
  const int64_t threads = (int64_t)T * (Kp / 32) * 8;
  if (threads == 0) return hipSuccess;
  hipLaunchKernelGGL(quant_mxfp4_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, x, T, I, Kp,
                     codes, sb);
  return hipGetLastError();
}

hipError_t launch_gemm_mx(const uint8_t* xq, const uint8_t* xs, const uint8_t* packed, const uint8_t* scales,
                          const int32_t* perm, const GemmTile* tiles, const int32_t* n_tiles, int64_t max_tiles,
                          float* part, int T, int K, int O, int G, hipStream_t stream, bool prepared, bool act_fp4) {
  const int Kp = mx_row_bytes(32 * (int64_t)G);
  const int n_ntiles = (O + NT - 1) / NT, n_wg = (O + NW - 1) / NW;
  // 8 XCDs x an even number of M-tiles each x the feature tiles
  const int64_t nblk = (max_tiles + 15) / 16 * 16 * n_wg;  // an even number of tiles per XCD
  if (nblk == 0) return hipSuccess;
  // activation codes: Kp bytes per token (MXFP8) or Kp / 2 (MXFP4)
  const uint32_t xq_bytes = (uint32_t)((int64_t)T * Kp / (act_fp4 ? 2 : 1)), xs_bytes = (uint32_t)((int64_t)T * Kp / 32);
  const dim3 grid((unsigned)nblk);
  if (prepared && act_fp4)
    launch_gemm_mx_t<true, true>(grid, xq, xs, packed, scales, perm, tiles, n_tiles, part, K, O, G, Kp, n_ntiles,
                                 n_wg, xq_bytes, xs_bytes, stream);
  else if (prepared)
    launch_gemm_mx_t<true, false>(grid, xq, xs, packed, scales, perm, tiles, n_tiles, part, K, O, G, Kp, n_ntiles,
                                  n_wg, xq_bytes, xs_bytes, stream);
  else if (act_fp4)
    launch_gemm_mx_t<false, true>(grid, xq, xs, packed, scales, perm, tiles, n_tiles, part, K, O, G, Kp, n_ntiles,
                                  n_wg, xq_bytes, xs_bytes, stream);
  else
    launch_gemm_mx_t<false, false>(grid, xq, xs, packed, scales, perm, tiles, n_tiles, part, K, O, G, Kp, n_ntiles,
                                   n_wg, xq_bytes, xs_bytes, stream);
  return hipGetLastError();
}

}  // namespace mxfp4
