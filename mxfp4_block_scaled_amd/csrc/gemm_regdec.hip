// Prefill-shaped grouped GEMM, weights decoded in registers:
// bf16 MFMA (v_mfma_f32_16x16x32_bf16) with fp32 accumulation, the same
// results contract as the LDS-staged kernel of gemm.hip (page "MXFP4 Routed
// Expert Linear", "Reconstruct the matrix in the right orientation": each
// output coordinate is a row of W_e dotted with the token; page "MXFP4
// Dequant", "How it works": code n of byte j, low nibble first, times
// 2^(s-127)).
//
// Two weight layouts. Canonical (CANON): packed (E, O, G, 16) and scales
// (E, O, G) as the caller holds them; the weight DMA fetches the 16-byte
// groups straight from that layout, four lanes to a row's 64 contiguous
// bytes, into one 1 KB block per 16-row fragment and chunk, and the scale
// bytes come into LDS in windows of 8 groups (each row's bytes read as whole
// dwords from the dword boundary below them).
// Prepared: the weights come in the prepared layout of prepare_mx_kernel (a load-time
// byte permutation: per expert, 128-row tile and chunk of 4 groups, the group
// slots of the 8 16-row fragments in MFMA lane order - slot l of fragment f =
// row 16 f + (l & 15), group 4q + (l >> 4) - as 8 blocks of 1 KB, block
// 4 h + s holding for lane l dword s of fragments 4 h .. 4 h + 3; and the
// slots' scale bytes, four fragments to a dword per lane).
//
// Work: the M-tiles of the bucketing (<= 128 pairs of one expert; a full
// tile also takes the partial tile of at most 16 pairs that follows it, see
// kMergeMax) x N-tiles of 512 weight rows (modes below: the routed linear,
// and the two stages of the SwiGLU expert block). Eight waves per workgroup,
// 2 (pairs) x 4 (rows): wave
// (wm, wn) owns pairs 64 wm .. +63 and the 128 rows of prepared tile
// 4 nt + wn, 8 x 4 MFMA tiles of 16 x 16. Inputs go in chunks of 128 (4
// groups). Per chunk the workgroup brings into LDS, by DMA (buffer loads that
// write LDS directly, no registers): the 128 gathered activation rows (row =
// perm / K; 32 KB; two-slot ring, one chunk ahead - they come from L2,
// shared by the N-tiles of the M-tile) and the 32 fragment blocks of its
// weights (32 KB; two-slot ring, one chunk ahead - they come from HBM), and
// the scale bytes: canonical, windows of 8 groups of the workgroup's rows,
// two slots; prepared, two dwords per wave and chunk straight to registers.
// Each weight byte is fetched once per workgroup; each activation row once
// per 512 weight rows. One full wait and one barrier per chunk.
//
// Operand A = weights: for MFMA k-step s (0..3) lane (r, c) reads dword d of
// its slot of all 8 fragments (prepared: d = s, two conflict-free 16-byte LDS
// reads of the interleaved blocks; canonical: d = (s + c) mod 4, eight 4-byte
// reads that the slot positions spread over 64 banks) and turns each dword's
// 8 codes into 8 bf16 with gfx950's scaled FP4 convert, scale applied (exact:
// E2M1 times a power of two is a bf16 value, or +-inf where it overflows). No
// decoded weight is stored anywhere. Operand B = activations: lane (p, c) of
// k-step s takes the 8 bf16 inputs 128q + 32c + 8d .. +7 of pair p - the
// inputs of the weight lane (r, c) of that k-step, so every product pairs x_i
// with w_i. The
// 16-byte pieces of activation row m sit at position piece ^ (m & 15) of its
// LDS row: the 16 lanes that LDS serves together (16 bytes each across its 64
// banks) read 16 rows at 16 distinct positions. Rows past the tile, inputs past I
// and prepared tiles past O read through an offset beyond their buffer
// resource: zeros, no memory traffic.
//
// Large scale bytes: E2M1 * 2^(s-127) leaves the bf16 range for s >= 253
// while the layer's value stays finite. A wave that meets such a byte (a
// wave-uniform test that ordinary data never passes) decodes from then on
// at scale byte s - 3 (0 for s < 3), having multiplied its accumulators by
// 2^-3, and multiplies them by 2^3 at the end: power-of-two scaling commutes
// with the exact products and the fp32 sums, so the result is the exact
// layer's up to fp32 rounding (weights with scale bytes 0..2 in such a tile,
// below 2^-121 in magnitude, are read at 2^-124). This also keeps scale byte
// 255, which the convert reads as NaN, away from the convert.
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace mxfp4 {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int kRsrcFlags = 0x00020000;
constexpr uint32_t kOob = 0x80000000u;
constexpr int MT = kGemmTileM;    // 128 pairs
constexpr int kWaves = 8;         // 2 (pairs) x 4 (rows)
constexpr int PT = 128;           // rows of a prepared weight tile (one per wave column)
constexpr int kWI = PT / 16;      // 16-row weight fragments per wave
constexpr int kWJ = 4;            // 16-pair activation fragments per wave
constexpr int NW = 4 * PT;        // weight rows per workgroup
constexpr int KC = 128;           // inputs per chunk (4 groups)
constexpr int ROWB = 2 * KC;      // LDS bytes of one activation row and chunk
constexpr int kXBytes = MT * ROWB;        // activation slot (32 KB)
constexpr int kWBytes = NW / 16 * 1024;   // weight slot: 32 fragment blocks of 1 KB
constexpr int kXDma = kXBytes / (1024 * kWaves);  // 1 KB requests per wave and chunk
constexpr int kWDma = kWBytes / (1024 * kWaves);
constexpr int kScLoads = 2;                        // scale dwords per wave and chunk
// canonical weights: a scale window is 8 groups (2 chunks) of the
// workgroup's 512 rows, each row's 8 bytes with the dword boundary below
// them (3 dwords, pitch 12 bytes), 3 DMA requests per wave
constexpr int kScPitch = 12;
constexpr int kScWords = kScPitch / 4;
constexpr int kScWin = NW * kScPitch;
constexpr int kScDma = kScWin / (256 * kWaves);
constexpr int kScZero = 16 * kScPitch * kWI;  // zero bytes after a window slot
// an expert's partial M-tile of at most kMergeMax pairs that follows its last
// full tile is multiplied by the full tile's workgroup
constexpr int kMergeMax = 16;
constexpr int kXEBytes = kMergeMax * ROWB;  // activation slot of the merged pairs (4 KB)
static_assert(kScDma * 256 * kWaves == kScWin, "scale window DMA");

constexpr uint32_t kShiftFrom = 253;  // scale bytes whose decoded weights may overflow bf16
constexpr uint32_t kShift = 3;        // scale-byte shift of a wave that met one

typedef __attribute__((address_space(3))) void* lds_ptr;

// What the rows and columns are:
//  kGather: activation rows are the tokens of the tile's pairs (perm / K);
//           output fp32 rows of `part` at the sorted positions.
//  kSwiGLU: activation rows as kGather; the weights are the stacked gate and
//           up matrices prepared with prepare_mx_kernel's SwiGLU row order
//           (prepared tile n: gate rows 64 n .. +63, then the up rows of the
//           same features), so a wave's fragments 0..3 hold the gate rows and
//           4..7 the up rows of 64 features; the epilogue writes bf16
//           h[position, f] = silu(gate) * up (page "MoE Expert Kernels:
//           Grouped Prefill and Mixed-Quant Compact Experts", section 1).
//  kDirect: activation rows are the sorted positions themselves (rows of h);
//           output fp32 rows of `part`.
enum Mode { kGather = 0, kSwiGLU = 1, kDirect = 2 };

template <int MODE, bool CANON>
__global__ void __launch_bounds__(512, 1) gemm_regdec_kernel(const uint16_t* __restrict__ x,
                                                             const uint8_t* __restrict__ pcodes,
                                                             const uint8_t* __restrict__ pscales,
                                                             const int32_t* __restrict__ perm,
                                                             const GemmTile* __restrict__ tiles,
                                                             const int32_t* __restrict__ n_tiles,
                                                             void* __restrict__ out, int K, int O, int G, int F,
                                                             int n_wg, int n_ptiles, uint32_t x_bytes) {
  // Workgroup i runs on XCD i mod 8: each XCD takes its M-tiles (below) with
  // all their N-tiles back to back, so the N-tiles of an M-tile share its
  // gathered activation rows in one L2.
  const int xcd_step = blockIdx.x >> 3;
  // tiles in pairs: XCD x takes tiles 2x, 2x + 1, 2x + 16, 2x + 17, ..., so that
  // the partial second M-tile of an expert usually follows its first on the
  // same XCD and finds the expert's weights in that L2
  const int jx = xcd_step / n_wg;
  const int ti = 2 * ((blockIdx.x & 7) + 8 * (jx >> 1)) + (jx & 1);
  const int nt = xcd_step % n_wg;
  const int n_t = n_tiles[0];
  if (ti >= n_t) return;
  const GemmTile tl = tiles[ti];
  // Merged remainders (not the SwiGLU gate/up stage, whose
  // epilogue needs a gate and an up fragment in one wave): a tile of at most
  // kMergeMax pairs that continues the rows of its expert's full tile right
  // before it in the list is multiplied by that tile's workgroup, which then
  // reads the expert's weights once for both; both workgroups test the same
  // two list entries, so every pair is multiplied exactly once.
  constexpr bool kMerge = MODE != kSwiGLU;
  int mtot = tl.mlen;  // pairs this workgroup multiplies: the tile's and a merged remainder's
  if constexpr (kMerge) {
    // the neighbours are read together with the tile (not after testing it)
    const GemmTile pv = tiles[ti > 0 ? ti - 1 : ti];
    const GemmTile nx = tiles[ti + 1 < n_t ? ti + 1 : ti];
    // keeps the compiler from moving the read of nx past the return below
    asm volatile("" ::"s"(nx.e), "s"(nx.row0), "s"(nx.mlen));
    // (bitwise tests, both before the return: no test guards a read)
    const bool absorbed =
        (ti > 0) & (tl.mlen <= kMergeMax) & (pv.e == tl.e) & (pv.mlen == MT) & (pv.row0 + MT == tl.row0);
    const bool absorbs =
        (ti + 1 < n_t) & (tl.mlen == MT) & (nx.e == tl.e) & (nx.mlen <= kMergeMax) & (nx.row0 == tl.row0 + MT);
    if (absorbed) return;
    if (absorbs) mtot = MT + nx.mlen;
  }
  const bool extra = kMerge && mtot > MT;  // workgroup-uniform

  __shared__ __attribute__((aligned(16))) uint8_t X0[kXBytes];
  __shared__ __attribute__((aligned(16))) uint8_t X1[kXBytes];
  __shared__ __attribute__((aligned(16))) uint8_t W0[kWBytes];
  __shared__ __attribute__((aligned(16))) uint8_t W1[kWBytes];
  // canonical: scale-byte windows of 8 groups, two slots, each followed by
  // zero bytes (separate arrays, and every read indexes one of them, so that
  // a read of one is never taken to wait for a DMA into the other)
  __shared__ __attribute__((aligned(16))) uint8_t Sc0[CANON ? kScWin + kScZero : 16];
  __shared__ __attribute__((aligned(16))) uint8_t Sc1[CANON ? kScWin + kScZero : 16];
  // the merged pairs' activation rows, two slots
  __shared__ __attribute__((aligned(16))) uint8_t XE0[MODE != kSwiGLU ? kXEBytes : 16];
  __shared__ __attribute__((aligned(16))) uint8_t XE1[MODE != kSwiGLU ? kXEBytes : 16];

  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int lr = lane & 15, lc = lane >> 4;
  const int wm = w >> 2, wn = w & 3;
  const int nq = (G + 3) / 4;  // chunks

  // ---- activation DMA: request j of wave w fills rows 16 w + 4 j .. +3 of a
  // slot (1 KB); lane l lands at row 16 w + 4 j + (l >> 4), position l & 15,
  // so it fetches piece (l & 15) ^ (row & 15) of that row.
  const int xld = 32 * G;  // bf16 inputs per activation row
  uint32_t x_off[kXDma];  // byte offset of the piece in chunk 0
#pragma unroll
  for (int j = 0; j < kXDma; j++) {
    const int m = 16 * w + 4 * j + (lane >> 4);
    const int piece = (lane & 15) ^ (m & 15);
    int row = -1;
    if (m < tl.mlen) row = MODE == kDirect ? tl.row0 + m : perm[tl.row0 + m] / K;
    x_off[j] = row >= 0 ? (uint32_t)row * (uint32_t)(2 * xld) + 16u * (uint32_t)piece : kOob;
  }
  // merged pairs: waves 0..3 fill rows 4 w .. 4 w + 3 of the merged slot
  // (pairs MT + 4 w + (l >> 4)), in the same piece order
  uint32_t xe_off = kOob;
  if (kMerge && extra && w < 4) {
    const int m = MT + 4 * w + (lane >> 4);
    const int piece = (lane & 15) ^ (m & 15);
    if (m < mtot) {
      const int row = MODE == kDirect ? tl.row0 + m : perm[tl.row0 + m] / K;
      xe_off = (uint32_t)row * (uint32_t)(2 * xld) + 16u * (uint32_t)piece;
    }
  }
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc((void*)x, (short)0, (int)x_bytes, kRsrcFlags);

  // ---- weight DMA: request j of wave w fills LDS block 4 w + j of a slot.
  // Prepared weights: code block 4 w + j of the workgroup (prepared tile
  // 4 nt + (w >> 1), block 4 (w & 1) + j: dword j of fragments 4 (w & 1) .. +3).
  // Canonical weights: fragment i = (4 w + j) & 7 of wave column
  // t = (4 w + j) >> 3, lane l fetching the 16 bytes of (row crow(t, i, l >> 2),
  // group 4 q + (((l & 3) - (l >> 4)) & 3)): each 4 lanes read the 64
  // contiguous bytes of one row (rows are 16 G bytes apart: one lane per row
  // would touch 16 cache lines per 16 lanes), and the slot of MFMA lane
  // (r, c) lies at position 4 r + ((c + (r >> 2)) & 3) of the block.
  // crow: the matrix row of fragment i, row r of wave column t.
  auto crow = [&](int t, int i, int r) -> int {
    if constexpr (MODE == kSwiGLU) {
      const int f = 64 * (4 * nt + t) + 16 * (i & 3) + r;
      return f < F ? (i < 4 ? f : F + f) : -1;
    } else {
      const int row = NW * nt + PT * t + 16 * i + r;
      return row < O ? row : -1;
    }
  };
  const int64_t ebase = CANON ? (int64_t)tl.e * O * G : (int64_t)tl.e * n_ptiles * nq * 512;
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(pcodes + ebase * 16), (short)0, CANON ? O * G * 16 : n_ptiles * nq * 8192, kRsrcFlags);
  const __amdgpu_buffer_rsrc_t rsc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(pscales + ebase), (short)0, CANON ? O * G : n_ptiles * nq * 512, kRsrcFlags);
  const int dpt = 4 * nt + (w >> 1);
  // prepared: byte offset of this lane's slot of the first fragment block, chunk 0 (chunk q: + 8192 q)
  const uint32_t w_off = dpt < n_ptiles ? (uint32_t)(((dpt * nq * 8 + 4 * (w & 1)) * 64 + lane) * 16) : kOob;
  // canonical: byte offset of this lane's group in chunk 0 per request (chunk q: + 64 q)
  uint32_t wc_off[CANON ? kWDma : 1];
  const int wgrp = ((lane & 3) - (lane >> 4)) & 3;  // canonical: this lane's group in its chunk
  if constexpr (CANON) {
#pragma unroll
    for (int j = 0; j < kWDma; j++) {
      const int row = crow((4 * w + j) >> 3, (4 * w + j) & 7, lane >> 2);
      wc_off[j] = row >= 0 ? ((uint32_t)row * (uint32_t)G + (uint32_t)wgrp) * 16u : kOob;
    }
  }
  // scale dwords of this wave's own tile (fragments 0..3 and 4..7), chunk 0 (chunk q: + 512 q)
  const int pt = 4 * nt + wn;
  const uint32_t s_off = pt < n_ptiles ? (uint32_t)((pt * nq * 2 * 64 + lane) * 4) : kOob;
  // canonical scales: the expert's bytes read as whole dwords from the dword
  // boundary below them (a dword that holds a valid byte lies in a valid
  // page); request m of wave w fills dwords d = 64 (3 w + m) + l of a window
  // slot: LDS row R = d / 3 (row crow(R >> 7, (R >> 4) & 7, R & 15)), dword d % 3
  const uintptr_t s_first = reinterpret_cast<uintptr_t>(pscales) + (uintptr_t)ebase;
  const int s_mis = CANON ? (int)(s_first & 3) : 0;
  const __amdgpu_buffer_rsrc_t rsa = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(s_first & ~(uintptr_t)3), (short)0, (s_mis + O * G + 3) & ~3, kRsrcFlags);
  uint32_t sw_off[CANON ? kScDma : 1];  // byte offset of this lane's dword, window 0 (window C: + 8 C)
  // byte of fragment i's row in a window slot where group 8 C starts:
  // sc_lds[i >> 2] + 16 kScPitch i (the rows of fragments 0..3 and of 4..7
  // share their offset within the dword: rows 16 apart, 16 G = 0 mod 4)
  int sc_lds[2];
  if constexpr (CANON) {
#pragma unroll
    for (int m = 0; m < kScDma; m++) {
      const int d = 64 * (kScDma * w + m) + lane, R = d / kScWords, k = d - kScWords * R;
      const int row = crow(R >> 7, (R >> 4) & 7, R & 15);
      sw_off[m] = row >= 0 ? (uint32_t)(((s_mis + row * G) >> 2) + k) * 4u : kOob;
    }
#pragma unroll
    for (int h = 0; h < 2; h++) {
      const int row = crow(wn, 4 * h, lr);
      sc_lds[h] = (PT * wn + lr) * kScPitch + (row >= 0 ? (s_mis + row * G) & 3 : 0);
    }
    if (extra && wm == 1) {
      // wave row 1 takes its fragments in the order 4..7, 0..3 (see fo below)
      const int t0 = sc_lds[0];
      sc_lds[0] = sc_lds[1] + 16 * kScPitch * 4;
      sc_lds[1] = t0 - 16 * kScPitch * 4;
    }
  }

  // prepared: two scale dwords per chunk (four fragments each), a two-slot ring
  uint32_t wsp[2][kScLoads];
  auto dma_x = [&](int q, uint8_t* dst, uint8_t* xe_dst) {
#pragma unroll
    for (int j = 0; j < kXDma; j++) {
      // an input past I moves the offset past the resource (the piece's first
      // input is 8 ((l & 15) ^ (row & 15)), row & 15 = 4 j + (l >> 4))
      const int first = 128 * q + 8 * ((lane & 15) ^ ((4 * j + lc) & 15));
      const uint32_t past = (uint32_t)(xld - 1 - first) >> 31 << 31;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_ptr)(dst + (16 * w + 4 * j) * ROWB), 16,
                                               (int)((x_off[j] + 256u * q) | past), 0, 0, 0);
    }
    if (kMerge && extra && w < 4) {
      const int first = 128 * q + 8 * ((lane & 15) ^ ((4 * w + lc) & 15));
      const uint32_t past = (uint32_t)(xld - 1 - first) >> 31 << 31;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_ptr)(xe_dst + 4 * w * ROWB), 16,
                                               (int)((xe_off + 256u * q) | past), 0, 0, 0);
    }
  };
  auto dma_w = [&](int q, uint8_t* dst, int slot) {
    if constexpr (CANON) {
      // a group past G moves the offset past the resource (zero codes)
      const uint32_t past = (uint32_t)(G - 1 - (4 * q + wgrp)) >> 31 << 31;
#pragma unroll
      for (int j = 0; j < kWDma; j++)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_ptr)(dst + (4 * w + j) * 1024), 16,
                                                 (int)((wc_off[j] + 64u * q) | past), 0, 0, 0);
    } else {
#pragma unroll
      for (int j = 0; j < kWDma; j++)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_ptr)(dst + (4 * w + j) * 1024), 16,
                                                 (int)((w_off + 8192u * q + 1024u * j) | (w_off & kOob)), 0, 0, 0);
#pragma unroll
      for (int h = 0; h < kScLoads; h++)
        wsp[slot][h] =
            __builtin_amdgcn_raw_buffer_load_b32(rsc, (int)((s_off + 512u * q + 256u * h) | (s_off & kOob)), 0, 0);
    }
  };
  // canonical: request m of scale window C into window slot dst
  auto dma_sc = [&](int C, int m, uint8_t* dst) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, (lds_ptr)(dst + (kScDma * w + m) * 256), 4,
                                             (int)(sw_off[m] + 8u * C), 0, 0, 0);
  };
  // whether this wave multiplies anything: pairs left in the tile, rows left in O
  const bool live = 64 * wm < tl.mlen && (MODE == kSwiGLU ? 64 * pt < F : NW * nt + PT * wn < O);

  v4f acc[kWI][kWJ];
#pragma unroll
  for (int i = 0; i < kWI; i++)
#pragma unroll
    for (int j = 0; j < kWJ; j++) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  // merged pairs: wave row wm multiplies them with 4 of its column's 8
  // fragments. In a workgroup with merged pairs, wave row 1 takes its
  // fragments in the order 4..7, 0..3 (iteration i holds fragment
  // (i + fo) & 7), so that iterations 0..3 are, for both wave rows, the
  // fragments whose merged products it owns: fragment 4 wm + i of the 16
  // merged pairs goes to accx[i].
  const int fo = extra ? 4 * wm : 0;
  v4f accx[4];
#pragma unroll
  for (int i = 0; i < 4; i++) accx[i] = v4f{0.f, 0.f, 0.f, 0.f};
  bool shifted = false;  // wave-uniform: decoding at scale byte s - kShift

  // the MFMAs of one chunk: activations xc, weight codes wc, the 8 scale bytes
  const int wpos = 4 * lr + ((lc + (lr >> 2)) & 3);  // canonical: this lane's slot in a weight block
  // canonical: this lane's dword 0 of iteration i's weight block is at wlo + 1024 i (i < 4), whi + 1024 (i - 4)
  const int wlo = (8 * wn + fo) * 1024 + 16 * wpos, whi = (8 * wn + 4 - fo) * 1024 + 16 * wpos;
  // prepared: iterations 0..3 read blocks plo + s (dword s of fragments fo .. fo + 3), 4..7 blocks phi + s
  const int plo = wn * kWI + fo, phi = wn * kWI + 4 - fo;
  auto mma_chunk = [&](auto ex, const uint8_t* xc, const uint8_t* wc, const uint8_t* xe,
                       const uint32_t(&sb_in)[kWI]) __attribute__((always_inline)) {
    constexpr bool EX = decltype(ex)::value;
    uint32_t sb[kWI];
    bool big = false;
#pragma unroll
    for (int i = 0; i < kWI; i++) {
      sb[i] = sb_in[i];
      // canonical: the bytes were read during the previous chunk; an empty asm
      // keeps the compiler from moving this chunk's use of them (and so the
      // wait for them) back to where they were read
      if constexpr (CANON) asm volatile("" : "+v"(sb[i]));
      big |= sb[i] >= kShiftFrom;
    }
    if (!shifted && __ballot(big) != 0) {
      shifted = true;
#pragma unroll
      for (int i = 0; i < kWI; i++)
#pragma unroll
        for (int j = 0; j < kWJ; j++) acc[i][j] *= 0.125f;
#pragma unroll
      for (int i = 0; i < 4; i++) accx[i] *= 0.125f;
    }
    float sc[kWI];
#pragma unroll
    for (int i = 0; i < kWI; i++)
      sc[i] = e8m0_operand(!shifted ? sb[i] : (sb[i] > kShift ? sb[i] - kShift : 0u));
#pragma unroll
    for (int s = 0; s < 4; s++) {
      // canonical: lane group c takes dword (s + c) & 3 of its slots at k-step
      // s (the same inputs for every row and column of the MFMA), which with
      // the slot positions puts the 64 lanes' 4-byte reads on 64 distinct
      // banks; its activations follow the same order
      const int sd = CANON ? (s + lc) & 3 : s;
      bf16x8 b[kWJ];
#pragma unroll
      for (int j = 0; j < kWJ; j++) {
        // row p = 64 wm + 16 j + lr (p & 15 = lr); rows past the tile hold zeros (their DMA read past the resource)
        b[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                              &xc[(64 * wm + 16 * j + lr) * ROWB + 16 * ((4 * lc + sd) ^ lr)]));
      }
      bf16x8 bx;
      if constexpr (EX) {
        // merged pair MT + lr of the same k-step (row lr of the merged slot, (MT + lr) & 15 = lr)
        bx = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&xe[lr * ROWB + 16 * ((4 * lc + sd) ^ lr)]));
      }
      uint32_t raw[kWI];
      if constexpr (CANON) {
        // dword sd of this lane's slot of each of the wave's fragments (blocks 8 wn .. 8 wn + 7,
        // iteration i taking fragment (i + fo) & 7)
#pragma unroll
        for (int i = 0; i < kWI; i++)
          raw[i] = *reinterpret_cast<const uint32_t*>(&wc[(i < 4 ? wlo + 1024 * i : whi + 1024 * (i - 4)) + 4 * sd]);
      } else {
        // dword s of this lane's slot of each fragment (8 codes each): blocks s and 4 + s of tile wn
        const u32x4 lo = *reinterpret_cast<const u32x4*>(&wc[(plo + s) * 1024 + 16 * lane]);
        const u32x4 hi = *reinterpret_cast<const u32x4*>(&wc[(phi + s) * 1024 + 16 * lane]);
#pragma unroll
        for (int t = 0; t < 4; t++) raw[t] = lo[t], raw[4 + t] = hi[t];
      }
#pragma unroll
      for (int i = 0; i < kWI; i++) {
        const bf16x8 a = decode8_bf16x8(raw[i], sc[i]);
#pragma unroll
        for (int j = 0; j < kWJ; j++)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[j], acc[i][j], 0, 0, 0);
        if constexpr (EX) {
          if (i < 4) accx[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bx, accx[i], 0, 0, 0);
        }
      }
    }
  };

  if constexpr (!CANON) {
    // One chunk q, activation and weight slots q mod 2 (compile-time): request
    // the activations, weights and scale dwords of chunk q + 1 (into the slots
    // read last during chunk q - 1), multiply chunk q, wait for all of this
    // wave's requests, barrier.
    auto step = [&](int q, auto xs, auto ex) __attribute__((always_inline)) {
      constexpr int R = decltype(xs)::value;
      const uint8_t* xc = R == 0 ? X0 : X1;
      const uint8_t* wc = R == 0 ? W0 : W1;
      if (q + 1 < nq) {
        dma_x(q + 1, R == 0 ? X1 : X0, R == 0 ? XE1 : XE0);
        dma_w(q + 1, R == 0 ? W1 : W0, R ^ 1);
      }
      __builtin_amdgcn_sched_barrier(0);  // keep the requests ahead of the MFMAs
      if (live) {
        // iteration i takes fragment (i + fo) & 7: the scale dwords swap with the fragment halves
        const uint32_t s0 = fo ? wsp[R][1] : wsp[R][0], s1 = fo ? wsp[R][0] : wsp[R][1];
        uint32_t sb[kWI];
#pragma unroll
        for (int i = 0; i < kWI; i++) sb[i] = ((i < 4 ? s0 : s1) >> (8 * (i & 3))) & 0xFFu;
        mma_chunk(ex, xc, wc, R == 0 ? XE0 : XE1, sb);
      }
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's requests have landed
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS reads are done
      __builtin_amdgcn_s_barrier();
    };
    using C0 = std::integral_constant<int, 0>;
    using C1 = std::integral_constant<int, 1>;
    dma_x(0, X0, XE0);
    dma_w(0, W0, 0);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __builtin_amdgcn_s_barrier();
    auto run = [&](auto ex) __attribute__((always_inline)) {
      int q = 0;
      for (; q + 1 < nq; q += 2) {
        step(q, C0{}, ex);
        step(q + 1, C1{}, ex);
      }
      if (q < nq) step(q, C0{}, ex);
    };
    if constexpr (kMerge) {
      if (extra)
        run(std::true_type{});
      else
        run(std::false_type{});
    } else {
      run(std::false_type{});
    }
  } else {
    // One chunk q, activation and weight slots q mod 2 and scale window slot
    // (q >> 1) mod 2 (all compile-time): at a window's first chunk request
    // the next window (into the other window slot, last read during the
    // window before), request the activations and weights of chunk q + 1,
    // read the scale bytes of chunk q + 1 from LDS (their latency hidden
    // behind the MFMAs), multiply chunk q, wait for all of this wave's
    // requests, barrier: the slots written during chunk q were last read
    // during chunk q - 1.
    const int nwin = (G + 7) / 8;
    // the 8 scale bytes of chunk q from window slot sw; a group past G would
    // read another row's byte and reads the zero bytes instead (a choice of
    // address, so nothing waits for these reads before they are used)
    // (the loop with merged pairs keeps them four to a register: it has no
    // registers to spare)
    auto read_sb = [&](int q, const uint8_t* sw, auto& sb) {
      constexpr bool PK = sizeof(sb) == 2 * sizeof(uint32_t);
      const bool in_g = 4 * q + lc < G;
      int off[2];
#pragma unroll
      for (int h = 0; h < 2; h++) off[h] = in_g ? 4 * (q & 1) + lc + sc_lds[h] : kScWin;
      if constexpr (PK) {
#pragma unroll
        for (int h = 0; h < 2; h++) {
          uint32_t v = 0;
#pragma unroll
          for (int t = 0; t < 4; t++) v |= (uint32_t)sw[off[h] + 16 * kScPitch * (4 * h + t)] << (8 * t);
          sb[h] = v;
        }
      } else {
#pragma unroll
        for (int i = 0; i < kWI; i++) sb[i] = sw[off[i >> 2] + 16 * kScPitch * i];
      }
    };
    auto step = [&](int q, auto xs, auto ws, auto ex, auto& sb_cur, auto& sb_next) __attribute__((always_inline)) {
      constexpr bool EX = decltype(ex)::value;
      constexpr int R = decltype(xs)::value, WS = decltype(ws)::value;
      const uint8_t* xc = R == 0 ? X0 : X1;
      const uint8_t* wc = R == 0 ? W0 : W1;
      uint8_t* s_this = WS == 0 ? Sc0 : Sc1;
      uint8_t* s_other = WS == 0 ? Sc1 : Sc0;
      if (R == 0 && (q >> 1) + 1 < nwin) {
#pragma unroll
        for (int m = 0; m < kScDma; m++) dma_sc((q >> 1) + 1, m, s_other);
      }
      if (q + 1 < nq) {
        dma_x(q + 1, R == 0 ? X1 : X0, R == 0 ? XE1 : XE0);
        dma_w(q + 1, R == 0 ? W1 : W0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);  // keep the requests ahead of the MFMAs
      if (live) {
        // chunk q + 1 is in this window (q even) or the next one (q odd)
        if (q + 1 < nq) read_sb(q + 1, R == 0 ? s_this : s_other, sb_next);
        if constexpr (EX) {
          uint32_t sb[kWI];
#pragma unroll
          for (int i = 0; i < kWI; i++) sb[i] = (sb_cur[i >> 2] >> (8 * (i & 3))) & 0xFFu;
          mma_chunk(ex, xc, wc, R == 0 ? XE0 : XE1, sb);
        } else {
          mma_chunk(ex, xc, wc, nullptr, sb_cur);
        }
#pragma unroll
        for (int h = 0; h < (EX ? 2 : kWI); h++) sb_cur[h] = sb_next[h];
      }
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's requests have landed
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS reads are done
      __builtin_amdgcn_s_barrier();
    };
    using C0 = std::integral_constant<int, 0>;
    using C1 = std::integral_constant<int, 1>;
    dma_x(0, X0, XE0);
    dma_w(0, W0, 0);
#pragma unroll
    for (int m = 0; m < kScDma; m++) dma_sc(0, m, Sc0);
    if (tid < kScZero / 16) {
      reinterpret_cast<u32x4*>(Sc0 + kScWin)[tid] = u32x4{0u, 0u, 0u, 0u};
      reinterpret_cast<u32x4*>(Sc1 + kScWin)[tid] = u32x4{0u, 0u, 0u, 0u};
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __builtin_amdgcn_s_barrier();
    // the chunk loop, with or without the merged pairs' MFMAs (two copies of
    // the loop, not a test per chunk: one copy's registers then never meet the other's)
    auto run = [&](auto ex) __attribute__((always_inline)) {
      constexpr bool EX = decltype(ex)::value;
      uint32_t sb_cur[EX ? 2 : kWI], sb_next[EX ? 2 : kWI];
      if (live) read_sb(0, Sc0, sb_cur);
      int q = 0;
      for (; q + 3 < nq; q += 4) {
        step(q, C0{}, C0{}, ex, sb_cur, sb_next);
        step(q + 1, C1{}, C0{}, ex, sb_cur, sb_next);
        step(q + 2, C0{}, C1{}, ex, sb_cur, sb_next);
        step(q + 3, C1{}, C1{}, ex, sb_cur, sb_next);
      }
      if (q < nq) step(q, C0{}, C0{}, ex, sb_cur, sb_next);
      if (q + 1 < nq) step(q + 1, C1{}, C0{}, ex, sb_cur, sb_next);
      if (q + 2 < nq) step(q + 2, C0{}, C1{}, ex, sb_cur, sb_next);
    };
    if constexpr (kMerge) {
      if (extra)
        run(std::true_type{});
      else
        run(std::false_type{});
    } else {
      run(std::false_type{});
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): no DMA may land in LDS after the workgroup ends
  if (shifted) {
#pragma unroll
    for (int i = 0; i < kWI; i++)
#pragma unroll
      for (int j = 0; j < kWJ; j++) acc[i][j] *= 8.0f;
#pragma unroll
    for (int i = 0; i < 4; i++) accx[i] *= 8.0f;
  }

  // lane (lr, lc) of MFMA tile (i, j): pair 64 wm + 16 j + lr, rows 4 lc .. 4 lc + 3 of fragment i
  if constexpr (MODE == kSwiGLU) {
    uint16_t* h = static_cast<uint16_t*>(out);
#pragma unroll
    for (int j = 0; j < kWJ; j++) {
      const int p = 64 * wm + 16 * j + lr;
      if (p >= tl.mlen) continue;
#pragma unroll
      for (int i = 0; i < kWI / 2; i++) {
        const int f = 64 * pt + 16 * i + 4 * lc;  // F % 4 == 0: all four or none
        if (f >= F) continue;
        // silu(g) * u = g / (1 + e^-g) * u, with the hardware reciprocal (1 ulp), rounded to bf16
        // (round to nearest even by the conversion instruction)
        bf16x4 v;
#pragma unroll
        for (int t = 0; t < 4; t++) {
          const float g = acc[i][j][t], u = acc[i + kWI / 2][j][t];
          v[t] = (__bf16)(g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u);
        }
        *reinterpret_cast<bf16x4*>(h + (int64_t)(tl.row0 + p) * F + f) = v;
      }
    }
  } else {
    float* part = static_cast<float*>(out);
#pragma unroll
    for (int j = 0; j < kWJ; j++) {
      const int p = 64 * wm + 16 * j + lr;
      if (p >= tl.mlen) continue;
      float* row = part + (int64_t)(tl.row0 + p) * O;
#pragma unroll
      for (int i = 0; i < kWI; i++) {
        // iteration i's fragment (i + fo) & 7
        const int r = NW * nt + PT * wn + 16 * (i < 4 ? i + fo : i - fo) + 4 * lc;  // O % 4 == 0: all four or none
        if (r < O) *reinterpret_cast<v4f*>(row + r) = acc[i][j];
      }
    }
    if (extra && MT + lr < mtot) {
      // merged pair MT + lr: fragments 4 wm .. 4 wm + 3 of this wave's column
      float* row = part + (int64_t)(tl.row0 + MT + lr) * O;
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int r = NW * nt + PT * wn + 16 * (i + fo) + 4 * lc;
        if (r < O) *reinterpret_cast<v4f*>(row + r) = accx[i];
      }
    }
  }
}

template <int MODE, bool CANON>
hipError_t launch_mode(const uint16_t* x, const uint8_t* pcodes, const uint8_t* pscales, const int32_t* perm,
                       const GemmTile* tiles, const int32_t* n_tiles, int64_t max_tiles, void* out, int64_t x_rows,
                       int K, int O, int G, int F, hipStream_t stream) {
  // O: rows of the prepared matrix (2F for kSwiGLU)
  const int n_wg = (O + NW - 1) / NW, n_ptiles = (O + PT - 1) / PT;
  // 8 XCDs x ceil(max_tiles / 8) M-tiles x the N-tiles
  const int64_t nblk = (max_tiles + 15) / 16 * 16 * n_wg;  // an even number of tiles per XCD
  if (nblk <= 0) return hipSuccess;
  const uint32_t x_bytes = (uint32_t)(x_rows * 64 * G);
  hipLaunchKernelGGL((gemm_regdec_kernel<MODE, CANON>), dim3((unsigned)nblk), dim3(64 * kWaves), 0, stream, x, pcodes, pscales,
                     perm, tiles, n_tiles, out, K, O, G, F, n_wg, n_ptiles, x_bytes);
  return hipGetLastError();
}

}  // namespace

bool gemm_regdec_supported(int64_t T, int64_t O, int64_t G) {
  // 32-bit byte offsets into the activations and into one expert's prepared
  // codes, whole 16-byte output stores
  const int64_t nq = (G + 3) / 4, prepared = (O + PT - 1) / PT * nq * 8192;
  return O % 4 == 0 && T * 64 * G < ((int64_t)1 << 31) && prepared < ((int64_t)1 << 31);
}

bool gemm_regdec_canon_supported(int64_t T, int64_t O, int64_t G) {
  // 32-bit byte offsets into the activations and into one expert's packed
  // bytes, whole 16-byte output stores
  return O % 4 == 0 && T * 64 * G < ((int64_t)1 << 31) && O * G * 16 < ((int64_t)1 << 31);
}

hipError_t launch_gemm_regdec_canon(const uint16_t* x, const uint8_t* packed, const uint8_t* scales,
                                    const int32_t* perm, const GemmTile* tiles, const int32_t* n_tiles,
                                    int64_t max_tiles, float* part, int T, int K, int O, int G, hipStream_t stream) {
  if (!gemm_regdec_canon_supported(T, O, G)) return hipErrorInvalidValue;
  return launch_mode<kGather, true>(x, packed, scales, perm, tiles, n_tiles, max_tiles, part, T, K, O, G, 0, stream);
}

hipError_t launch_gemm_regdec_canon_swiglu(const uint16_t* x, const uint8_t* gu_packed, const uint8_t* gu_scales,
                                           const int32_t* perm, const GemmTile* tiles, const int32_t* n_tiles,
                                           int64_t max_tiles, uint16_t* h, int T, int K, int F, int G,
                                           hipStream_t stream) {
  if (F % 4 || !gemm_regdec_canon_supported(T, 2 * (int64_t)F, G)) return hipErrorInvalidValue;
  return launch_mode<kSwiGLU, true>(x, gu_packed, gu_scales, perm, tiles, n_tiles, max_tiles, h, T, K, 2 * F, G, F,
                                    stream);
}

hipError_t launch_gemm_regdec_canon_direct(const uint16_t* h, const uint8_t* packed, const uint8_t* scales,
                                           const GemmTile* tiles, const int32_t* n_tiles, int64_t max_tiles,
                                           float* part, int64_t P, int O, int G, hipStream_t stream) {
  if (!gemm_regdec_canon_supported(P, O, G)) return hipErrorInvalidValue;
  return launch_mode<kDirect, true>(h, packed, scales, nullptr, tiles, n_tiles, max_tiles, part, P, 1, O, G, 0,
                                    stream);
}

hipError_t launch_gemm_regdec(const uint16_t* x, const uint8_t* pcodes, const uint8_t* pscales, const int32_t* perm,
                              const GemmTile* tiles, const int32_t* n_tiles, int64_t max_tiles, float* part, int T,
                              int K, int O, int G, hipStream_t stream) {
  if (!gemm_regdec_supported(T, O, G)) return hipErrorInvalidValue;
  return launch_mode<kGather, false>(x, pcodes, pscales, perm, tiles, n_tiles, max_tiles, part, T, K, O, G, 0, stream);
}

hipError_t launch_gemm_regdec_swiglu(const uint16_t* x, const uint8_t* pcodes, const uint8_t* pscales,
                                     const int32_t* perm, const GemmTile* tiles, const int32_t* n_tiles,
                                     int64_t max_tiles, uint16_t* h, int T, int K, int F, int G, hipStream_t stream) {
  if (F % 4 || !gemm_regdec_supported(T, 2 * (int64_t)F, G)) return hipErrorInvalidValue;
  return launch_mode<kSwiGLU, false>(x, pcodes, pscales, perm, tiles, n_tiles, max_tiles, h, T, K, 2 * F, G, F, stream);
}

hipError_t launch_gemm_regdec_direct(const uint16_t* h, const uint8_t* pcodes, const uint8_t* pscales,
                                     const GemmTile* tiles, const int32_t* n_tiles, int64_t max_tiles, float* part,
                                     int64_t P, int O, int G, hipStream_t stream) {
  if (!gemm_regdec_supported(P, O, G)) return hipErrorInvalidValue;
  return launch_mode<kDirect, false>(h, pcodes, pscales, nullptr, tiles, n_tiles, max_tiles, part, P, 1, O, G, 0, stream);
}

}  // namespace mxfp4
