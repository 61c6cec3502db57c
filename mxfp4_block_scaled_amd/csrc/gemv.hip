// Decode-shaped path: routing, dequant-GEMV and combine in one launch.
//
// Each workgroup owns 16 output rows and computes, for every selected
// expert, those rows of W_e x_t for all of the expert's pairs, keeps the
// per-pair partial rows in LDS and finally writes
//     y[t, o] = shared[t, o] + sum_{k<K} p[t,k] * partial[(t,k), o]
// with the sum over k in order (page "MXFP4 Routed Expert Linear", "Route,
// weight, and add the shared path"). Only the selected experts' bytes are
// read; each 16-byte group is loaded once (128-bit loads) and used for every
// token of that expert. No decoded weight leaves the registers.
//
// Routing: at most 64 pairs per launch (the host splits tokens into
// chunks). Every wave finds the distinct experts itself: lane i holds pair
// i, and log2(E) ballots give each lane the mask of pairs that chose its
// expert. No LDS and no barrier stand between the routing load and the
// first weight loads.
//
// Arithmetic: v_mfma_f32_16x16x32_bf16. The A operand is 16 weight rows by
// 32 inputs, decoded exactly into bf16 by the scaled FP4 convert (every
// E2M1 value times 2^(s-127) is a bf16 value unless it overflows). The B
// operand is 16 columns, one per (pair, piece): bf16 activations are one
// piece; fp32 activations are split exactly into three bf16 pieces by
// truncation (x = x0 + x1 + x2 for every normal fp32 x), so every product
// w * x_i is exact and the MFMA accumulates in fp32 -- the result keeps
// fp32 accuracy. For MFMA step i lane (r, q) = (lane & 15, lane >> 4)
// holds group 4i+q of row r and feeds its dword j to MFMA j; the B operand
// uses the same permutation of k, so each MFMA sums matching products.
//
// Prepared weights (PREP, the fragment-major layout of prepare_mx_kernel):
// a workgroup's 16 rows are one fragment, and each 1 KB block (one chunk of 4
// groups) is exactly the MFMA operand, lane (r, q) holding group 4i + q of
// row r: an iteration is two 16-byte loads per lane straight into the
// operand registers plus one scale byte each, no transpose. Workgroups are
// ordered so that the four fragments that share a lane's scale dword run on
// the same XCD (one L2).
//
// Memory: an iteration covers 8 groups of the 16 rows. Lane (lr, lg) loads
// group lg of rows lr and 8 + lr (8 whole 128-byte row segments per load)
// and the matching scale bytes; a per-wave LDS buffer with padded rows
// turns that into the MFMA layout without bank conflicts. Work item =
// (distinct expert, chunk of 16 columns, k-split). A wave walks its items as
// one stream of iterations with kRing iterations of loads in flight, across
// item boundaries. The activations are staged once per workgroup in LDS
// (each row followed by an all-zero group that the lanes past a split read).
#include "device_common.h"
#include "launch.h"
#include "wave_routing.h"

namespace mxfp4 {
namespace {

constexpr int kDecThreads = 512;
constexpr int kDecWaves = kDecThreads / 64;
constexpr int kRing = 4;   // iterations (8 groups of the 16 rows each) whose loads a wave keeps in flight
constexpr int kRows = 16;  // output rows per workgroup (one MFMA tile)
constexpr int kTrRow = 8 * 16 + 16;           // bytes per row of a wave's transpose buffer (padded)
constexpr int kTrBytes = kRows * kTrRow + kRows * 8;  // weights then scale bytes
constexpr uint32_t kOobGroup = 0x08000000u;   // group offset beyond any expert's resource
constexpr uint32_t kOob32 = 0x80000000u;      // byte offset beyond any resource
constexpr int kRsrcFlags = 0x00020000;        // raw buffer, 32-bit data format

template <bool XF32, bool PREP>
__global__ void __launch_bounds__(kDecThreads) decode_fused_kernel(
    const void* __restrict__ xv, const uint8_t* __restrict__ packed, const uint8_t* __restrict__ scales,
    const int32_t* __restrict__ sel, const float* __restrict__ p, const void* shared, void* y, int T, int E, int O,
    int G, int K, int S, int nbits, int32_t* __restrict__ n_invalid, int chunk_index) {
  constexpr int NP = XF32 ? 3 : 1;  // bf16 pieces per activation
  extern __shared__ __attribute__((aligned(16))) uint8_t dyn[];
  __shared__ float p_lds[kMaxFusedPairs];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index: uniform, kept in a scalar register
  const int r = lane & 15, q = lane >> 4;
  const int P = T * K, I = 32 * G, IL = I + 40;  // IL: a zero group 32G..32G+31, then 8 of padding
  // PREP: row blocks 32 c + 4 x .. 32 c + 4 x + 3 (x = XCD) for block indices 32 c + x + 8 k, k < 4
  int rb = blockIdx.x;
  if (PREP && (rb | 31) < (int)gridDim.x) rb = (rb & ~31) + ((rb & 7) << 2) + ((rb >> 3) & 3);
  const int o0 = rb * kRows;
  uint16_t* xs = reinterpret_cast<uint16_t*>(dyn);  // [T][NP][IL] bf16
  const size_t xs_bytes = ((size_t)T * NP * IL * 2 + 15) & ~(size_t)15;
  float* part = reinterpret_cast<float*>(dyn + xs_bytes);  // [S][P*NP][16]
  uint8_t* tr = dyn + xs_bytes + (size_t)S * P * NP * kRows * 4 + (size_t)w * kTrBytes;  // this wave's transpose buffer

  // ---- routing input first, then the loads that do not depend on it:
  // p, shared and (up to two 16-byte chunks per thread of) x, written to LDS
  // after the weight loads have been issued
  const int e_l = lane < P ? sel[lane] : -1;
  const float my_p = tid < P ? p[tid] : 0.f;
  const int t_first = tid >> 4, rr_first = tid & 15;
  const bool first_ok = t_first < T && o0 + rr_first < O;
  float sh_first = 0.f;
  if (first_ok) {
    const int64_t yo = (int64_t)t_first * O + o0 + rr_first;
    sh_first = XF32 ? static_cast<const float*>(shared)[yo] : bf16_to_f32(static_cast<const uint16_t*>(shared)[yo]);
  }
  const int cpr = XF32 ? I / 4 : I / 8;  // 16-byte chunks per row of x
  const int nxc = T * cpr;
  const u32x4* x16 = static_cast<const u32x4*>(xv);
  u32x4 xpre0 = {0u, 0u, 0u, 0u}, xpre1 = {0u, 0u, 0u, 0u};
  if (tid < nxc) xpre0 = x16[tid];
  if (tid + kDecThreads < nxc) xpre1 = x16[tid + kDecThreads];

  // ---- routing (every wave, registers only)
  const WaveRoute rt = route_wave(e_l, lane, P, E, nbits);
  const uint64_t valid = rt.valid, pm_u = rt.pm_u;
  const int U = rt.U, e_u = rt.e_u;
  const int n8 = (G + 7) >> 3;
  const int gs8 = (n8 + S - 1) / S;  // iterations (8 groups each) per k-split
  const int ncol_u = lane < U ? __popcll(pm_u) * NP : 0;
  // Usually every expert's (pair, piece) columns fit one chunk of 16, and
  // item i is simply (expert i / S, split i % S); otherwise a prefix sum of
  // the per-expert chunk counts maps items to experts.
  const bool single = __ballot(ncol_u > 16) == 0;
  int incl = 0, NI = U * S;
  if (!single) {
    incl = ((ncol_u + 15) >> 4) * S;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int v = __shfl_up(incl, d, kWave);
      if (lane >= d) incl += v;
    }
    NI = __builtin_amdgcn_readlane(incl, 63);
  }
  struct Item {
    int e, ks, cc, gbeg, nit;
    uint64_t pm;
  };
  auto item_info = [&](int item) {
    Item it;
    int u, rem;
    if (single) {
      u = item / S;
      rem = item - u * S;
    } else {
      u = __popcll(__ballot(lane < U && incl <= item));
      rem = item - (u > 0 ? __builtin_amdgcn_readlane(incl, u - 1) : 0);
    }
    it.cc = rem / S;
    it.ks = rem - it.cc * S;
    it.e = __builtin_amdgcn_readlane(e_u, u);
    it.pm = readlane64(pm_u, u);
    it.gbeg = it.ks * gs8 * 8;
    it.nit = (min(G, it.gbeg + gs8 * 8) - it.gbeg + 7) >> 3;
    return it;
  };
  const int n_mine = NI > w ? (NI - w + kDecWaves - 1) / kDecWaves : 0;
  int total = 0;  // iterations of this wave over all its items
  for (int j = 0; j < n_mine; j++) {
    const int ks = single ? (w + kDecWaves * j) % S : item_info(w + kDecWaves * j).ks;
    const int gb = ks * gs8 * 8;
    total += (min(G, gb + gs8 * 8) - gb + 7) >> 3;
  }

  // ---- load cursor. An iteration covers 8 groups of the 16 rows: lane
  // (lr, lg) = (lane >> 3, lane & 7) loads group gbase + lg of rows lr and
  // 8 + lr (two loads of 8 whole 128-byte row segments each) and their scale
  // bytes. Loads go through buffer resources sized to the selected expert; a
  // row past O and every load past the wave's last item use an offset beyond
  // the resource and read zeros without memory traffic, so every slot issues
  // the same loads and the waits pipeline.
  const int lr = lane >> 3, lg = lane & 7;
  // prepared layout: tile n = o0 / 128, fragment f of the tile, nq chunks of 4 groups
  const int nq = (G + 3) / 4, n_pt = (O + 127) / 128, pf = (o0 >> 4) & 7, pn = o0 >> 7;
  const int nrec_w = PREP ? n_pt * nq * 8192 : O * G * 16, nrec_s = PREP ? n_pt * nq * 512 : O * G;
  int l_j = 0, l_it = 0, l_nit = 1;
  bool l_done = n_mine == 0;
  const uint8_t* l_wb = packed;
  const uint8_t* l_sb = scales;
  uint32_t l_off[2];  // group offset (row-major in the expert) of this lane's first group, per load
  auto l_refresh = [&]() {
    const Item it = item_info(w + kDecWaves * l_j);
    l_nit = it.nit;
    l_wb = packed + (int64_t)it.e * nrec_w;
    l_sb = scales + (int64_t)it.e * nrec_s;
    if constexpr (PREP) {
      // slot of chunk gbeg / 4 (+ 2 per iteration, + 1 for the second load)
      l_off[0] = (uint32_t)(((pn * nq + it.gbeg / 4) * 8 + pf) * 64 + lane);
      l_off[1] = l_off[0] + 512u;
    } else {
#pragma unroll
      for (int t = 0; t < 2; t++) {
        const int o = o0 + 8 * t + lr;
        l_off[t] = o < O ? (uint32_t)(o * G + it.gbeg + lg) : kOobGroup;
      }
    }
  };
  if (!l_done) l_refresh();
  u32x4 rw[kRing][2];
  uint8_t rs[kRing][2];
  auto issue_load = [&](int s) {
    const __amdgpu_buffer_rsrc_t rsw = __builtin_amdgcn_make_buffer_rsrc((void*)l_wb, (short)0, nrec_w, kRsrcFlags);
    const __amdgpu_buffer_rsrc_t rss = __builtin_amdgcn_make_buffer_rsrc((void*)l_sb, (short)0, nrec_s, kRsrcFlags);
#pragma unroll
    for (int t = 0; t < 2; t++) {
      if constexpr (PREP) {
        // chunk gbeg / 4 + 2 it + t; one past the expert's last chunk reads the
        // next tile's codes (or beyond the resource: zeros) and meets the zero
        // activation group; the scale byte: dword of fragments 4 (f / 4) ..,
        // byte f % 4
        const uint32_t si = l_off[t] + 1024u * (uint32_t)l_it;  // slot index
        const uint32_t ck = si >> 9;                             // (tile, chunk) of the slot
        const uint32_t so = ((ck * 2u + (uint32_t)(pf >> 2)) * 64u + (uint32_t)lane) * 4u + (uint32_t)(pf & 3);
        rw[s][t] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsw, (int)(l_done ? kOob32 : si * 16u), 0, kCodeLoadPolicy));
        rs[s][t] = __builtin_amdgcn_raw_buffer_load_b8(rss, (int)(l_done ? kOob32 : so), 0, 0);
      } else {
        // a lane past its split reads the following group (the next row at the
        // end of a row; beyond the resource at the end of the expert); it
        // meets the zero activation group, so it adds nothing
        const uint32_t gi = l_done ? kOobGroup : l_off[t] + (uint32_t)(8 * l_it);
        rw[s][t] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsw, (int)(gi * 16u), 0, kCodeLoadPolicy));
        rs[s][t] = __builtin_amdgcn_raw_buffer_load_b8(rss, (int)gi, 0, 0);
      }
    }
    if (!l_done && ++l_it == l_nit) {
      l_it = 0;
      if (++l_j < n_mine) l_refresh();
      else l_done = true;
    }
  };
#pragma unroll
  for (int s = 0; s < kRing; s++) issue_load(s);

  // ---- x -> LDS (fp32: three bf16 pieces per value), p -> LDS
  auto stage_chunk = [&](int idx, u32x4 v) {
    const int t = idx / cpr, c = idx - t * cpr;
    if constexpr (XF32) {
      uint32_t a0, a1, a2, b0, b1, b2, c0, c1, c2, d0, d1, d2;
      split3(__uint_as_float(v[0]), a0, a1, a2);
      split3(__uint_as_float(v[1]), b0, b1, b2);
      split3(__uint_as_float(v[2]), c0, c1, c2);
      split3(__uint_as_float(v[3]), d0, d1, d2);
      uint16_t* base = xs + (t * NP) * IL + 4 * c;
      *reinterpret_cast<uint2*>(base) = make_uint2(a0 | (b0 << 16), c0 | (d0 << 16));
      *reinterpret_cast<uint2*>(base + IL) = make_uint2(a1 | (b1 << 16), c1 | (d1 << 16));
      *reinterpret_cast<uint2*>(base + 2 * IL) = make_uint2(a2 | (b2 << 16), c2 | (d2 << 16));
    } else {
      *reinterpret_cast<u32x4*>(xs + t * IL + 8 * c) = v;
    }
  };
  if (tid < nxc) stage_chunk(tid, xpre0);
  if (tid + kDecThreads < nxc) stage_chunk(tid + kDecThreads, xpre1);
  // the rest of x (large activations), 8 chunks per thread in flight at a time
  for (int base = tid + 2 * kDecThreads; base < nxc; base += 8 * kDecThreads) {
    u32x4 v[8];
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const int idx = base + i * kDecThreads;
      v[i] = x16[idx < nxc ? idx : 0];
    }
#pragma unroll
    for (int i = 0; i < 8; i++)
      if (base + i * kDecThreads < nxc) stage_chunk(base + i * kDecThreads, v[i]);
  }
  for (int i = tid; i < T * NP * 4; i += kDecThreads)  // the zero group of every row
    *reinterpret_cast<u32x4*>(xs + (i >> 2) * IL + I + 8 * (i & 3)) = u32x4{0u, 0u, 0u, 0u};
  if (tid < P) p_lds[tid] = my_p;
  __syncthreads();

  // ---- compute cursor
  int c_j = 0, c_it = 0, c_gbeg = 0, c_gend = 0, c_nit = 0, c_ks = 0;
  const uint16_t* bptr = xs;  // this lane's B column (a row of xs)
  bool col_ok = false;
  int colidx = 0;
  auto c_refresh = [&]() {
    const Item it = item_info(w + kDecWaves * c_j);
    c_gbeg = it.gbeg;
    c_nit = it.nit;
    c_gend = min(G, it.gbeg + 8 * it.nit);
    c_ks = it.ks;
    const int gc = it.cc * 16 + r;  // column of this lane: (pair, piece)
    col_ok = gc < __popcll(it.pm) * NP;
    const int pi = col_ok ? gc / NP : 0;
    const int pc = col_ok ? gc - pi * NP : 0;
    const int pair = nth_set_bit(it.pm, pi);
    colidx = pair * NP + pc;
    bptr = xs + ((pair / K) * NP + pc) * IL;
  };
  if (n_mine > 0) c_refresh();
  f32x4 acc = {0.f, 0.f, 0.f, 0.f}, acc_hi = {0.f, 0.f, 0.f, 0.f};
  for (int base = 0; base < total; base += kRing) {
#pragma unroll
    for (int s = 0; s < kRing; s++) {
      // keep each slot's work after the previous slot's: consuming slot s
      // must wait for slot s's loads only
      __builtin_amdgcn_sched_barrier(0);
      if (base + s < total) {
        // canonical: transpose through this wave's LDS buffer (rows as loaded,
        // 8 groups each, padded rows: conflict-free both ways), then lane (r, q)
        // takes group 4i + q of row r for MFMA step i; prepared: the loads are
        // already that
        if constexpr (!PREP) {
#pragma unroll
          for (int t = 0; t < 2; t++) {
            *reinterpret_cast<u32x4*>(tr + (8 * t + lr) * kTrRow + lg * 16) = rw[s][t];
            tr[kRows * kTrRow + (8 * t + lr) * 8 + lg] = rs[s][t];
          }
        }
#pragma unroll
        for (int i = 0; i < 2; i++) {
          const u32x4 wq = PREP ? rw[s][i] : *reinterpret_cast<const u32x4*>(tr + r * kTrRow + (4 * i + q) * 16);
          const uint32_t sv = PREP ? (uint32_t)rs[s][i] : (uint32_t)tr[kRows * kTrRow + r * 8 + 4 * i + q];
          uint32_t wd[4][4];
          // scale bytes >= 253 can make E2M1 * 2^(s-127) overflow bf16: such a
          // lane's group is decoded at 2^(s-135) into a second accumulator,
          // multiplied by 2^8 when the item ends (exact)
          const bool hi = sv >= 253u;
          const float sc = e8m0_operand(hi ? sv - 8u : sv);
#pragma unroll
          for (int j = 0; j < 4; j++) decode8_bf16_fast(wq[j], sc, wd[j]);
          // activations of this group; past the split: the zero group
          const int g = c_gbeg + 8 * c_it + 4 * i + q;
          const uint16_t* bp = bptr + 32 * (g < c_gend ? g : G);
          if (__builtin_expect(__ballot(hi) == 0, 1)) {
#pragma unroll
            for (int j = 0; j < 4; j++) {
              const u32x4 bv = *reinterpret_cast<const u32x4*>(bp + 8 * j);
              const u32x4 av = {wd[j][0], wd[j][1], wd[j][2], wd[j][3]};
              acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av),
                                                            __builtin_bit_cast(bf16x8, bv), acc, 0, 0, 0);
            }
          } else {
#pragma unroll
            for (int j = 0; j < 4; j++) {
              const u32x4 bv = *reinterpret_cast<const u32x4*>(bp + 8 * j);
              const u32x4 av = {wd[j][0], wd[j][1], wd[j][2], wd[j][3]};
              const u32x4 z = {0u, 0u, 0u, 0u};
              acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, hi ? z : av),
                                                            __builtin_bit_cast(bf16x8, bv), acc, 0, 0, 0);
              acc_hi = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, hi ? av : z),
                                                               __builtin_bit_cast(bf16x8, bv), acc_hi, 0, 0, 0);
            }
          }
        }
        if (++c_it == c_nit) {
          // acc[i] = row 4q + i of the tile, column r of this item
#pragma unroll
          for (int i = 0; i < 4; i++) acc[i] = fmaf(256.f, acc_hi[i], acc[i]);
          acc_hi = f32x4{0.f, 0.f, 0.f, 0.f};
          if (col_ok) {
            float* dst = part + ((size_t)c_ks * P * NP + colidx) * kRows + 4 * q;
            *reinterpret_cast<f32x4*>(dst) = acc;
          }
          acc = f32x4{0.f, 0.f, 0.f, 0.f};
          c_it = 0;
          if (++c_j < n_mine) c_refresh();
        }
      }
      issue_load(s);
    }
  }
  __syncthreads();

  // ---- combine: k-ordered fp32 sum of p * partial, then shared, one rounding
  for (int idx = tid; idx < T * kRows; idx += kDecThreads) {
    const int t = idx >> 4, rr = idx & 15, oo = o0 + rr;
    if (oo >= O) continue;
    float a = 0.f;
    for (int k = 0; k < K; k++) {
      const int qp = t * K + k;
      if (!((valid >> qp) & 1ull)) continue;
      float v = 0.f;
      for (int ks = 0; ks < S; ks++)
#pragma unroll
        for (int pc = 0; pc < NP; pc++) v += part[((size_t)ks * P * NP + qp * NP + pc) * kRows + rr];
      a = fmaf(p_lds[qp], v, a);
    }
    const int64_t yo = (int64_t)t * O + oo;
    float sh;
    if (idx == tid) sh = sh_first;
    else sh = XF32 ? static_cast<const float*>(shared)[yo] : bf16_to_f32(static_cast<const uint16_t*>(shared)[yo]);
    if constexpr (XF32) static_cast<float*>(y)[yo] = sh + a;
    else static_cast<uint16_t*>(y)[yo] = f32_to_bf16_rne(sh + a);
  }
  if (blockIdx.x == 0 && tid == 0 && n_invalid)
    n_invalid[0] = (chunk_index == 0 ? 0 : n_invalid[0]) + (P - __popcll(valid));
}

int bits_for_experts(int E) {
  int nb = 0;
  while ((1 << nb) < E) nb++;
  return nb;
}

// k-splits: enough work items for the workgroup's waves when few experts
// are selected, every split non-empty.
int decode_splits(int T, int K, int E, int G) {
  const int P = T * K;
  const int uexp = P < E ? P : E;
  int S = uexp >= kDecWaves ? 1 : kDecWaves / uexp;
  const int n8 = (G + 7) / 8;
  if (S > n8) S = n8;
  const int per = (n8 + S - 1) / S;
  return (n8 + per - 1) / per;
}

size_t decode_lds_bytes(int T, int K, int G, int dtype, int S) {
  const int NP = dtype == 0 ? 3 : 1;
  const size_t xs = ((size_t)T * NP * (32 * (size_t)G + 40) * 2 + 15) & ~(size_t)15;
  return xs + (size_t)S * T * K * NP * kRows * 4 + (size_t)kDecWaves * kTrBytes;
}

}  // namespace

int decode_tokens_per_launch(int K, int E, int G, int dtype) {
  if (K > kMaxFusedPairs) return 0;
  int tc = kMaxFusedPairs / K;
  while (tc > 0 && decode_lds_bytes(tc, K, G, dtype, decode_splits(tc, K, E, G)) > (size_t)kDecodeMaxLds) tc--;
  return tc;
}

namespace {
template <bool PREP>
hipError_t launch_decode(const void* x, const uint8_t* packed, const uint8_t* scales, const int32_t* sel,
                         const float* p, const void* shared, void* y, int T, int E, int O, int G, int K, int dtype,
                         int32_t* n_invalid, int chunk_index, hipStream_t stream) {
  if (T * K > kMaxFusedPairs || !gemv_rows_supported(O, G)) return hipErrorInvalidValue;
  const int S = decode_splits(T, K, E, G);
  const size_t lds = decode_lds_bytes(T, K, G, dtype, S);
  if (lds > (size_t)kDecodeMaxLds) return hipErrorInvalidValue;
  const int nb = bits_for_experts(E);
  const dim3 grid((O + kRows - 1) / kRows);
  if (dtype == 0) {
    const hipError_t attr = allow_dynamic_lds<&decode_fused_kernel<true, PREP>>(kDecodeMaxLds);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((decode_fused_kernel<true, PREP>), grid, dim3(kDecThreads), lds, stream, x, packed, scales, sel,
                       p, shared, y, T, E, O, G, K, S, nb, n_invalid, chunk_index);
  } else {
    const hipError_t attr = allow_dynamic_lds<&decode_fused_kernel<false, PREP>>(kDecodeMaxLds);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((decode_fused_kernel<false, PREP>), grid, dim3(kDecThreads), lds, stream, x, packed, scales,
                       sel, p, shared, y, T, E, O, G, K, S, nb, n_invalid, chunk_index);
  }
  return hipGetLastError();
}
}  // namespace

hipError_t launch_decode_fused(const void* x, const uint8_t* packed, const uint8_t* scales, const int32_t* sel,
                               const float* p, const void* shared, void* y, int T, int E, int O, int G, int K,
                               int dtype, int32_t* n_invalid, int chunk_index, hipStream_t stream) {
  return launch_decode<false>(x, packed, scales, sel, p, shared, y, T, E, O, G, K, dtype, n_invalid, chunk_index,
                              stream);
}

hipError_t launch_decode_prepared(const void* x, const uint8_t* pcodes, const uint8_t* pscales, const int32_t* sel,
                                  const float* p, const void* shared, void* y, int T, int E, int O, int G, int K,
                                  int dtype, int32_t* n_invalid, int chunk_index, hipStream_t stream) {
  return launch_decode<true>(x, pcodes, pscales, sel, p, shared, y, T, E, O, G, K, dtype, n_invalid, chunk_index,
                             stream);
}

}  // namespace mxfp4
