// Decode-shaped path, row-contiguous form: routing, dequant-GEMV and
// combine in one launch, on the vector ALUs.
//
// Each workgroup owns R output rows and, for every selected expert, computes
// those rows of W_e x_t for the expert's pairs, keeps the per-pair partial
// rows in LDS and finally writes
//     y[t, o] = shared[t, o] + sum_{k<K} p[t,k] * partial[(t,k), o]
// with the sum over k in order (page "MXFP4 Routed Expert Linear", "Route,
// weight, and add the shared path"). Only the selected experts' bytes are
// read, each 16-byte group once, and it serves every token of its expert.
//
// Memory side. A team of L lanes (L = 16, 32 or 64) reads L consecutive
// groups of one weight row per load, i.e. L*16 contiguous bytes, with the L
// matching scale bytes (contiguous too): a wave-wide load touches 8 cache
// lines of weights and 64/L of scales. Loads go through buffer resources
// sized to the selected expert: a lane with nothing to load passes an
// offset beyond the resource, gets zeros and costs no memory traffic, so
// every slot issues the same loads and the waits pipeline.
//
// Arithmetic (page "MXFP4 Dequant", "How it works": code n is E2M1[n]
// times 2^(s-127)). One group shares its scale, so a lane takes the dot
// product of the group's exact E2M1 values with the activations in fp32
// (fp32 activations: fp32 FMA; bf16 activations: v_dot2_f32_bf16) and
// multiplies it by 2^(s-127) with ldexp: exact, and no decoded weight can
// overflow whatever the scale byte. The L lanes of a row are summed by a
// fixed butterfly when the work item ends, so results are deterministic.
//
// Work item = (distinct expert, batch of up to kTmax of its pairs, k-split,
// group of RW rows). A wave walks its items as one stream of slots (one
// slot = kRpl rows x L groups of one item) with kRing slots of loads in
// flight, across item boundaries. Activations are staged once per
// workgroup in LDS as [token][16-byte chunk c][group], so the L lanes of a
// team read L consecutive 16-byte chunks; one extra all-zero group column
// serves the lanes past the end of a split.
#include "device_common.h"
#include "launch.h"
#include "wave_routing.h"

namespace mxfp4 {
namespace {

#ifndef MXFP4_ROWS_RING
#define MXFP4_ROWS_RING 2  // slots whose loads a wave keeps in flight
#endif
// waves of a large-activation workgroup (16 rows either way)
#ifndef MXFP4_ROWS_BIG_WAVES
#define MXFP4_ROWS_BIG_WAVES 16
#endif
#ifndef MXFP4_ROWS_TMAX
#define MXFP4_ROWS_TMAX 4
#endif
constexpr int kRing = MXFP4_ROWS_RING;
constexpr int kRpl = 2;   // weight rows per lane in a slot
constexpr int kTmax = MXFP4_ROWS_TMAX;  // pairs per work item (an expert with more pairs gets more items)
constexpr int kXPre = 4;   // 16-byte chunks of x per thread loaded with the routing input
// group offset beyond any expert's resource (O * G < 2^27): loads return zero
constexpr uint32_t kOobGroup = 0x08000000u;
constexpr int kRsrcFlags = 0x00020000;  // raw buffer, 32-bit data format

// n / d for 0 <= n < 2^24, d > 0: float estimate, then exact correction.
__device__ __forceinline__ int div_small(int n, int d) {
  int t = (int)((float)n * __builtin_amdgcn_rcpf((float)d));
  while (t > 0 && t * d > n) t--;
  while ((t + 1) * d <= n) t++;
  return t;
}

template <bool XF32, int L, int NW>
__global__ void __launch_bounds__(NW * 64) gemv_rows_kernel(
    const void* __restrict__ xv, const uint8_t* __restrict__ packed, const uint8_t* __restrict__ scales,
    const int32_t* __restrict__ sel, const float* __restrict__ p, const void* shared, void* y, int T, int E, int O,
    int G, int K, int S, int gs, int nbits, int32_t* __restrict__ n_invalid, int chunk_index) {
  constexpr int RI = 64 / L;        // rows per wave-wide load
  constexpr int RW = RI * kRpl;     // rows per work item
  constexpr int R = NW == 4 ? 8 : 16;  // rows per workgroup
  constexpr int NRG = R / RW;       // row groups per workgroup (a power of two)
  constexpr int CH = XF32 ? 8 : 4;  // 16-byte activation chunks per group
  constexpr int kThreads = NW * 64, kWaves = NW;
  static_assert(NRG >= 1 && (NRG & (NRG - 1)) == 0, "row groups");
  extern __shared__ __attribute__((aligned(16))) uint8_t dyn[];
  __shared__ float p_lds[kMaxFusedPairs];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane % L, h = lane / L;  // group within the team's L, row team
  const int P = T * K, GP = G + 1;       // GP: group columns in LDS (last one zero)
  const int o0 = blockIdx.x * R;
  uint8_t* xs = dyn;  // [T][CH][GP] chunks of 16 bytes
  float* part = reinterpret_cast<float*>(dyn + (size_t)T * CH * GP * 16);  // [S][P][R]

  // ---- routing input first, then the loads that do not depend on it
  const int e_l = lane < P ? sel[lane] : -1;
  const float my_p = tid < P ? p[tid] : 0.f;
  const int t_first = tid / R, rr_first = tid - t_first * R;
  const bool first_ok = t_first < T && o0 + rr_first < O;
  float sh_first = 0.f;
  if (first_ok) {
    const int64_t yo = (int64_t)t_first * O + o0 + rr_first;
    sh_first = XF32 ? static_cast<const float*>(shared)[yo] : bf16_to_f32(static_cast<const uint16_t*>(shared)[yo]);
  }
  const int rowc = G * CH, nxc = T * rowc;  // 16-byte chunks of x per token, in all
  const u32x4* x16 = static_cast<const u32x4*>(xv);
  u32x4 xpre[kXPre];
#pragma unroll
  for (int i = 0; i < kXPre; i++) {
    const int q = tid + i * kThreads;
    xpre[i] = x16[q < nxc ? q : 0];
  }

  // ---- routing (every wave, registers only)
  const WaveRoute rt = route_wave(e_l, lane, P, E, nbits);
  const int t_of_pair = div_small(lane, K);  // lane i: token of pair i
  const int U = rt.U;
  // Items are numbered i = q * per_batch + (ks * NRG + rg), q indexing the
  // (expert, pair batch) pairs in expert order. Usually no expert has more
  // than kTmax pairs and q is the expert; otherwise a prefix sum of the
  // per-expert batch counts maps q to its expert. A wave takes items
  // w, w + NW, ...; its cursors step through them without divisions.
  const int per_batch = S * NRG;
  const int ntok_u = lane < U ? __popcll(rt.pm_u) : 0;
  const bool single = __ballot(ntok_u > kTmax) == 0;
  int inclb = 0, NQ = U;
  if (!single) {
    inclb = (ntok_u + kTmax - 1) / kTmax;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int v = __shfl_up(inclb, d, 64);
      if (lane >= d) inclb += v;
    }
    NQ = __builtin_amdgcn_readlane(inclb, 63);
  }
  const int NI = NQ * per_batch;
  struct Cursor {
    int q, within;  // (expert, batch) index and position inside it
  };
  auto first_item = [&]() {
    Cursor c{0, w};
    while (c.within >= per_batch) c.within -= per_batch, c.q++;
    return c;
  };
  auto next_item = [&](Cursor& c) {
    c.within += kWaves;
    while (c.within >= per_batch) c.within -= per_batch, c.q++;
  };
  struct Item {
    int e, b, ks, rg, gbeg, gend, nm;
    uint64_t pm;
  };
  auto item_info = [&](const Cursor& c) {
    Item it;
    int u = c.q;
    it.b = 0;
    if (!single) {
      u = __popcll(__ballot(lane < U && inclb <= c.q));
      it.b = c.q - (u > 0 ? __builtin_amdgcn_readlane(inclb, u - 1) : 0);
    }
    it.ks = c.within / NRG;
    it.rg = c.within % NRG;
    it.e = __builtin_amdgcn_readlane(rt.e_u, u);
    it.pm = readlane64(rt.pm_u, u);
    it.gbeg = it.ks * gs;
    it.gend = min(G, it.gbeg + gs);
    it.nm = (it.gend - it.gbeg + L - 1) / L;
    return it;
  };
  const int n_mine = NI > w ? (NI - w + kWaves - 1) / kWaves : 0;
  int total = 0;  // slots of this wave over all its items
  {
    Cursor c = first_item();
    for (int jj = 0; jj < n_mine; jj++, next_item(c)) {
      const int gb = (c.within / NRG) * gs;
      total += (min(G, gb + gs) - gb + L - 1) / L;
    }
  }

  // ---- load cursor: every slot issues kRpl 16-byte weight loads and kRpl
  // scale-byte loads, at per-row offsets fixed when the item starts. A row
  // past the end of the matrix reads beyond the expert's buffer resource
  // (zeros, no memory traffic); a lane past the end of its k-split reads
  // whatever group follows, which adds nothing: its activations are the
  // zero column.
  const int nrec_w = O * G * 16, nrec_s = O * G;
  int l_j = 0, l_m = 0, l_nm = 1;
  bool l_done = n_mine == 0;
  Cursor l_cur = first_item();
  const uint8_t* l_wb = packed;
  const uint8_t* l_sb = scales;
  uint32_t l_off[kRpl];  // this lane's first group (row-major in the expert), per row
  auto l_refresh = [&]() {
    const Item it = item_info(l_cur);
    l_nm = it.nm;
    l_wb = packed + (int64_t)it.e * nrec_w;
    l_sb = scales + (int64_t)it.e * nrec_s;
#pragma unroll
    for (int i = 0; i < kRpl; i++) {
      const int o = o0 + it.rg * RW + i * RI + h;
      l_off[i] = o < O ? (uint32_t)(o * G + it.gbeg + j) : kOobGroup;
    }
  };
  if (!l_done) l_refresh();
  u32x4 rw[kRing][kRpl];
  uint8_t rs[kRing][kRpl];
  auto issue_load = [&](int s) {
    const __amdgpu_buffer_rsrc_t rsw = __builtin_amdgcn_make_buffer_rsrc((void*)l_wb, (short)0, nrec_w, kRsrcFlags);
    const __amdgpu_buffer_rsrc_t rss = __builtin_amdgcn_make_buffer_rsrc((void*)l_sb, (short)0, nrec_s, kRsrcFlags);
#pragma unroll
    for (int i = 0; i < kRpl; i++) {
      // past the wave's last item: beyond the resource (zeros, no memory traffic)
      const uint32_t gi = l_done ? kOobGroup : l_off[i] + (uint32_t)(L * l_m);
      rw[s][i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsw, (int)(gi * 16u), 0, kCodeLoadPolicy));
      rs[s][i] = __builtin_amdgcn_raw_buffer_load_b8(rss, (int)gi, 0, 0);
    }
    if (!l_done && ++l_m == l_nm) {
      l_m = 0;
      next_item(l_cur);
      if (++l_j < n_mine) l_refresh();
      else l_done = true;
    }
  };
#pragma unroll
  for (int s = 0; s < kRing; s++) issue_load(s);

  // ---- x -> LDS as [t][c][g], plus the zero column g = G; p -> LDS
  auto stage_chunk = [&](int q, u32x4 v) {
    const int t = div_small(q, rowc), r2 = q - t * rowc;
    const int g = r2 / CH, c = r2 % CH;
    *reinterpret_cast<u32x4*>(xs + ((size_t)(t * CH + c) * GP + g) * 16) = v;
  };
#pragma unroll
  for (int i = 0; i < kXPre; i++)
    if (tid + i * kThreads < nxc) stage_chunk(tid + i * kThreads, xpre[i]);
  // the rest of x (large activations), 8 chunks per thread in flight at a time
  for (int base = tid + kXPre * kThreads; base < nxc; base += 8 * kThreads) {
    u32x4 v[8];
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const int idx = base + i * kThreads;
      v[i] = x16[idx < nxc ? idx : 0];
    }
#pragma unroll
    for (int i = 0; i < 8; i++)
      if (base + i * kThreads < nxc) stage_chunk(base + i * kThreads, v[i]);
  }
  for (int i = tid; i < T * CH; i += kThreads)
    *reinterpret_cast<u32x4*>(xs + ((size_t)i * GP + G) * 16) = u32x4{0u, 0u, 0u, 0u};
  if (tid < P) p_lds[tid] = my_p;
  __syncthreads();

  // ---- compute cursor
  int c_j = 0, c_m = 0, c_nm = 1, c_gbeg = 0, c_gend = 0, c_ks = 0, c_rg = 0, c_nt = 0;
  int c_pt[kTmax];  // pair | token << 8 of the item's pairs
  const int xrow = CH * GP * 16;  // LDS bytes per token of x
  Cursor c_cur = first_item();
  auto c_refresh = [&]() {
    const Item it = item_info(c_cur);
    c_gbeg = it.gbeg;
    c_gend = it.gend;
    c_nm = it.nm;
    c_ks = it.ks;
    c_rg = it.rg;
    c_nt = min(kTmax, __popcll(it.pm) - it.b * kTmax);
    uint64_t m = it.pm;
    for (int sk = 0; sk < it.b * kTmax; sk++) m &= m - 1;
#pragma unroll
    for (int tt = 0; tt < kTmax; tt++) {
      const int pair = m ? (int)__builtin_ctzll(m) : 0;
      m &= m - 1;
      c_pt[tt] = pair | (__builtin_amdgcn_readlane(t_of_pair, pair) << 8);
    }
  };
  if (n_mine > 0) c_refresh();
  float acc[kRpl][kTmax];
#pragma unroll
  for (int i = 0; i < kRpl; i++)
#pragma unroll
    for (int tt = 0; tt < kTmax; tt++) acc[i][tt] = 0.f;

  for (int base = 0; base < total; base += kRing) {
#pragma unroll
    for (int s = 0; s < kRing; s++) {
      // consuming slot s waits for slot s's loads only
      __builtin_amdgcn_sched_barrier(0);
      if (base + s < total) {
        const int g = c_gbeg + j + L * c_m;
        const int gx = g < c_gend ? g : G;  // past the split: the zero column
        // the group's dot product is taken on the unscaled E2M1 values and
        // then multiplied by 2^(s-127) (exact, and no decoded weight can
        // overflow, whatever the scale byte)
        int ex[kRpl];
#pragma unroll
        for (int i = 0; i < kRpl; i++) ex[i] = (int)rs[s][i] - 127;
        const float one = e8m0_operand(127u);
        if constexpr (!XF32) {
          uint32_t wd[kRpl][16];
#pragma unroll
          for (int i = 0; i < kRpl; i++)
#pragma unroll
            for (int wi = 0; wi < 4; wi++) decode8_bf16_fast(rw[s][i][wi], one, &wd[i][4 * wi]);
#pragma unroll
          for (int tt = 0; tt < kTmax; tt++) {
            if (tt < c_nt) {
              const uint8_t* xb = xs + (c_pt[tt] >> 8) * xrow + gx * 16;
              u32x4 xc[CH];
#pragma unroll
              for (int c = 0; c < CH; c++) xc[c] = *reinterpret_cast<const u32x4*>(xb + (size_t)c * GP * 16);
#pragma unroll
              for (int i = 0; i < kRpl; i++) {
                float a = 0.f;
#pragma unroll
                for (int k = 0; k < 16; k++)
                  a = dot2_bf16(wd[i][k], xc[k >> 2][k & 3], a);
                acc[i][tt] += __builtin_amdgcn_ldexpf(a, ex[i]);
              }
            }
          }
        } else {
#pragma unroll
          for (int tt = 0; tt < kTmax; tt++) {
            if (tt < c_nt) {
              const uint8_t* xb = xs + (c_pt[tt] >> 8) * xrow + gx * 16;
              float a[kRpl];
#pragma unroll
              for (int i = 0; i < kRpl; i++) a[i] = 0.f;
              // the group's 32 activations in two halves of 16 (registers)
#pragma unroll
              for (int half = 0; half < 2; half++) {
                u32x4 xc[4];
#pragma unroll
                for (int c = 0; c < 4; c++)
                  xc[c] = *reinterpret_cast<const u32x4*>(xb + (size_t)(4 * half + c) * GP * 16);
#pragma unroll
                for (int i = 0; i < kRpl; i++)
#pragma unroll
                  for (int wh = 0; wh < 2; wh++) {
                    const uint32_t wq = rw[s][i][2 * half + wh];
                    const f32x2 v0 = cvt_fp4x2_f32<0>(wq, one), v1 = cvt_fp4x2_f32<1>(wq, one);
                    const f32x2 v2 = cvt_fp4x2_f32<2>(wq, one), v3 = cvt_fp4x2_f32<3>(wq, one);
                    const u32x4 xa = xc[2 * wh], xb2 = xc[2 * wh + 1];
                    a[i] = fmaf(v0.x, __uint_as_float(xa[0]), a[i]);
                    a[i] = fmaf(v0.y, __uint_as_float(xa[1]), a[i]);
                    a[i] = fmaf(v1.x, __uint_as_float(xa[2]), a[i]);
                    a[i] = fmaf(v1.y, __uint_as_float(xa[3]), a[i]);
                    a[i] = fmaf(v2.x, __uint_as_float(xb2[0]), a[i]);
                    a[i] = fmaf(v2.y, __uint_as_float(xb2[1]), a[i]);
                    a[i] = fmaf(v3.x, __uint_as_float(xb2[2]), a[i]);
                    a[i] = fmaf(v3.y, __uint_as_float(xb2[3]), a[i]);
                  }
              }
#pragma unroll
              for (int i = 0; i < kRpl; i++) acc[i][tt] += __builtin_amdgcn_ldexpf(a[i], ex[i]);
            }
          }
        }
        if (++c_m == c_nm) {
          // the item is done: sum each row over its L lanes, store partials
#pragma unroll
          for (int tt = 0; tt < kTmax; tt++) {
            if (tt < c_nt) {
#pragma unroll
              for (int i = 0; i < kRpl; i++) {
                float v = acc[i][tt];
#pragma unroll
                for (int m = 1; m < L; m <<= 1) v += __shfl_xor(v, m, 64);
                if (j == 0) part[((size_t)c_ks * P + (c_pt[tt] & 255)) * R + c_rg * RW + i * RI + h] = v;
              }
            }
          }
#pragma unroll
          for (int i = 0; i < kRpl; i++)
#pragma unroll
            for (int tt = 0; tt < kTmax; tt++) acc[i][tt] = 0.f;
          c_m = 0;
          next_item(c_cur);
          if (++c_j < n_mine) c_refresh();
        }
      }
      issue_load(s);
    }
  }
  __syncthreads();

  // ---- combine: k-ordered fp32 sum of p * partial, then shared, one rounding
  for (int idx = tid; idx < T * R; idx += kThreads) {
    const int t = idx / R, rr = idx % R, oo = o0 + rr;
    if (oo >= O) continue;
    float a = 0.f;
    for (int k = 0; k < K; k++) {
      const int qp = t * K + k;
      if (!((rt.valid >> qp) & 1ull)) continue;
      float v = 0.f;
      for (int ks = 0; ks < S; ks++) v += part[((size_t)ks * P + qp) * R + rr];
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
    n_invalid[0] = (chunk_index == 0 ? 0 : n_invalid[0]) + (P - __popcll(rt.valid));
}

int bits_for(int E) {
  int nb = 0;
  while ((1 << nb) < E) nb++;
  return nb;
}

// Lanes per row for a split of gs groups: the fewest idle lanes in the last
// load of a row, the wider team on a tie.
int lanes_per_row(int gs) {
  int best = 64, best_waste = (gs + 63) / 64 * 64 - gs;
  for (int L : {32, 16}) {
    const int waste = (gs + L - 1) / L * L - gs;
    if (waste < best_waste) best = L, best_waste = waste;
  }
  return best;
}

struct RowsPlan {
  int R, NW, L, S, gs;  // rows and waves per workgroup, lanes per row, k-splits, groups per split
};

// k-splits: enough work items for the workgroup's waves when few experts
// are selected, every split non-empty.
// Small activations: 4-wave workgroups of 8 rows (many workgroups, all
// resident at once). Large activations: 16-wave workgroups of 16 rows: the
// staged x limits a CU to one workgroup, whose 16 waves (4 per SIMD) keep
// enough loads in flight and hide the arithmetic.
RowsPlan rows_plan(int T, int K, int E, int G, int dtype) {
  const int P = T * K, uexp = P < E ? P : E;
  const int64_t xbytes = (int64_t)T * G * 32 * (dtype == 0 ? 4 : 2);
  const bool big = xbytes > 32 * 1024;
  const int NW = big ? MXFP4_ROWS_BIG_WAVES : 4, R = big ? 16 : 8;
  RowsPlan pl{R, NW, 64, 1, G};
  for (int S = 1; S <= G; S++) {
    const int gs = (G + S - 1) / S;
    const int L = lanes_per_row(gs);
    const int nrg = R / (64 / L * kRpl);
    pl = RowsPlan{R, NW, L, (G + gs - 1) / gs, gs};
    if ((int64_t)uexp * pl.S * nrg >= NW) break;
  }
  return pl;
}

size_t rows_lds_bytes(int T, int K, int G, int dtype, int S, int R) {
  const int CH = dtype == 0 ? 8 : 4;
  return (size_t)T * CH * (G + 1) * 16 + (size_t)S * T * K * R * 4;
}

template <bool XF32, int L, int NW>
hipError_t launch_rows_nw(const RowsPlan& pl, size_t lds, const void* x, const uint8_t* packed, const uint8_t* scales,
                       const int32_t* sel, const float* p, const void* shared, void* y, int T, int E, int O, int G,
                       int K, int32_t* n_invalid, int chunk_index, hipStream_t stream) {
  const hipError_t attr = allow_dynamic_lds<&gemv_rows_kernel<XF32, L, NW>>(kDecodeMaxLds);
  if (attr != hipSuccess) return attr;
  const dim3 grid((O + pl.R - 1) / pl.R);
  hipLaunchKernelGGL((gemv_rows_kernel<XF32, L, NW>), grid, dim3(NW * 64), lds, stream, x, packed, scales, sel, p,
                     shared, y, T, E, O, G, K, pl.S, pl.gs, bits_for(E), n_invalid, chunk_index);
  return hipGetLastError();
}

template <bool XF32, int L>
hipError_t launch_rows(const RowsPlan& pl, size_t lds, const void* x, const uint8_t* packed, const uint8_t* scales,
                       const int32_t* sel, const float* p, const void* shared, void* y, int T, int E, int O, int G,
                       int K, int32_t* n_invalid, int chunk_index, hipStream_t stream) {
  if (pl.NW == 4)
    return launch_rows_nw<XF32, L, 4>(pl, lds, x, packed, scales, sel, p, shared, y, T, E, O, G, K, n_invalid,
                                      chunk_index, stream);
  return launch_rows_nw<XF32, L, MXFP4_ROWS_BIG_WAVES>(pl, lds, x, packed, scales, sel, p, shared, y, T, E, O, G,
                                                      K, n_invalid, chunk_index, stream);
}

}  // namespace

bool gemv_rows_supported(int O, int G) { return (int64_t)O * G * 16 < (int64_t)1 << 31; }

int gemv_rows_tokens_per_launch(int K, int E, int G, int dtype) {
  if (K > kMaxFusedPairs) return 0;
  int tc = kMaxFusedPairs / K;
  while (tc > 0) {
    const RowsPlan pl = rows_plan(tc, K, E, G, dtype);
    if (rows_lds_bytes(tc, K, G, dtype, pl.S, pl.R) <= (size_t)kDecodeMaxLds) break;
    tc--;
  }
  return tc;
}

hipError_t launch_gemv_rows(const void* x, const uint8_t* packed, const uint8_t* scales, const int32_t* sel,
                            const float* p, const void* shared, void* y, int T, int E, int O, int G, int K, int dtype,
                            int32_t* n_invalid, int chunk_index, hipStream_t stream) {
  if (T * K > kMaxFusedPairs || !gemv_rows_supported(O, G)) return hipErrorInvalidValue;
  const RowsPlan pl = rows_plan(T, K, E, G, dtype);
  const size_t lds = rows_lds_bytes(T, K, G, dtype, pl.S, pl.R);
  if (lds > (size_t)kDecodeMaxLds) return hipErrorInvalidValue;
  const bool f32 = dtype == 0;
  switch (pl.L) {
    case 16:
      return f32 ? launch_rows<true, 16>(pl, lds, x, packed, scales, sel, p, shared, y, T, E, O, G, K, n_invalid,
                                         chunk_index, stream)
                 : launch_rows<false, 16>(pl, lds, x, packed, scales, sel, p, shared, y, T, E, O, G, K, n_invalid,
                                          chunk_index, stream);
    case 32:
      return f32 ? launch_rows<true, 32>(pl, lds, x, packed, scales, sel, p, shared, y, T, E, O, G, K, n_invalid,
                                         chunk_index, stream)
                 : launch_rows<false, 32>(pl, lds, x, packed, scales, sel, p, shared, y, T, E, O, G, K, n_invalid,
                                          chunk_index, stream);
    default:
      return f32 ? launch_rows<true, 64>(pl, lds, x, packed, scales, sel, p, shared, y, T, E, O, G, K, n_invalid,
                                         chunk_index, stream)
                 : launch_rows<false, 64>(pl, lds, x, packed, scales, sel, p, shared, y, T, E, O, G, K, n_invalid,
                                          chunk_index, stream);
  }
}

}  // namespace mxfp4
