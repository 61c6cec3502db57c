// Decode-shaped path: one launch does the bucketing, the dequant-GEMV and
// the combine for a few tokens.
//
// Each workgroup owns a tile of output rows and computes, for every selected
// expert, that expert's rows of W_e x_t for all of its pairs; it keeps those
// per-pair partial rows in LDS and finally writes
//     y[t, o] = shared[t, o] + sum_{k<K} p[t,k] * partial[(t,k), o]
// with the sum over k in order (page "MXFP4 Routed Expert Linear", "Route,
// weight, and add the shared path"). Only the selected experts' bytes are
// read; each 16-byte group is loaded once and used for every token of that
// expert. No decoded weight leaves the registers.
//
// Bucketing in the workgroup: every pair gets its position in the stable
// sort by expert by counting the pairs before it (ties by pair number), so
// the segments, their order and the positions are the same in every
// workgroup and every run.
#include "device_common.h"
#include "launch.h"

namespace mxfp4 {
namespace {

__device__ __forceinline__ uint64_t lanes_below(int lane) { return (lane == 0) ? 0ull : (~0ull >> (64 - lane)); }

struct FusedBuckets {
  int key[kMaxFusedPairs];           // expert of pair i, or E when out of range
  int sorted_pair[kMaxFusedPairs];   // pair at sorted position r
  int slot_of_pair[kMaxFusedPairs];  // sorted position of pair i, -1 if out of range
  int seg_expert[kMaxFusedPairs];    // expert of segment u (increasing)
  int seg_begin[kMaxFusedPairs + 1]; // first sorted position of segment u
  int n_seg;
  int n_invalid;
  int wave_cnt[16];
};

template <int NT>
__device__ void bucket_in_block(const int32_t* __restrict__ sel, int P, int E, FusedBuckets& b) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  if (tid == 0) b.n_invalid = 0;
  __syncthreads();
  for (int i = tid; i < P; i += NT) {
    const int e = sel[i];
    const bool ok = e >= 0 && e < E;
    b.key[i] = ok ? e : E;
    if (!ok) atomicAdd(&b.n_invalid, 1);
  }
  __syncthreads();
  for (int i = tid; i < P; i += NT) {
    const int ki = b.key[i];
    int r = 0;
    for (int j = 0; j < P; j++) {
      const int kj = b.key[j];
      r += (kj < ki) | ((kj == ki) & (j < i));
    }
    b.sorted_pair[r] = i;
    b.slot_of_pair[i] = (ki < E) ? r : -1;
  }
  __syncthreads();
  int base = 0;
  for (int r0 = 0; r0 < P; r0 += NT) {
    const int r = r0 + tid;
    bool start = false;
    int kr = E;
    if (r < P) {
      kr = b.key[b.sorted_pair[r]];
      start = kr < E && (r == 0 || b.key[b.sorted_pair[r - 1]] != kr);
    }
    const uint64_t m = __ballot(start);
    if (lane == 0) b.wave_cnt[w] = __popcll(m);
    __syncthreads();
    int before = 0, tot = 0;
    for (int i = 0; i < NT / 64; i++) {
      const int c = b.wave_cnt[i];
      before += (i < w) ? c : 0;
      tot += c;
    }
    if (start) {
      const int u = base + before + __popcll(m & lanes_below(lane));
      b.seg_expert[u] = kr;
      b.seg_begin[u] = r;
    }
    base += tot;
    __syncthreads();
  }
  if (tid == 0) {
    b.n_seg = base;
    b.seg_begin[base] = P - b.n_invalid;
  }
  __syncthreads();
}

// ------------------------------------------------------------------ fp32
// One wave per (expert, row): lane j takes groups j, j+64, ...; the 32
// unscaled table values of a group are dotted with x in fp32 and the group
// partial is scaled by 2^(s-127) with ldexp (the same value as scaling every
// weight first, up to where fp32 under- or overflows); a fixed butterfly sums
// the 64 lanes.
template <int R>
__global__ void __launch_bounds__(256) gemv_f32_fused_kernel(
    const float* __restrict__ x, const uint8_t* __restrict__ packed, const uint8_t* __restrict__ scales,
    const int32_t* __restrict__ sel, const float* __restrict__ p, const float* shared, float* y, int T, int E, int O,
    int G, int K, int32_t* __restrict__ n_invalid, int chunk_index) {
  __shared__ FusedBuckets bk;
  __shared__ float part[kMaxFusedPairs * R];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int P = T * K;
  const int64_t I = 32 * (int64_t)G;
  bucket_in_block<256>(sel, P, E, bk);
  const int U = bk.n_seg;
  const int o0 = blockIdx.x * R;
  for (int it = w; it < U * R; it += 4) {
    const int u = it / R, r = it - u * R, o = o0 + r;
    if (o >= O) continue;
    const int e = bk.seg_expert[u], sb = bk.seg_begin[u], n = bk.seg_begin[u + 1] - sb;
    const uint8_t* prow = packed + ((int64_t)e * O + o) * (int64_t)G * 16;
    const uint8_t* srow = scales + ((int64_t)e * O + o) * (int64_t)G;
    for (int q0 = 0; q0 < n; q0 += 4) {
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
      const float* xr[4];
#pragma unroll
      for (int qi = 0; qi < 4; qi++) {
        const int pr = (q0 + qi < n) ? bk.sorted_pair[sb + q0 + qi] : 0;
        xr[qi] = x + (int64_t)(pr / K) * I;
      }
      for (int g = lane; g < G; g += 64) {
        const uint4 wv = *reinterpret_cast<const uint4*>(prow + (int64_t)g * 16);
        const int s = srow[g];
        float wf[32];
        decode8_f32_unscaled(wv.x, wf);
        decode8_f32_unscaled(wv.y, wf + 8);
        decode8_f32_unscaled(wv.z, wf + 16);
        decode8_f32_unscaled(wv.w, wf + 24);
#pragma unroll
        for (int qi = 0; qi < 4; qi++) {
          if (q0 + qi < n) {
            const float4* xv = reinterpret_cast<const float4*>(xr[qi] + 32 * g);
            float gp = 0.f;
#pragma unroll
            for (int v = 0; v < 8; v++) {
              const float4 xx = xv[v];
              gp = fmaf(wf[4 * v + 0], xx.x, gp);
              gp = fmaf(wf[4 * v + 1], xx.y, gp);
              gp = fmaf(wf[4 * v + 2], xx.z, gp);
              gp = fmaf(wf[4 * v + 3], xx.w, gp);
            }
            acc[qi] += __builtin_amdgcn_ldexpf(gp, s - 127);
          }
        }
      }
#pragma unroll
      for (int qi = 0; qi < 4; qi++) {
        if (q0 + qi < n) {
          const float v = wave_sum(acc[qi]);
          if (lane == 0) part[(sb + q0 + qi) * R + r] = v;
        }
      }
    }
  }
  __syncthreads();
  for (int idx = tid; idx < T * R; idx += 256) {
    const int t = idx / R, r = idx - t * R, o = o0 + r;
    if (o >= O) continue;
    float a = 0.f;
    for (int k = 0; k < K; k++) {
      const int sp = bk.slot_of_pair[t * K + k];
      if (sp >= 0) a = fmaf(p[t * K + k], part[sp * R + r], a);
    }
    const int64_t yo = (int64_t)t * O + o;
    y[yo] = shared[yo] + a;
  }
  if (blockIdx.x == 0 && tid == 0 && n_invalid) n_invalid[0] = (chunk_index == 0 ? 0 : n_invalid[0]) + bk.n_invalid;
}

// ------------------------------------------------------------------ bf16
// One wave per (expert, 16-row tile): v_mfma_f32_16x16x32_bf16 with the
// decoded weights as the 16 x 32 operand and up to 16 of the expert's pairs
// as the 32 x 16 operand. Lane (r, q) = (lane & 15, lane >> 4) loads the
// whole 16-byte group 4*it + q of row r and feeds its dword j to MFMA j;
// the x operand uses the same permutation of k, so each MFMA still sums
// matching weight/activation products. The scale is applied in the decode
// (exact in bf16), so the MFMA accumulates W_e x exactly as defined.
template <int WAVES>
__global__ void __launch_bounds__(WAVES * 64) gemv_bf16_fused_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ packed, const uint8_t* __restrict__ scales,
    const int32_t* __restrict__ sel, const float* __restrict__ p, const uint16_t* shared, uint16_t* y, int T, int E,
    int O, int G, int K, int32_t* __restrict__ n_invalid, int chunk_index) {
  constexpr int R = 16;
  __shared__ FusedBuckets bk;
  __shared__ float part[kMaxFusedPairs * R];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int r = lane & 15, q = lane >> 4;
  const int P = T * K;
  const int64_t I = 32 * (int64_t)G;
  bucket_in_block<WAVES * 64>(sel, P, E, bk);
  const int U = bk.n_seg;
  const int o0 = blockIdx.x * R;
  const int o = o0 + r;
  const bool row_ok = o < O;
  for (int u = w; u < U; u += WAVES) {
    const int e = bk.seg_expert[u], sb = bk.seg_begin[u], n = bk.seg_begin[u + 1] - sb;
    const uint8_t* prow = packed + ((int64_t)e * O + (row_ok ? o : 0)) * (int64_t)G * 16;
    const uint8_t* srow = scales + ((int64_t)e * O + (row_ok ? o : 0)) * (int64_t)G;
    for (int c0 = 0; c0 < n; c0 += 16) {
      const bool col_ok = c0 + r < n;
      const int pr = col_ok ? bk.sorted_pair[sb + c0 + r] : 0;
      const uint16_t* xrow = x + (int64_t)(pr / K) * I;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
      for (int g0 = 0; g0 < G; g0 += 4) {
        const int g = g0 + q;
        const bool g_ok = g < G;
        u32x4 wv = {0u, 0u, 0u, 0u};
        uint32_t s = 127;
        if (row_ok && g_ok) {
          wv = *reinterpret_cast<const u32x4*>(prow + (int64_t)g * 16);
          s = srow[g];
        }
        u32x4 xv[4];
#pragma unroll
        for (int j = 0; j < 4; j++) xv[j] = u32x4{0u, 0u, 0u, 0u};
        if (col_ok && g_ok) {
          const u32x4* xp = reinterpret_cast<const u32x4*>(xrow + 32 * (int64_t)g);
#pragma unroll
          for (int j = 0; j < 4; j++) xv[j] = xp[j];
        }
        uint32_t wd[4][4];
        if (__builtin_expect(__ballot(s == 255) != 0, 0)) {
#pragma unroll
          for (int j = 0; j < 4; j++) {
            if (s == 255) decode8_bf16_slow(wv[j], s, wd[j]);
            else decode8_bf16_fast(wv[j], e8m0_operand(s), wd[j]);
          }
        } else {
          const float sc = e8m0_operand(s);
#pragma unroll
          for (int j = 0; j < 4; j++) decode8_bf16_fast(wv[j], sc, wd[j]);
        }
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const u32x4 a = {wd[j][0], wd[j][1], wd[j][2], wd[j][3]};
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, xv[j]),
                                                        acc, 0, 0, 0);
        }
      }
      // acc[i] = row 4q + i of the tile, column (pair) lane & 15
      if (col_ok) {
        const int pos = sb + c0 + r;
#pragma unroll
        for (int i = 0; i < 4; i++) part[pos * R + 4 * q + i] = acc[i];
      }
    }
  }
  __syncthreads();
  for (int idx = tid; idx < T * R; idx += WAVES * 64) {
    const int t = idx / R, rr = idx - t * R, oo = o0 + rr;
    if (oo >= O) continue;
    float a = 0.f;
    for (int k = 0; k < K; k++) {
      const int sp = bk.slot_of_pair[t * K + k];
      if (sp >= 0) a = fmaf(p[t * K + k], part[sp * R + rr], a);
    }
    const int64_t yo = (int64_t)t * O + oo;
    y[yo] = f32_to_bf16_rne(bf16_to_f32(shared[yo]) + a);
  }
  if (blockIdx.x == 0 && tid == 0 && n_invalid) n_invalid[0] = (chunk_index == 0 ? 0 : n_invalid[0]) + bk.n_invalid;
}

}  // namespace

hipError_t launch_gemv_f32_fused(const float* x, const uint8_t* packed, const uint8_t* scales, const int32_t* sel,
                                 const float* p, const float* shared, float* y, int T, int E, int O, int G, int K,
                                 int32_t* n_invalid, int chunk_index, hipStream_t stream) {
  constexpr int R = 4;
  const int nblk = (O + R - 1) / R;
  hipLaunchKernelGGL(gemv_f32_fused_kernel<R>, dim3(nblk), dim3(256), 0, stream, x, packed, scales, sel, p, shared, y,
                     T, E, O, G, K, n_invalid, chunk_index);
  return hipGetLastError();
}

hipError_t launch_gemv_bf16_fused(const uint16_t* x, const uint8_t* packed, const uint8_t* scales, const int32_t* sel,
                                  const float* p, const uint16_t* shared, uint16_t* y, int T, int E, int O, int G, int K,
                                  int32_t* n_invalid, int chunk_index, hipStream_t stream) {
  constexpr int WAVES = 8;
  const int nblk = (O + 15) / 16;
  hipLaunchKernelGGL(gemv_bf16_fused_kernel<WAVES>, dim3(nblk), dim3(WAVES * 64), 0, stream, x, packed, scales, sel, p,
                     shared, y, T, E, O, G, K, n_invalid, chunk_index);
  return hipGetLastError();
}

}  // namespace mxfp4
