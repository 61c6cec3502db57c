// Router upstream of the layer: from router logits to the selected experts
// sel[t, k] and their mixture weights p[t, k] (page "MoE Expert Kernels:
// Grouped Prefill and Mixed-Quant Compact Experts", section 1: a softmax
// router renormalised over the chosen k, floor 6.103515625e-5 on the chosen
// mass, and a sigmoid router whose correction bias steers the selection
// only; the exo pull request page, router bullets: ties go to the lower
// expert index, the selection stays in descending order, the chosen scores
// are summed left to right and divided by sum + 1e-20, times a scale).
//
// A group of L lanes (32 or 64) serves one token; lane j of the group
// holds experts j, j + L, j + 2L, ... (VPL of them, in registers). Each key
// is mapped to an unsigned integer with the same order (NaN as -inf, -0 as
// +0), and the selection takes K rounds of a group-wide arg-max on the 64-bit
// pair (key, ~index), whose maximum is the larger key with, on equal keys,
// the lower index. Within a row of 16 lanes the arg-max is four DPP steps
// (xor 1, xor 2, half-row mirror, row mirror): every lane ends with the
// row's result, with no trip through LDS; one or two cross-row shuffles
// finish the group. Each lane offers its best key not yet taken (it
// keeps its two best and rescans only when both are gone); padding slots
// hold the sentinel 0, below every real key, so the K experts are distinct
// and in [0, E) whatever the logits hold. The softmax router, and the
// sigmoid router without a bias, rank by the logits themselves (they order
// exactly like the exact probabilities or scores); the weights are
// recomputed from the K chosen logits with the same fp32 arithmetic as the
// all-expert pass. All arithmetic is fp32.
#include "device_common.h"
#include "launch.h"

namespace mxfp4 {
namespace {

constexpr float kMassFloor = 6.103515625e-5f;
constexpr float kSigmoidEps = 1e-20f;

// DPP controls (all lanes active, every source inside the row)
constexpr int kXor1 = 0xB1;        // quad_perm [1, 0, 3, 2]
constexpr int kXor2 = 0x4E;        // quad_perm [2, 3, 0, 1]
constexpr int kHalfMirror = 0x141;  // lane i <- lane 7 - i within each half row
constexpr int kMirror = 0x140;      // lane i <- lane 15 - i within the row

template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), CTRL, 0xF, 0xF, false));
}

// 1 / (1 + e^-x) with the hardware reciprocal (1 ulp); 0 at -inf, 1 at +inf
__device__ __forceinline__ float sigmoid(float x) { return __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

// An unsigned integer in the float's order: NaN reads as -inf (IEEE max
// returns the number), -0 as +0 (the addition), and every key is >= 1 (-inf
// maps to 0x007fffff), so 0 is free for the padding sentinel.
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(fmaxf(f, -__builtin_huge_valf()) + 0.0f);
  return u ^ (static_cast<uint32_t>(static_cast<int32_t>(u) >> 31) | 0x80000000u);
}

__device__ __forceinline__ void max_pair(uint32_t& hi, uint32_t& lo, uint32_t ohi, uint32_t olo) {
  const uint64_t a = (static_cast<uint64_t>(hi) << 32) | lo, o = (static_cast<uint64_t>(ohi) << 32) | olo;
  const bool take = o > a;
  hi = take ? ohi : hi;
  lo = take ? olo : lo;
}

// the two largest keys of a lane that are not yet taken, with their slots;
// strict comparisons keep the lower slot (the lower expert) first on ties
template <int VPL>
__device__ __forceinline__ void local_top2(const uint32_t (&key)[VPL], uint32_t taken, uint32_t& h0, uint32_t& i0,
                                           uint32_t& h1, uint32_t& i1) {
  h0 = 0, i0 = 0, h1 = 0, i1 = 0;
#pragma unroll
  for (int v = 0; v < VPL; v++) {
    const uint32_t k = ((taken >> v) & 1) ? 0u : key[v];
    const bool first = k > h0, second = k > h1;
    h1 = first ? h0 : (second ? k : h1);
    i1 = first ? i0 : (second ? static_cast<uint32_t>(v) : i1);
    h0 = first ? k : h0;
    i0 = first ? static_cast<uint32_t>(v) : i0;
  }
}

template <int CTRL>
__device__ __forceinline__ void dpp_max_pair(uint32_t& hi, uint32_t& lo) {
  max_pair(hi, lo, dpp<CTRL>(hi), dpp<CTRL>(lo));
}

// all-reduce over the L lanes of a group (L = 32 or 64, groups aligned)
template <int L>
__device__ __forceinline__ void group_max_pair(uint32_t& hi, uint32_t& lo) {
  dpp_max_pair<kXor1>(hi, lo);
  dpp_max_pair<kXor2>(hi, lo);
  dpp_max_pair<kHalfMirror>(hi, lo);
  dpp_max_pair<kMirror>(hi, lo);
  if constexpr (L >= 32) max_pair(hi, lo, __shfl_xor(hi, 16, 64), __shfl_xor(lo, 16, 64));
  if constexpr (L >= 64) max_pair(hi, lo, __shfl_xor(hi, 32, 64), __shfl_xor(lo, 32, 64));
}

template <int L>
__device__ __forceinline__ float group_max(float v) {
  v = fmaxf(v, __uint_as_float(dpp<kXor1>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp<kXor2>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp<kHalfMirror>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp<kMirror>(__float_as_uint(v))));
  if constexpr (L >= 32) v = fmaxf(v, __shfl_xor(v, 16, 64));
  if constexpr (L >= 64) v = fmaxf(v, __shfl_xor(v, 32, 64));
  return v;
}

template <int L>
__device__ __forceinline__ float group_sum(float v) {
  v += __uint_as_float(dpp<kXor1>(__float_as_uint(v)));
  v += __uint_as_float(dpp<kXor2>(__float_as_uint(v)));
  v += __uint_as_float(dpp<kHalfMirror>(__float_as_uint(v)));
  v += __uint_as_float(dpp<kMirror>(__float_as_uint(v)));
  if constexpr (L >= 32) v += __shfl_xor(v, 16, 64);
  if constexpr (L >= 64) v += __shfl_xor(v, 32, 64);
  return v;
}

template <int L, int VPL>
__global__ void __launch_bounds__(256) route_kernel(const float* __restrict__ logits, const float* __restrict__ bias,
                                                    int T, int E, int K, int mode, float scale,
                                                    int32_t* __restrict__ sel, float* __restrict__ p) {
  constexpr int kGroups = 64 / L;  // tokens per wave
  const int lane = threadIdx.x & 63;
  const int j = lane & (L - 1);
  const int wave_t0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * kGroups;
  if (wave_t0 >= T) return;  // wave-uniform; a partly filled wave keeps every lane for the DPP steps
  const int t = wave_t0 + lane / L;
  const bool live = t < T;
  const float* row = logits + (int64_t)(live ? t : wave_t0) * E;
  constexpr float kNegInf = -__builtin_huge_valf();

  // every load in bounds (clamped to the row's last expert), then masked; a
  // group past the batch reads the wave's first row and stores nothing
  float lg[VPL];
#pragma unroll
  for (int v = 0; v < VPL; v++) {
    const int e = j + L * v;
    const float x = row[e < E ? e : E - 1];
    lg[v] = e < E ? x : kNegInf;
  }
  uint32_t key[VPL];
  float m = 0.f, z = 1.f;
  if (mode == 0) {
    m = kNegInf;
#pragma unroll
    for (int v = 0; v < VPL; v++) m = fmaxf(m, lg[v]);
    m = group_max<L>(m);
    float s = 0.f;
#pragma unroll
    for (int v = 0; v < VPL; v++) s += (j + L * v < E) ? __expf(lg[v] - m) : 0.f;
    z = group_sum<L>(s);
#pragma unroll
    for (int v = 0; v < VPL; v++) key[v] = (j + L * v < E) ? order_key(lg[v]) : 0u;
  } else if (bias) {  // uniform
    float b[VPL];
#pragma unroll
    for (int v = 0; v < VPL; v++) b[v] = bias[j + L * v < E ? j + L * v : E - 1];
#pragma unroll
    for (int v = 0; v < VPL; v++) {
      const uint32_t kk = order_key(sigmoid(lg[v]) + b[v]);
      key[v] = (j + L * v < E) ? kk : 0u;
    }
  } else {
    // no bias: the sigmoid is increasing, so the logits rank like the exact scores
#pragma unroll
    for (int v = 0; v < VPL; v++) key[v] = (j + L * v < E) ? order_key(lg[v]) : 0u;
  }

  // Each lane keeps its two best untaken keys; a round compares the heads
  // across the group, the owner of the winner pops its head and, once both
  // are gone, rescans its keys past the taken ones.
  uint32_t taken = 0;  // bit v: slot v already chosen (VPL <= 32)
  uint32_t h0, i0, h1, i1;
  local_top2<VPL>(key, taken, h0, i0, h1, i1);
  int my_sel = 0;
  for (int k = 0; k < K; k++) {
    uint32_t hi = h0, lo = ~static_cast<uint32_t>(j + L * i0);
    group_max_pair<L>(hi, lo);
    const uint32_t win = ~lo;
    const bool own = (win & (L - 1)) == static_cast<uint32_t>(j);
    if (j == k) my_sel = static_cast<int>(win);
    taken |= own ? (1u << i0) : 0u;
    h0 = own ? h1 : h0;
    i0 = own ? i1 : i0;
    h1 = own ? 0u : h1;
    if (own && h0 == 0) local_top2<VPL>(key, taken, h0, i0, h1, i1);
  }

  // the weights, from the chosen logits with the arithmetic of the pass above
  float sc = 0.f;
  if (j < K) {
    const float l = row[my_sel];
    sc = mode == 0 ? __expf(l - m) / z : sigmoid(l);
  }
  float mass = 0.f;
  const int base = lane & ~(L - 1);
  for (int k = 0; k < K; k++) mass += __shfl(sc, base + k, 64);  // left to right
  if (live && j < K) {
    const float den = mode == 0 ? fmaxf(mass, kMassFloor) : mass + kSigmoidEps;
    sel[(int64_t)t * K + j] = my_sel;
    p[(int64_t)t * K + j] = sc / den * scale;
  }
}

// Group-limited sigmoid router (the CPU kernels page, section 1, its first
// router): choice score c_e = sigmoid(logit_e) + bias_e (NaN read as -inf);
// groups of eg = E / n_group consecutive experts, scored by the sum of
// their two largest choice scores; the topk_group best groups are kept
// (ties to the lower group); the K best choice scores inside them are
// chosen (ties to the lower expert); the weights are the unbiased sigmoid
// scores of the chosen, divided by their left-to-right sum + 1e-20 when
// renorm is set, times scale. One wave per token: lane j holds experts
// j, j + 64, ...; the choice scores also go to LDS, where lane g < n_group
// scans group g for its two best; the groups are then chosen by
// topk_group rounds of the wave-wide arg-max, and the experts of the
// dropped groups get the sentinel key 0 before the K rounds.
constexpr int kGroupedWaves = 4;

template <int VPL>
__global__ void __launch_bounds__(64 * kGroupedWaves) route_grouped_kernel(
    const float* __restrict__ logits, const float* __restrict__ bias, int T, int E, int K, int n_group,
    int topk_group, int renorm, float scale, int32_t* __restrict__ sel, float* __restrict__ p) {
  __shared__ float cs[kGroupedWaves][64 * VPL];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int t0 = blockIdx.x * kGroupedWaves + w;
  const bool live = t0 < T;
  const int t = live ? t0 : T - 1;  // a wave past the batch repeats the last token and stores nothing
  const float* row = logits + (int64_t)t * E;
  const int eg = E / n_group;
  constexpr float kNegInf = -__builtin_huge_valf();
  uint32_t key[VPL];
#pragma unroll
  for (int v = 0; v < VPL; v++) {
    const int e = lane + 64 * v;
    const int ec = e < E ? e : E - 1;
    const float b = bias ? bias[ec] : 0.f;
    const float c = fmaxf(sigmoid(row[ec]) + b, kNegInf);  // NaN -> -inf
    if (e < E) cs[w][e] = c;
    key[v] = e < E ? order_key(c) : 0u;
  }
  __syncthreads();
  // group scores: lane g scans its group for the two largest choice scores
  uint32_t gk = 0;
  if (lane < n_group) {
    float a = kNegInf, b = kNegInf;
    for (int i = 0; i < eg; i++) {
      const float c = cs[w][lane * eg + i];
      const bool first = c > a, second = c > b;
      b = first ? a : (second ? c : b);
      a = first ? c : a;
    }
    gk = order_key(a + b);
  }
  uint64_t kept = 0;
  for (int r = 0; r < topk_group; r++) {
    uint32_t hi = gk, lo = ~static_cast<uint32_t>(lane);
    group_max_pair<64>(hi, lo);
    const uint32_t g = ~lo;
    kept |= uint64_t(1) << g;
    gk = (static_cast<uint32_t>(lane) == g) ? 0u : gk;
  }
#pragma unroll
  for (int v = 0; v < VPL; v++) {
    const int e = lane + 64 * v;
    const bool in = e < E && ((kept >> (e / eg)) & 1);
    key[v] = in ? key[v] : 0u;
  }
  uint32_t taken = 0;
  uint32_t h0, i0, h1, i1;
  local_top2<VPL>(key, taken, h0, i0, h1, i1);
  int my_sel = 0;
  for (int k = 0; k < K; k++) {
    uint32_t hi = h0, lo = ~static_cast<uint32_t>(lane + 64 * i0);
    group_max_pair<64>(hi, lo);
    const uint32_t win = ~lo;
    const bool own = (win & 63u) == static_cast<uint32_t>(lane);
    if (lane == k) my_sel = static_cast<int>(win);
    taken |= own ? (1u << i0) : 0u;
    h0 = own ? h1 : h0;
    i0 = own ? i1 : i0;
    h1 = own ? 0u : h1;
    if (own && h0 == 0) local_top2<VPL>(key, taken, h0, i0, h1, i1);
  }
  const float sc = lane < K ? sigmoid(row[my_sel]) : 0.f;
  float mass = 0.f;
  for (int k = 0; k < K; k++) mass += __shfl(sc, k, 64);  // left to right
  if (live && lane < K) {
    sel[(int64_t)t * K + lane] = my_sel;
    p[(int64_t)t * K + lane] = (renorm ? sc / (mass + kSigmoidEps) : sc) * scale;
  }
}

constexpr int kVplChoices[] = {1, 2, 4, 8, 12, 16, 24, 32};  // E <= 1024 at 32 lanes

template <int L, int VPL>
void launch_one(const float* logits, const float* bias, int T, int E, int K, int mode, float scale, int32_t* sel,
                float* p, hipStream_t stream) {
  constexpr int kTokensPerBlock = 4 * (64 / L);
  const dim3 grid((T + kTokensPerBlock - 1) / kTokensPerBlock), block(256);
  hipLaunchKernelGGL((route_kernel<L, VPL>), grid, block, 0, stream, logits, bias, T, E, K, mode, scale, sel, p);
}

template <int L>
hipError_t launch_lanes(int vpl, const float* logits, const float* bias, int T, int E, int K, int mode, float scale,
                        int32_t* sel, float* p, hipStream_t stream) {
  switch (vpl) {
    case 1: launch_one<L, 1>(logits, bias, T, E, K, mode, scale, sel, p, stream); break;
    case 2: launch_one<L, 2>(logits, bias, T, E, K, mode, scale, sel, p, stream); break;
    case 4: launch_one<L, 4>(logits, bias, T, E, K, mode, scale, sel, p, stream); break;
    case 8: launch_one<L, 8>(logits, bias, T, E, K, mode, scale, sel, p, stream); break;
    case 12: launch_one<L, 12>(logits, bias, T, E, K, mode, scale, sel, p, stream); break;
    case 16: launch_one<L, 16>(logits, bias, T, E, K, mode, scale, sel, p, stream); break;
    case 24: launch_one<L, 24>(logits, bias, T, E, K, mode, scale, sel, p, stream); break;
    case 32: launch_one<L, 32>(logits, bias, T, E, K, mode, scale, sel, p, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

int route_values_per_lane(int E, int lanes) {
  if (lanes != 32 && lanes != 64) return 0;
  const int need = (E + lanes - 1) / lanes;
  for (int v : kVplChoices)
    if (v >= need) return v;
  return 0;
}

int route_lanes(int64_t T, int E, int K) {
  // 32 lanes a token from 512 tokens up (measured: at 4096 x 128 and
  // 8192 x 384 it beats both 16 lanes, whose longer per-lane scans run at
  // two waves a SIMD, and 64, whose extra cross-row step costs every round);
  // 64 for smaller batches, whose few waves want the shortest chain, and
  // whenever K > 32
  const int lanes = (T >= 512 && K <= 32) ? 32 : 64;
  return route_values_per_lane(E, lanes) ? lanes : 0;
}

hipError_t launch_route_grouped(const float* logits, const float* bias, int T, int E, int K, int n_group,
                               int topk_group, int renorm, float scale, int32_t* sel, float* p, hipStream_t stream) {
  const int vpl = (E + 63) / 64;
  if (E < 2 || E > 1024 || n_group < 1 || n_group > 64 || E % n_group || E / n_group < 2 || topk_group < 1 ||
      topk_group > n_group || K < 1 || K > 64 || K > topk_group * (E / n_group))
    return hipErrorInvalidValue;
  if (T == 0) return hipSuccess;
  const dim3 grid((T + kGroupedWaves - 1) / kGroupedWaves), block(64 * kGroupedWaves);
#define MXFP4_ROUTE_GROUPED_CASE(V)                                                                             \
  case V:                                                                                                      \
    hipLaunchKernelGGL((route_grouped_kernel<V>), grid, block, 0, stream, logits, bias, T, E, K, n_group,     \
                       topk_group, renorm, scale, sel, p);                                                     \
    break;
  switch (vpl <= 2 ? vpl : (vpl <= 4 ? 4 : (vpl <= 8 ? 8 : 16))) {
    MXFP4_ROUTE_GROUPED_CASE(1)
    MXFP4_ROUTE_GROUPED_CASE(2)
    MXFP4_ROUTE_GROUPED_CASE(4)
    MXFP4_ROUTE_GROUPED_CASE(8)
    MXFP4_ROUTE_GROUPED_CASE(16)
    default: return hipErrorInvalidValue;
  }
#undef MXFP4_ROUTE_GROUPED_CASE
  return hipGetLastError();
}

hipError_t launch_route(const float* logits, const float* bias, int T, int E, int K, int mode, float scale,
                        int32_t* sel, float* p, hipStream_t stream, int lanes) {
  if (lanes == 0) lanes = route_lanes(T, E, K);
  const int vpl = route_values_per_lane(E, lanes);
  if (vpl == 0 || K < 1 || K > lanes || K > E) return hipErrorInvalidValue;
  if (T == 0) return hipSuccess;
  return lanes == 32 ? launch_lanes<32>(vpl, logits, bias, T, E, K, mode, scale, sel, p, stream)
                     : launch_lanes<64>(vpl, logits, bias, T, E, K, mode, scale, sel, p, stream);
}

}  // namespace mxfp4
