// Wave-local routing of up to 64 (token, choice) pairs: lane i holds pair
// i's expert; ballots over the expert index bits group the pairs by expert
// without LDS, atomics or barriers. The distinct experts are numbered in
// the order of their first pair, so the grouping (and everything computed
// from it) is deterministic.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxfp4 {

__device__ __forceinline__ uint64_t lanes_below(int lane) { return (lane == 0) ? 0ull : (~0ull >> (64 - lane)); }

// Position of the n-th set bit of m (m has more than n set bits), by a
// branch-free binary search on popcounts.
__device__ __forceinline__ int nth_set_bit(uint64_t m, int n) {
  int pos = 0;
#pragma unroll
  for (int width = 32; width >= 1; width >>= 1) {
    const uint64_t low = m & ((width == 64 ? 0ull : (1ull << width)) - 1ull);
    const int c = __popcll(low);
    const bool up = n >= c;
    n -= up ? c : 0;
    pos += up ? width : 0;
    m = up ? (m >> width) : low;
  }
  return pos;
}

__device__ __forceinline__ uint64_t readlane64(uint64_t v, int src) {
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, src);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(v >> 32), src);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t shfl64(uint64_t v, int src) {
  const uint32_t lo = __shfl((uint32_t)v, src, 64);
  const uint32_t hi = __shfl((uint32_t)(v >> 32), src, 64);
  return ((uint64_t)hi << 32) | lo;
}

struct WaveRoute {
  uint64_t valid;  // pairs whose expert index lies in [0, E)
  int U;           // distinct experts among them
  uint64_t pm_u;   // lane u < U: mask of the pairs that chose expert u
  int e_u;         // lane u < U: expert u
};

// e_l: lane's expert index (any value for lane >= P); nbits = ceil(log2 E).
__device__ __forceinline__ WaveRoute route_wave(int e_l, int lane, int P, int E, int nbits) {
  const bool ok = lane < P && e_l >= 0 && e_l < E;
  uint64_t peers = __ballot(ok);  // pairs with the same expert as this lane
  for (int b = 0; b < nbits; b++) {
    const bool bit = (e_l >> b) & 1;
    const uint64_t ones = __ballot(ok && bit);
    peers &= bit ? ones : ~ones;
  }
  WaveRoute rt;
  const uint64_t firsts = __ballot(ok && (peers & lanes_below(lane)) == 0);
  rt.valid = __ballot(ok);
  rt.U = __popcll(firsts);
  const int src_u = lane < rt.U ? nth_set_bit(firsts, lane) : 0;
  rt.pm_u = shfl64(peers, src_u);
  rt.e_u = __shfl(e_l, src_u, 64);
  return rt;
}

}  // namespace mxfp4
