// Token-to-expert bucketing: a stable counting sort of the P = T*K
// (token, slot) pairs by expert index (page "MoE Expert Kernels: Grouped
// Prefill and Mixed-Quant Compact Experts", section 2: histogram, then
// scatter; expert e owns the contiguous positions [off_e, off_e + cnt_e),
// filled in pair order). All arithmetic is on integers, so the result is the
// same whatever the schedule.
//
// Multi-block algorithm (large P):
//   1. hist:    each chunk of pairs counts its experts in LDS -> bcount[c][e]
//   2. scan:    one workgroup sums the chunk counts, scans over experts,
//               turns bcount into per-chunk base positions, and writes the
//               grouped-GEMM M-tile list
//   3. scatter: one wave per chunk walks its pairs 64 at a time; a lane's
//               rank among equal experts comes from ballots (no atomics),
//               so positions follow pair order exactly.
// One-block algorithm (small P): the same three steps in one workgroup.
#include "device_common.h"
#include "launch.h"

namespace mxfp4 {
namespace {

constexpr int kScanThreads = 1024;

__device__ __forceinline__ uint64_t lanes_below(int lane) { return (lane == 0) ? 0ull : (~0ull >> (64 - lane)); }

// Exclusive prefix sum of a[0..n) in place (LDS), by all NT threads of the
// block; returns the total to every thread.
template <int NT>
__device__ int block_exclusive_scan(int* a, int n, int* wave_tot /* LDS, NT/64 + 1 */) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int per = (n + NT - 1) / NT;
  const int begin = min(n, tid * per), end = min(n, begin + per);
  int local = 0;
  for (int i = begin; i < end; i++) local += a[i];
  int incl = local;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int v = __shfl_up(incl, d, 64);
    if (lane >= d) incl += v;
  }
  if (lane == 63) wave_tot[w] = incl;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int i = 0; i < NT / 64; i++) {
      int v = wave_tot[i];
      wave_tot[i] = run;
      run += v;
    }
    wave_tot[NT / 64] = run;
  }
  __syncthreads();
  int run = incl - local + wave_tot[w];
  for (int i = begin; i < end; i++) {
    int v = a[i];
    a[i] = run;
    run += v;
  }
  int total = wave_tot[NT / 64];
  __syncthreads();
  return total;
}

// Rank of this lane's key among the active lanes of its wave that hold the
// same key and a lower lane id; `peers` gets the mask of all lanes holding
// the key. Inactive lanes (ok = false) take part in the ballots only.
__device__ __forceinline__ void match_rank(bool ok, int key, int nbits, uint64_t& peers, int& rank) {
  const int lane = threadIdx.x & 63;
  uint64_t m = __ballot(ok);
  for (int b = 0; b < nbits; b++) {
    const bool bit = (key >> b) & 1;
    const uint64_t ones = __ballot(ok && bit);
    m &= bit ? ones : ~ones;
  }
  peers = m;
  rank = __popcll(m & lanes_below(lane));
}

__host__ __device__ inline int bits_for(int E) {
  int nb = 0;
  while ((1 << nb) < E) nb++;
  return nb;
}

// Writes the M-tile list of the grouped GEMM from count/offsets (LDS copy
// of count in `count_lds`; `tmp` is clobbered). The work is ordered longest
// first by expert: experts with more pairs come first (equal counts: the
// lower index first), each expert's tiles stay together - its full tiles of
// kGemmTileM pairs, then its partial tile - so that the partial tile runs
// right after the full ones and finds the expert's weights in L2. (The order
// is a permutation of experts by rank = number of experts with more pairs,
// or as many and a lower index; up to kSortMaxE experts, beyond that the
// experts keep their index order.) Each tile's height is its expert's pairs
// left (at most kGemmTileM); the kernels skip the 32-row MFMA sub-tiles past it.
constexpr int kSortMaxE = 1024;

template <int NT>
__device__ void write_tiles(const int* count_lds, int* tmp, int E, const int32_t* offsets, GemmTile* tiles,
                            int32_t* n_tiles, int* wave_tot) {
  __shared__ int order[kSortMaxE];  // position -> expert
  const bool ranked = E <= kSortMaxE;
  if (ranked) {
    for (int e = threadIdx.x; e < E; e += NT) {
      const int c = count_lds[e];
      int r = 0;
      // every lane reads the same counts (an LDS broadcast), eight at a time
      int f = 0;
      for (; f + 8 <= E; f += 8) {
        int cf[8];
#pragma unroll
        for (int i = 0; i < 8; i++) cf[i] = count_lds[f + i];
#pragma unroll
        for (int i = 0; i < 8; i++) r += (cf[i] > c) || (cf[i] == c && f + i < e);
      }
      for (; f < E; f++) {
        const int cf = count_lds[f];
        r += (cf > c) || (cf == c && f < e);
      }
      order[r] = e;
    }
    __syncthreads();
  }
  for (int i = threadIdx.x; i < E; i += NT) tmp[i] = (count_lds[ranked ? order[i] : i] + kGemmTileM - 1) / kGemmTileM;
  __syncthreads();
  const int total = block_exclusive_scan<NT>(tmp, E, wave_tot);
  for (int i = threadIdx.x; i < E; i += NT) {
    const int e = ranked ? order[i] : i;
    const int c = count_lds[e], base = offsets[e];
    for (int j = 0, t = tmp[i]; j * kGemmTileM < c; j++, t++) {
      GemmTile tl;
      tl.e = e;
      tl.row0 = base + j * kGemmTileM;
      tl.mlen = min(kGemmTileM, c - j * kGemmTileM);
      tl.pad = 0;
      tiles[t] = tl;
    }
  }
  if (threadIdx.x == 0) n_tiles[0] = total;
}

__global__ void __launch_bounds__(256) bucket_hist_kernel(const int32_t* __restrict__ sel, int P, int E, int chunk,
                                                          int32_t* __restrict__ bcount, int nchunks) {
  extern __shared__ int hist[];
  __shared__ int invalid;
  const int c = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
  if (threadIdx.x == 0) invalid = 0;
  __syncthreads();
  const int begin = c * chunk, end = min(P, begin + chunk);
  for (int i = begin + threadIdx.x; i < end; i += blockDim.x) {
    const int e = sel[i];
    if (e >= 0 && e < E) atomicAdd(&hist[e], 1);  // integer counts: order-free
    else atomicAdd(&invalid, 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) bcount[(size_t)c * E + e] = hist[e];
  if (threadIdx.x == 0) bcount[(size_t)nchunks * E + c] = invalid;
}

__global__ void __launch_bounds__(kScanThreads) bucket_scan_kernel(int32_t* __restrict__ bcount, int nchunks, int E,
                                                                   BucketOut out) {
  extern __shared__ int sh[];
  int* cnt = sh;              // [E]
  int* tmp = sh + E;          // [E]
  int* wave_tot = sh + 2 * E; // [17]
  __shared__ int inv_red[kScanThreads / 64];
  // the chunk loops are unrolled so that many of their (independent) loads are in flight at once
  for (int e = threadIdx.x; e < E; e += kScanThreads) {
    int total = 0;
#pragma unroll 16
    for (int c = 0; c < nchunks; c++) total += bcount[(size_t)c * E + e];
    cnt[e] = total;
    tmp[e] = total;
    out.count[e] = total;
  }
  int inv = 0;
  for (int c = threadIdx.x; c < nchunks; c += kScanThreads) inv += bcount[(size_t)nchunks * E + c];
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) inv += __shfl_xor(inv, m, 64);
  if ((threadIdx.x & 63) == 0) inv_red[threadIdx.x >> 6] = inv;
  __syncthreads();
  const int total = block_exclusive_scan<kScanThreads>(tmp, E, wave_tot);
  for (int e = threadIdx.x; e < E; e += kScanThreads) {
    out.offsets[e] = tmp[e];
    int run = tmp[e];
#pragma unroll 16
    for (int c = 0; c < nchunks; c++) {  // chunk c's first position for expert e
      const int v = bcount[(size_t)c * E + e];
      bcount[(size_t)c * E + e] = run;
      run += v;
    }
  }
  if (threadIdx.x == 0) {
    out.offsets[E] = total;
    int s = 0;
    for (int i = 0; i < kScanThreads / 64; i++) s += inv_red[i];
    out.n_invalid[0] = s;
  }
  __syncthreads();
  if (out.tiles) write_tiles<kScanThreads>(cnt, tmp, E, out.offsets, out.tiles, out.n_tiles, wave_tot);
}

// One wave per chunk. The expert indices of kScatterBatch steps of 64 pairs
// are loaded before the first of them is ranked, and a step waits only for
// its LDS reads of the cursors (the stores of earlier steps stay in flight).
constexpr int kScatterBatch = 16;
__global__ void __launch_bounds__(64) bucket_scatter_kernel(const int32_t* __restrict__ sel, int P, int E, int chunk,
                                                            const int32_t* __restrict__ bases, int nbits,
                                                            int32_t* __restrict__ perm, int32_t* __restrict__ slot_of_pair) {
  extern __shared__ int cursor[];
  const int c = blockIdx.x, lane = threadIdx.x;
  for (int e = lane; e < E; e += 64) cursor[e] = bases[(size_t)c * E + e];
  __syncthreads();
  const int begin = c * chunk, end = min(P, begin + chunk);
  for (int i0 = begin; i0 < end; i0 += 64 * kScatterBatch) {
    int ev[kScatterBatch];
#pragma unroll
    for (int b = 0; b < kScatterBatch; b++) {
      const int i = i0 + 64 * b + lane;
      ev[b] = i < end ? sel[i] : -1;
    }
#pragma unroll
    for (int b = 0; b < kScatterBatch; b++) {
      if (i0 + 64 * b >= end) break;  // wave-uniform
      const int i = i0 + 64 * b + lane;
      const bool in = i < end;
      const int e = ev[b];
      const bool ok = in && e >= 0 && e < E;
      uint64_t peers;
      int rank;
      match_rank(ok, ok ? e : 0, nbits, peers, rank);
      int slot = -1;
      if (ok) slot = cursor[e] + rank;
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): all reads of cursor precede the updates below
      __builtin_amdgcn_wave_barrier();
      if (ok && rank == 0) cursor[e] += __popcll(peers);
      __builtin_amdgcn_wave_barrier();
      if (ok) perm[slot] = i;
      if (in) slot_of_pair[i] = slot;
    }
  }
}

__global__ void __launch_bounds__(kScanThreads) bucket_one_block_kernel(const int32_t* __restrict__ sel, int P, int E,
                                                                        int nbits, BucketOut out) {
  extern __shared__ int sh[];
  int* cnt = sh;              // [E]
  int* tmp = sh + E;          // [E]
  int* wave_tot = sh + 2 * E; // [17]
  __shared__ int invalid;
  for (int e = threadIdx.x; e < E; e += kScanThreads) cnt[e] = 0;
  if (threadIdx.x == 0) invalid = 0;
  __syncthreads();
  for (int i = threadIdx.x; i < P; i += kScanThreads) {
    const int e = sel[i];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
    else atomicAdd(&invalid, 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kScanThreads) {
    tmp[e] = cnt[e];
    out.count[e] = cnt[e];
  }
  __syncthreads();
  const int total = block_exclusive_scan<kScanThreads>(tmp, E, wave_tot);
  for (int e = threadIdx.x; e < E; e += kScanThreads) out.offsets[e] = tmp[e];
  if (threadIdx.x == 0) {
    out.offsets[E] = total;
    out.n_invalid[0] = invalid;
  }
  __syncthreads();
  // scatter by wave 0 in pair order; tmp[] is the running cursor
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    for (int i0 = 0; i0 < P; i0 += 64) {
      const int i = i0 + lane;
      const bool in = i < P;
      const int e = in ? sel[i] : -1;
      const bool ok = in && e >= 0 && e < E;
      uint64_t peers;
      int rank;
      match_rank(ok, ok ? e : 0, nbits, peers, rank);
      int slot = -1;
      if (ok) slot = tmp[e] + rank;
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): all reads of the cursors precede the updates below
      __builtin_amdgcn_wave_barrier();
      if (ok && rank == 0) tmp[e] += __popcll(peers);
      __builtin_amdgcn_wave_barrier();
      if (ok) out.perm[slot] = i;
      if (in) out.slot_of_pair[i] = slot;
    }
  }
  __syncthreads();
  if (out.tiles) {
    write_tiles<kScanThreads>(cnt, tmp, E, out.offsets, out.tiles, out.n_tiles, wave_tot);
  }
}

}  // namespace

hipError_t launch_bucket_multi(const int32_t* sel, int P, int E, int32_t* bcount, BucketOut out, hipStream_t stream) {
  const int nchunks = (int)bucket_chunks(P);
  const int chunk = (int)bucket_chunk_size(P);
  const int nbits = bits_for(E);
  hipLaunchKernelGGL(bucket_hist_kernel, dim3(nchunks), dim3(256), E * sizeof(int), stream, sel, P, E, chunk,
                     bcount, nchunks);
  hipLaunchKernelGGL(bucket_scan_kernel, dim3(1), dim3(kScanThreads), (2 * E + 32) * sizeof(int), stream, bcount,
                     nchunks, E, out);
  hipLaunchKernelGGL(bucket_scatter_kernel, dim3(nchunks), dim3(64), E * sizeof(int), stream, sel, P, E, chunk,
                     bcount, nbits, out.perm, out.slot_of_pair);
  return hipGetLastError();
}

hipError_t launch_bucket_one_block(const int32_t* sel, int P, int E, BucketOut out, hipStream_t stream) {
  const int nbits = bits_for(E);
  hipLaunchKernelGGL(bucket_one_block_kernel, dim3(1), dim3(kScanThreads), (2 * E + 32) * sizeof(int), stream, sel, P,
                     E, nbits, out);
  return hipGetLastError();
}

}  // namespace mxfp4
