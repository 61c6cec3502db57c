// Host-side launchers of the gfx950 kernels (internal to the library).
// Every launcher enqueues on `stream` and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <mutex>

namespace mxfp4 {

// Let KERNEL use `bytes` of dynamic LDS (beyond the default limit): the
// attribute is set once per device, from whichever host thread gets there
// first, and every later call returns that call's status.
constexpr int kMaxDevices = 64;
template <auto* KERNEL>
hipError_t allow_dynamic_lds(int bytes) {
  static std::once_flag once[kMaxDevices];
  static hipError_t status[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(once[dev], [&] {
    status[dev] = hipFuncSetAttribute(reinterpret_cast<const void*>(KERNEL),
                                      hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  });
  return status[dev];
}

// Largest number of pairs (T*K) one fused decode-shaped launch handles
// (one per lane of a wave).
constexpr int kMaxFusedPairs = 64;
// LDS one decode-shaped workgroup may use (activations + partial rows).
constexpr int kDecodeMaxLds = 156 * 1024;

// Grouped-GEMM tile sizes (pairs x output features) and the bucketing chunk.
constexpr int kGemmTileM = 128;
constexpr int kGemmTileN = 128;
constexpr int kBucketChunk = 1024;

// One M-tile of the grouped GEMM: expert e owns sorted positions
// row0 .. row0+mlen-1 of this tile.
struct GemmTile {
  int32_t e;
  int32_t row0;
  int32_t mlen;
  int32_t pad;
};

// Upper bound on the number of M-tiles: sum_e ceil(count_e / MT) <= P/MT + min(E, P).
inline int64_t gemm_max_tiles(int64_t P, int64_t E) {
  return P / kGemmTileM + (E < P ? E : P);
}
// Pairs per bucketing chunk: kBucketChunk, grown (in steps of 64) so that
// there are never more than kMaxBucketChunks chunks.
constexpr int64_t kMaxBucketChunks = 256;
inline int64_t bucket_chunk_size(int64_t P) {
  int64_t c = (P + kMaxBucketChunks - 1) / kMaxBucketChunks;
  c = (c + 63) / 64 * 64;
  return c < kBucketChunk ? kBucketChunk : c;
}
inline int64_t bucket_chunks(int64_t P) { return P <= 0 ? 0 : (P + bucket_chunk_size(P) - 1) / bucket_chunk_size(P); }

// ---- bucketing (count, offsets, perm, slot_of_pair, n_invalid, GEMM tiles)
struct BucketOut {
  int32_t* count;         // [E]
  int32_t* offsets;       // [E+1]
  int32_t* perm;          // [P]
  int32_t* slot_of_pair;  // [P]
  int32_t* n_invalid;     // [1]
  GemmTile* tiles;        // [gemm_max_tiles] or null
  int32_t* n_tiles;       // [1] or null
};
// bcount: [bucket_chunks(P) * E] + [bucket_chunks(P)] int32 scratch
hipError_t launch_bucket_multi(const int32_t* sel, int P, int E, int32_t* bcount, BucketOut out,
                               hipStream_t stream);
hipError_t launch_bucket_one_block(const int32_t* sel, int P, int E, BucketOut out, hipStream_t stream);

// ---- decode-shaped fused path: routing, dequant-GEMV and combine.
// Both decode-shaped kernels need O * G * 16 < 2^31 (gemv_rows_supported).
// dtype 0 = fp32 x/shared/y, 1 = bf16. n_invalid (may be null) receives the
// number of out-of-range indices, accumulated over successive chunk launches
// (chunk_index 0 starts at zero).
hipError_t launch_decode_fused(const void* x, const uint8_t* packed, const uint8_t* scales, const int32_t* sel,
                               const float* p, const void* shared, void* y, int T, int E, int O, int G, int K,
                               int dtype, int32_t* n_invalid, int chunk_index, hipStream_t stream);
// The same MFMA decode kernel on weights in the fragment-major prepared
// layout of launch_prepare_mx (pcodes: its code slots, pscales: its scale
// array); needs gemm_mx_supported's per-expert size bound.
hipError_t launch_decode_prepared(const void* x, const uint8_t* pcodes, const uint8_t* pscales, const int32_t* sel,
                                  const float* p, const void* shared, void* y, int T, int E, int O, int G, int K,
                                  int dtype, int32_t* n_invalid, int chunk_index, hipStream_t stream);
// Most tokens one decode-shaped launch takes for these sizes (0: none fits).
int decode_tokens_per_launch(int K, int E, int G, int dtype);

// Row-contiguous decode-shaped kernel (vector ALUs, buffer loads): same
// contract as launch_decode_fused; needs O * G * 16 < 2^31.
bool gemv_rows_supported(int O, int G);
int gemv_rows_tokens_per_launch(int K, int E, int G, int dtype);
hipError_t launch_gemv_rows(const void* x, const uint8_t* packed, const uint8_t* scales, const int32_t* sel,
                            const float* p, const void* shared, void* y, int T, int E, int O, int G, int K, int dtype,
                            int32_t* n_invalid, int chunk_index, hipStream_t stream);

// One-token decode-shaped kernel (activations in registers): T = 1, any K
// up to kMaxFusedPairs, G <= 256, O * G * 16 < 2^31; n_cu = the device's
// compute units (the grid is sized from it). n_invalid (may be null)
// receives the number of out-of-range indices.
bool gemv_one_supported(int O, int G, int K);
hipError_t launch_gemv_one(const void* x, const uint8_t* packed, const uint8_t* scales, const int32_t* sel,
                           const float* p, const void* shared, void* y, int E, int O, int G, int K, int dtype,
                           int32_t* n_invalid, int n_cu, hipStream_t stream);

// ---- block-scaled variant: MXFP8 activations x MXFP4 weights on the scaled MFMA.
// Activation rows are padded to mx_row_bytes(I) = 128 * ceil(I / 128) codes.
int mx_row_bytes(int64_t I);
bool gemm_mx_supported(int64_t T, int64_t O, int64_t G);  // O % 4 == 0, T * Kp and O * G * 16 below 2^31
hipError_t launch_quant_mxfp8(const uint16_t* x, int T, int I, int Kp, uint8_t* codes, uint8_t* sb,
                              hipStream_t stream);
// MXFP4 activations: codes (T, Kp / 2), two to a byte low nibble first, and
// scale bytes (T, Kp / 32)
hipError_t launch_quant_mxfp4(const uint16_t* x, int T, int I, int Kp, uint8_t* codes, uint8_t* sb,
                              hipStream_t stream);
// prepared = true: `packed` is a buffer written by launch_prepare_mx (its scale
// array follows the packed slots) and `scales` points at that scale array.
// act_fp4: xq holds MXFP4 activation codes (T, Kp / 2) instead of MXFP8 (T, Kp).
hipError_t launch_gemm_mx(const uint8_t* xq, const uint8_t* xs, const uint8_t* packed, const uint8_t* scales,
                          const int32_t* perm, const GemmTile* tiles, const int32_t* n_tiles, int64_t max_tiles,
                          float* part, int T, int K, int O, int G, hipStream_t stream, bool prepared = false,
                          bool act_fp4 = false);
// the prepared weight layout of the block-scaled variant: 16 bytes of codes and
// one scale byte per group slot, slots = E * ceil(O / 128) * (Kp / 128) * 512
size_t mx_prepared_bytes(int64_t E, int64_t O, int64_t G);
// swiglu_F > 0: the SwiGLU row order (O = 2F stacked gate/up rows; prepared
// tile n = gate rows 64 n .. +63, then the up rows of the same features).
// interleaved: the dword-interleaved code blocks the bf16 register-decode
// GEMM reads (else fragment-major, for the block-scaled variant).
hipError_t launch_prepare_mx(const uint8_t* packed, const uint8_t* scales, int64_t E, int O, int G, uint8_t* prepared,
                             hipStream_t stream, int swiglu_F = 0, bool interleaved = false);

// ---- router: logits (T, E) fp32 -> sel (T, K) int32, p (T, K) fp32.
// mode 0 softmax, 1 sigmoid with a selection-only bias (may be null).
// One token per group of `lanes` lanes (32 or 64; 0 = route_lanes' choice).
// Needs 1 <= E <= 1024 and 1 <= K <= min(E, 64); route_lanes returns a group
// width that holds them (K <= lanes, E <= 64 * lanes).
int route_values_per_lane(int E, int lanes);
int route_lanes(int64_t T, int E, int K);
hipError_t launch_route(const float* logits, const float* bias, int T, int E, int K, int mode, float scale,
                        int32_t* sel, float* p, hipStream_t stream, int lanes = 0);
// Group-limited sigmoid router: E <= 1024, n_group | E with E / n_group >= 2
// and n_group <= 64, 1 <= topk_group <= n_group, 1 <= K <= min(64,
// topk_group * E / n_group); renorm: divide by the chosen scores' sum + 1e-20.
hipError_t launch_route_grouped(const float* logits, const float* bias, int T, int E, int K, int n_group,
                               int topk_group, int renorm, float scale, int32_t* sel, float* p, hipStream_t stream);

// ---- prefill-shaped path: grouped GEMM over the tiles, then the combine.
// The grouped GEMM addresses the activations (np bf16 planes of T x 32G) and
// one expert's packed bytes with 32-bit byte offsets: np * T * 32G * 2 < 2^31
// and O * G * 16 < 2^31.
bool gemm_supported(int64_t T, int64_t O, int64_t G, int np = 1);
hipError_t launch_gemm_bf16(const uint16_t* x, const uint8_t* packed, const uint8_t* scales, const int32_t* perm,
                            const GemmTile* tiles, const int32_t* n_tiles, int64_t max_tiles, float* part, int T, int K,
                            int O, int G, hipStream_t stream);
// fp32 activations: launch_split3 writes the exact three-piece bf16 split of
// the n (a multiple of 4) values of x as three planes of n (xs: 3n bf16);
// launch_gemm_f32 is launch_gemm_bf16 on those planes (every weight fragment
// multiplied by all three pieces into one fp32 accumulator).
hipError_t launch_split3(const float* x, int64_t n, uint16_t* xs, hipStream_t stream);
hipError_t launch_gemm_f32(const uint16_t* xs, const uint8_t* packed, const uint8_t* scales, const int32_t* perm,
                           const GemmTile* tiles, const int32_t* n_tiles, int64_t max_tiles, float* part, int T, int K,
                           int O, int G, hipStream_t stream);
// The same on weights in the prepared layout of launch_prepare_mx (pcodes:
// its code slots, pscales: its scale array), decoded in registers (8-wave
// workgroups over 128 pairs x 512 rows); needs gemm_regdec_supported:
// O % 4 == 0 and 32-bit offsets into the activations and one expert's codes.
bool gemm_regdec_supported(int64_t T, int64_t O, int64_t G);
hipError_t launch_gemm_regdec(const uint16_t* x, const uint8_t* pcodes, const uint8_t* pscales, const int32_t* perm,
                              const GemmTile* tiles, const int32_t* n_tiles, int64_t max_tiles, float* part, int T,
                              int K, int O, int G, hipStream_t stream);
// SwiGLU block on prepared weights: gate/up stage (weights prepared in the
// SwiGLU row order, O = 2F; writes bf16 h (P, F)) and down stage (A rows =
// rows of h; writes fp32 part rows).
hipError_t launch_gemm_regdec_swiglu(const uint16_t* x, const uint8_t* pcodes, const uint8_t* pscales,
                                     const int32_t* perm, const GemmTile* tiles, const int32_t* n_tiles,
                                     int64_t max_tiles, uint16_t* h, int T, int K, int F, int G, hipStream_t stream);
hipError_t launch_gemm_regdec_direct(const uint16_t* h, const uint8_t* pcodes, const uint8_t* pscales,
                                     const GemmTile* tiles, const int32_t* n_tiles, int64_t max_tiles, float* part,
                                     int64_t P, int O, int G, hipStream_t stream);
// The register-decode GEMM on canonical weights (packed (E, O, G, 16),
// scales (E, O, G)): the same kernel, its weight DMA fetching each lane's
// 16-byte group straight from the canonical layout and its scale bytes
// loaded per lane; needs gemm_regdec_canon_supported: O % 4 == 0 and 32-bit
// offsets into the activations and one expert's packed bytes. The SwiGLU
// gate/up stage takes (E, 2F, G, 16) with gate rows over up rows, F % 4 == 0.
bool gemm_regdec_canon_supported(int64_t T, int64_t O, int64_t G);
hipError_t launch_gemm_regdec_canon(const uint16_t* x, const uint8_t* packed, const uint8_t* scales,
                                    const int32_t* perm, const GemmTile* tiles, const int32_t* n_tiles,
                                    int64_t max_tiles, float* part, int T, int K, int O, int G, hipStream_t stream);
hipError_t launch_gemm_regdec_canon_swiglu(const uint16_t* x, const uint8_t* gu_packed, const uint8_t* gu_scales,
                                           const int32_t* perm, const GemmTile* tiles, const int32_t* n_tiles,
                                           int64_t max_tiles, uint16_t* h, int T, int K, int F, int G,
                                           hipStream_t stream);
hipError_t launch_gemm_regdec_canon_direct(const uint16_t* h, const uint8_t* packed, const uint8_t* scales,
                                           const GemmTile* tiles, const int32_t* n_tiles, int64_t max_tiles,
                                           float* part, int64_t P, int O, int G, hipStream_t stream);
// SwiGLU expert block, gate/up stage: weights (E, 2F, G, 16) with gate rows
// [0, F) over up rows [F, 2F); writes h[sorted position, f] = bf16 of
// silu(gate) * up, h being (P, F).
hipError_t launch_gemm_swiglu(const uint16_t* x, const uint8_t* gu_packed, const uint8_t* gu_scales,
                              const int32_t* perm, const GemmTile* tiles, const int32_t* n_tiles, int64_t max_tiles,
                              uint16_t* h, int T, int K, int F, int G, hipStream_t stream);
// Down stage: A rows are the rows of h at the sorted positions themselves
// (h is (P, 32G) bf16); writes fp32 part rows like launch_gemm_bf16.
hipError_t launch_gemm_direct(const uint16_t* h, const uint8_t* packed, const uint8_t* scales, const GemmTile* tiles,
                              const int32_t* n_tiles, int64_t max_tiles, float* part, int64_t P, int O, int G,
                              hipStream_t stream);
hipError_t launch_combine(const float* part, const int32_t* slot_of_pair, const float* p,
                          const void* shared, void* y, int T, int K, int O, int dtype,
                          hipStream_t stream);

// ---- plain streaming read of `bytes` (a multiple of 16) from a 16-byte
// aligned buffer; `blocks` workgroups of 256 threads (0: up to 2048); sink
// holds one uint32 per workgroup and is written only by a 2^-32 chance.
hipError_t launch_stream_read(const void* buf, int64_t bytes, int blocks, uint32_t* sink, hipStream_t stream);

// ---- exported decode (test and inspection)
hipError_t launch_decode_rows(const uint8_t* packed_rows, const uint8_t* scales_rows, int64_t nrows,
                              int64_t G, int dtype, void* out, hipStream_t stream);

}  // namespace mxfp4
