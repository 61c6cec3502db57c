/*
 * mxfp4_moe.h - C ABI of the MXFP4 routed-expert linear on AMD MI355X (gfx950).
 *
 * The operation (page "MXFP4 Routed Expert Linear", Kimi K3, section
 * "Route, weight, and add the shared path"; page "MXFP4 Experts", shape
 * paragraph):
 *
 *     y[t, :] = shared[t, :] + sum_{k < K} p[t, k] * W_{sel[t, k]} x[t, :]
 *
 * W_e is O x I with I = 32 G. It is stored as packed bytes [E, O, G, 16]
 * (two E2M1 codes per byte, low nibble first) and E8M0 scale bytes [E, O, G]
 * (the packed shape without its last axis, page "MXFP4 Dequant", "How it
 * works"). Code n of byte b is n_lo = b & 15 then n_hi = b >> 4; it maps
 * through the E2M1 table {0, .5, 1, 1.5, 2, 3, 4, 6, -0, -.5, -1, -1.5, -2,
 * -3, -4, -6} and is multiplied by 2^(s - 127) for its group's scale byte s
 * (page "MXFP4 Routed Expert Linear", "What is stored in one group" and
 * "Apply the shared group scale"). Group g fills input columns 32g..32g+31
 * of its row ("Reconstruct the matrix in the right orientation").
 *
 * Only the experts that appear in sel are read ("Decode only selected
 * experts"); no decoded weight matrix is ever written to device memory.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers.   Every tensor pointer is a device pointer owned by the caller.
 *             The library never frees, retains or writes an input.
 * Layout.     Dense row-major:
 *               x       [T, 32G]  fp32 or bf16 (bf16 = raw 16-bit patterns)
 *               packed  [E, O, G, 16] uint8
 *               scales  [E, O, G]     uint8
 *               sel     [T, K]    int32 expert indices
 *               p       [T, K]    fp32 mixture weights (used as given; never
 *                                 renormalised)
 *               shared  [T, O]    same dtype as x
 *               y       [T, O]    same dtype as x, fully overwritten
 * Alignment.  packed and x must be 16-byte aligned; scales, sel, p, shared
 *             and y need only the natural alignment of their element type.
 * Aliasing.   y may be exactly shared (each element is read and then written
 *             by the same thread); any other overlap of y with an input is
 *             rejected with MXFP4_ERR_INVALID_ARG.
 * Selection.  A token may list an expert more than once; every listed slot
 *             contributes (list semantics). An index outside [0, E) breaks
 *             a stated precondition: that slot contributes nothing, and it is
 *             reported only when MXFP4_FLAG_CHECK is set.
 * Rounding.   Products are accumulated in fp32; y is shared + (the k-ordered
 *             fp32 sum of p * partial), rounded once to y's dtype (round to
 *             nearest even). Results are bitwise deterministic run to run.
 * Streams.    Work is enqueued on `stream` (0 = the null stream) of the
 *             current HIP device; every call returns without waiting for the
 *             GPU unless MXFP4_FLAG_CHECK is set.
 * Errors.     Every call returns an mxfp4_status. Argument checks happen on
 *             the host before anything is enqueued and need no GPU. T = 0 is
 *             valid and enqueues nothing. A device that is not gfx950 gets
 *             MXFP4_ERR_UNSUPPORTED_DEVICE: there is no fallback path.
 * Threads.    All entry points are reentrant; the only shared state is a
 *             per-device cache of the architecture check and, per kernel and
 *             device, the one-time opt-in to large dynamic LDS (taken once,
 *             under std::call_once).
 * Large scale bytes. Every path returns the layer's value up to fp32
 *             rounding for every scale byte 0..255 (2^(s-127)), also where a
 *             decoded weight E2M1 * 2^(s-127) itself would overflow fp32 or
 *             bf16 (s >= 253): the decode-shaped kernels scale each group's
 *             dot product by 2^(s-127) after it is taken, the grouped GEMMs
 *             decode a tile that holds such a byte at 2^(s-130) and scale the
 *             tile's sums by 2^3 (the block-scaled MXFP8 variant excepted:
 *             see its entry point). A value whose magnitude exceeds the output
 *             type's range is +-inf there, as a rounding of the exact value.
 */
#ifndef MXFP4_MOE_H
#define MXFP4_MOE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mxfp4_status {
  MXFP4_OK = 0,
  MXFP4_ERR_INVALID_ARG = -1,        /* null pointer, bad size, misalignment, overlap */
  MXFP4_ERR_UNSUPPORTED_DEVICE = -2, /* the current device is not gfx950 */
  MXFP4_ERR_HIP = -3,                /* a HIP runtime call or a launch failed */
  MXFP4_ERR_WORKSPACE_TOO_SMALL = -4,
  MXFP4_ERR_INVALID_INDEX = -5,      /* with MXFP4_FLAG_CHECK: some sel entry outside [0, E) */
  MXFP4_ERR_UNSUPPORTED = -6         /* a forced path that does not exist for these sizes:
                                        the decode-shaped path needs one expert's packed bytes
                                        O*G*16 < 2^31 and one token's rows in LDS; the
                                        prefill-shaped path needs O*G*16 < 2^31 and
                                        T*32G*2 (bf16) or 3*T*32G*2 (fp32) below 2^31 */
} mxfp4_status;

typedef enum mxfp4_dtype {
  MXFP4_DTYPE_F32 = 0,
  MXFP4_DTYPE_BF16 = 1
} mxfp4_dtype;

/* Flags of the _ex entry points. */
#define MXFP4_FLAG_FORCE_GEMV 0x1u /* decode-shaped path (dequant-GEMV, fused combine) */
#define MXFP4_FLAG_FORCE_GEMM 0x2u /* prefill-shaped path (bucketing, MFMA grouped GEMM, combine) */
#define MXFP4_FLAG_CHECK 0x4u      /* synchronise `stream` and report out-of-range indices */
#define MXFP4_FLAG_GEMV_MFMA 0x8u  /* decode-shaped path on the MFMA kernel (16-row tiles) instead of
                                      the row-contiguous vector-ALU kernel */
/* Flags of mxfp4_moe_bucket. */
#define MXFP4_FLAG_BUCKET_ONE_BLOCK 0x10u  /* one workgroup does histogram, scan and scatter */
#define MXFP4_FLAG_BUCKET_MULTI_BLOCK 0x20u /* per-chunk histograms, a scan, per-chunk scatter */

/* Limits checked on the host. */
#define MXFP4_MAX_EXPERTS 8192
#define MXFP4_MAX_PAIRS (1 << 26) /* T * K */

/* Path identifiers returned by mxfp4_moe_select_path. */
#define MXFP4_PATH_GEMV 1
#define MXFP4_PATH_GEMM 2

/*
 * mxfp4_moe_linear - y = shared + sum_k p[t,k] W_{sel[t,k]} x[t], fp32 x/shared/y.
 * The argument list is the operation's: inputs x, packed, scales, sel, p,
 * shared; output y; sizes T (tokens), E (experts), O (output features),
 * G (groups per row, I = 32G), K (slots per token); the stream.
 * Scratch memory, when the chosen path needs it, is taken with
 * hipMallocAsync / hipFreeAsync on `stream`; use mxfp4_moe_linear_ex with a
 * caller workspace to avoid allocation (e.g. under graph capture).
 */
int mxfp4_moe_linear(const float* x, const uint8_t* packed, const uint8_t* scales,
                     const int32_t* sel, const float* p, const float* shared, float* y,
                     int64_t T, int64_t E, int64_t O, int64_t G, int64_t K, hipStream_t stream);

/* The same with bf16 x, shared and y (raw 16-bit patterns). p stays fp32. */
int mxfp4_moe_linear_bf16(const uint16_t* x, const uint8_t* packed, const uint8_t* scales,
                          const int32_t* sel, const float* p, const uint16_t* shared, uint16_t* y,
                          int64_t T, int64_t E, int64_t O, int64_t G, int64_t K, hipStream_t stream);

/*
 * mxfp4_moe_workspace_size - bytes of device workspace that
 * mxfp4_moe_linear_ex needs for these sizes, dtype and flags (written to
 * *bytes; 0 is a valid answer). Host-only; needs no GPU.
 */
int mxfp4_moe_workspace_size(int64_t T, int64_t E, int64_t O, int64_t G, int64_t K, int dtype,
                             uint32_t flags, size_t* bytes);

/*
 * mxfp4_moe_linear_ex - the operation with an explicit dtype (mxfp4_dtype),
 * flags and a caller-owned device workspace of at least
 * mxfp4_moe_workspace_size bytes (256-byte aligned). It allocates nothing
 * and does not synchronise unless MXFP4_FLAG_CHECK is set, so it may be
 * captured in a HIP graph. Calls that share one workspace must not overlap.
 * Paths (page "MoE Expert Kernels: Grouped Prefill and Mixed-Quant Compact
 * Experts", section 5: the schedule changes, the contract does not): the
 * decode-shaped path (routing, dequant-GEMV and combine in one launch) when
 * one launch takes every pair (at most 64 pairs, activations in LDS);
 * otherwise bucketing, the grouped GEMM on bf16 MFMA (fp32 activations as
 * their exact split into three bf16 pieces, every piece multiplied by the
 * same decoded weights into one fp32 sum) and the combine. Both paths meet
 * the same bars.
 */
int mxfp4_moe_linear_ex(const void* x, const uint8_t* packed, const uint8_t* scales,
                        const int32_t* sel, const float* p, const void* shared, void* y,
                        int64_t T, int64_t E, int64_t O, int64_t G, int64_t K, int dtype,
                        uint32_t flags, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * mxfp4_moe_linear_noalloc - mxfp4_moe_linear_ex (same arguments, dtype,
 * flags, results and errors) without a workspace argument and without any
 * allocation, for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc). It works in
 * a scratch array the library holds in device memory, one copy per device
 * (MXFP4_NOALLOC_SCRATCH_BYTES, kept until the process ends); its address is
 * looked up once per device on the first call there. Calls whose workspace
 * (mxfp4_moe_workspace_size) exceeds the array return
 * MXFP4_ERR_WORKSPACE_TOO_SMALL before anything is enqueued: every
 * decode-shaped call fits, prefill-shaped calls up to about
 * T * K * O * 4 = 30 MB of partial rows. All calls on one device share its
 * array, so calls that overlap on one device (two streams, two host threads)
 * race; order them, or use mxfp4_moe_linear_ex with workspaces of their own.
 */
#define MXFP4_NOALLOC_SCRATCH_BYTES (32u << 20)
int mxfp4_moe_linear_noalloc(const void* x, const uint8_t* packed, const uint8_t* scales,
                             const int32_t* sel, const float* p, const void* shared, void* y,
                             int64_t T, int64_t E, int64_t O, int64_t G, int64_t K, int dtype,
                             uint32_t flags, hipStream_t stream);

/*
 * mxfp4_moe_select_path - which path the _ex call takes for these sizes,
 * dtype and flags: MXFP4_PATH_GEMV or MXFP4_PATH_GEMM, or a negative
 * mxfp4_status. Host-only.
 */
int mxfp4_moe_select_path(int64_t T, int64_t E, int64_t O, int64_t G, int64_t K, int dtype,
                          uint32_t flags);

/*
 * mxfp4_moe_bucket - the token-to-expert bucketing on its own: a stable
 * counting sort of the P = T*K pairs (pair i = t*K + k) by expert index
 * (page "MoE Expert Kernels: Grouped Prefill and Mixed-Quant Compact
 * Experts", section 2: histogram, then scatter into per-expert contiguous
 * segments). Outputs (device, caller-owned, int32):
 *   count[E]          pairs per expert
 *   offsets[E + 1]    exclusive prefix sum of count
 *   perm[P]           perm[offsets[e] + r] = the r-th pair (in pair order) that chose e;
 *                     entries from offsets[E] on are left untouched (invalid pairs)
 *   slot_of_pair[P]   inverse of perm; -1 for a pair whose index is outside [0, E)
 *   n_invalid[1]      number of such pairs
 * flags selects the algorithm (MXFP4_FLAG_BUCKET_*; 0 = automatic). The
 * workspace (mxfp4_moe_bucket_workspace_size bytes) is caller-owned.
 */
int mxfp4_moe_bucket_workspace_size(int64_t T, int64_t K, int64_t E, uint32_t flags, size_t* bytes);
int mxfp4_moe_bucket(const int32_t* sel, int64_t T, int64_t K, int64_t E, int32_t* count,
                     int32_t* offsets, int32_t* perm, int32_t* slot_of_pair, int32_t* n_invalid,
                     uint32_t flags, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * mxfp4_decode_rows - decode rows row0 .. row0+nrows-1 of expert e into
 * out[nrows, 32G] (dtype fp32 or bf16), exactly: each value is
 * E2M1[n] * 2^(s - 127) rounded to the output type, which is exact except
 * where the value overflows to +-inf (s >= 253). This is the decode the
 * product kernels use, exported so that it can be tested bit for bit. It
 * writes decoded weights to memory and is not part of the fused path.
 */
int mxfp4_decode_rows(const uint8_t* packed, const uint8_t* scales, int64_t E, int64_t O,
                      int64_t G, int64_t e, int64_t row0, int64_t nrows, int dtype, void* out,
                      hipStream_t stream);

/*
 * mxfp4_moe_gemm_stage - run again only the grouped GEMM of the
 * prefill-shaped path (bf16): the bucketing results and M-tile list are the
 * ones a previous mxfp4_moe_linear_ex call with the same sizes, dtype
 * MXFP4_DTYPE_BF16 and the prefill-shaped path (chosen for these sizes or
 * forced with MXFP4_FLAG_FORCE_GEMM) left in `workspace`; the fp32 partial
 * rows it writes go to the same workspace. For timing and inspection of
 * that one kernel (page "MoE Expert Kernels: Grouped Prefill and
 * Mixed-Quant Compact Experts", section 2: one matmul per expert segment).
 * Returns MXFP4_ERR_WORKSPACE_TOO_SMALL and MXFP4_ERR_INVALID_ARG as _ex
 * does. The workspace must hold that call's results untouched: the kernel
 * trusts the expert indices, positions and tile list it finds there, so
 * anything else is undefined behaviour.
 */
int mxfp4_moe_gemm_stage(const void* x, const uint8_t* packed, const uint8_t* scales,
                         int64_t T, int64_t E, int64_t O, int64_t G, int64_t K,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * mxfp4_moe_swiglu_ex - the routed SwiGLU expert block, bf16 x, shared, y
 * (raw 16-bit patterns), p fp32:
 *   y[t] = shared[t] + sum_k p[t,k] * Down_e(silu(Gate_e x[t]) * (Up_e x[t])),  e = sel[t,k],
 * silu(v) = v / (1 + e^-v) (page "MoE Expert Kernels: Grouped Prefill and
 * Mixed-Quant Compact Experts", section 1: every routed expert is a SwiGLU
 * whose routing-weighted outputs are summed; the exo pull request page
 * stacks gate and up along the output rows, read here as gate first).
 *   gu_packed (E, 2F, G, 16), gu_scales (E, 2F, G): rows [0, F) gate, rows
 *     [F, 2F) up, over I = 32G inputs (x is (T, I));
 *   dn_packed (E, O, F/32, 16), dn_scales (E, O, F/32): the down projection;
 *   shared, y: (T, O).
 * F must be a positive multiple of 32. Each pair's intermediate silu(gate) *
 * up is rounded to bf16 (the down projection's MFMA operand); the
 * projections accumulate in fp32 and the K slots are summed in order in fp32,
 * as in mxfp4_moe_linear_ex. Work: bucketing, a grouped GEMM with the SwiGLU
 * in its epilogue, a grouped GEMM of the down projection over the sorted
 * rows, the combine. Caller-owned device workspace of
 * mxfp4_moe_swiglu_workspace_size bytes (256-byte aligned); flags 0 or
 * MXFP4_FLAG_CHECK. Allocates nothing; may be captured in a graph. Errors as
 * mxfp4_moe_linear_ex; MXFP4_ERR_UNSUPPORTED when T*I*2, T*K*F*2, 2F*G*16 or
 * O*F/2 bytes reach 2^31. Same aliasing rule: y may be shared, nothing else.
 */
int mxfp4_moe_swiglu_workspace_size(int64_t T, int64_t E, int64_t F, int64_t G, int64_t O, int64_t K,
                                    size_t* bytes);
int mxfp4_moe_swiglu_ex(const uint16_t* x, const uint8_t* gu_packed, const uint8_t* gu_scales,
                        const uint8_t* dn_packed, const uint8_t* dn_scales, const int32_t* sel,
                        const float* p, const uint16_t* shared, uint16_t* y, int64_t T, int64_t E,
                        int64_t F, int64_t G, int64_t O, int64_t K, uint32_t flags, void* workspace,
                        size_t workspace_bytes, hipStream_t stream);

/*
 * mxfp4_quantize_mxfp8 - activations to MXFP8: per token and block of 32
 * inputs one E8M0 scale byte s (2^(s-127)) and 32 E4M3 codes (OCP
 * Microscaling family, blocks of 32 codes sharing one E8M0 scale: page
 * "MXFP4 Dequant", "Overview"). Readings, the pages being silent: E4M3 has
 * bias 7, 3 mantissa bits, largest value 448; the scale is the smallest power
 * of two 2^X with max|block| <= 448 * 2^X (X clamped to [-127, 127]; an
 * all-zero block takes -127); each code is x / 2^X rounded to nearest, ties
 * to even, sign kept.
 *   x (T, I) bf16 raw bits, I a positive multiple of 32, 8-byte aligned,
 *   finite (an infinite or NaN input leaves its block's codes and scale byte
 *   unspecified; the exact layer's result is not finite either);
 *   codes (T, ld) and scale_bytes (T, ld / 32), ld >= I a multiple of 32,
 *   codes 4-byte aligned; columns [I, ld) get zero codes and scale bytes 0.
 * T * ld < 2^31; no overlap. MXFP4_ERR_INVALID_ARG otherwise. Enqueued on
 * `stream`, no allocation.
 */
int mxfp4_quantize_mxfp8(const uint16_t* x, int64_t T, int64_t I, int64_t ld, uint8_t* codes, uint8_t* scale_bytes,
                         hipStream_t stream);

/*
 * mxfp4_moe_linear_mxfp8_ex - the block-scaled variant of the layer (bf16
 * x, shared, y; p fp32): the routed linear of mxfp4_moe_linear_ex computed
 * with the activations quantised to MXFP8 as mxfp4_quantize_mxfp8 does and
 * multiplied by the packed weights and scale bytes as stored on gfx950's
 * block-scaled MFMA (no weight dequantisation):
 *   y[t] = shared[t] + sum_k p[t,k] * W_sel[t,k] q(x[t]).
 * This is an approximation of mxfp4_moe_linear_ex (the activation rounding,
 * relative L2 error a few percent), reported separately from it. Weight
 * scale bytes must be below 255 (the MFMA reads 255 as NaN). Needs O % 4 == 0,
 * T * 128 * ceil(32G / 128) < 2^31 and O * G * 16 < 2^31, else
 * MXFP4_ERR_UNSUPPORTED. Work: bucketing, quantisation, a grouped GEMM on the
 * scaled MFMA, the combine. Caller-owned workspace of
 * mxfp4_moe_mxfp8_workspace_size bytes (256-byte aligned); flags 0 or
 * MXFP4_FLAG_CHECK. Allocates nothing; may be captured in a graph. Other
 * errors and the aliasing rule as mxfp4_moe_linear_ex.
 */
int mxfp4_moe_mxfp8_workspace_size(int64_t T, int64_t E, int64_t O, int64_t G, int64_t K, size_t* bytes);
int mxfp4_moe_linear_mxfp8_ex(const uint16_t* x, const uint8_t* packed, const uint8_t* scales, const int32_t* sel,
                              const float* p, const uint16_t* shared, uint16_t* y, int64_t T, int64_t E, int64_t O,
                              int64_t G, int64_t K, uint32_t flags, void* workspace, size_t workspace_bytes,
                              hipStream_t stream);

/*
 * Load-time weight repack for the block-scaled variant and the prepared
 * decode-shaped path (mxfp4_moe_decode_prepared_ex). The prepared buffer
 * holds, per expert, per N-tile of 128 output rows, per chunk of 128 inputs
 * (4 groups) and per 16-row fragment, 64 group slots of 16 code bytes in the
 * order the scaled MFMA's weight operand takes them (slot l: row 16 f + (l mod
 * 16) of the tile, group 4 q + l / 16), so that every wave-wide weight request
 * reads 1 KB of consecutive bytes; after all code slots come the slots' scale
 * bytes, per (expert, tile, chunk) and half of the 8 fragments as 64 lanes x 4
 * bytes (byte 4 l + f mod 4 for fragment f, slot l), so that one 4-byte
 * request per lane brings a lane its four fragments' scales. Rows past O and
 * groups past G are zero. The canonical [E, O, G, 16] / [E, O, G] arrays are
 * the pages' format (page "MXFP4 Experts", shape paragraph); this is a byte
 * permutation of them plus zero padding, nothing is decoded.
 *   mxfp4_mx_prepared_size: bytes of the prepared buffer (17 per slot).
 *   mxfp4_prepare_mx: packed (E, O, G, 16) and scales (E, O, G) device arrays
 *     (packed 16-byte aligned) -> prepared (16-byte aligned, bytes >= the
 *     size; no overlap). Enqueued on `stream`; call once per weight set.
 *   mxfp4_moe_linear_mxfp8_prepared_ex: mxfp4_moe_linear_mxfp8_ex reading the
 *     prepared buffer instead of packed and scales; the same workspace size,
 *     flags, errors and results bit for bit.
 * Sizes as mxfp4_moe_linear_mxfp8_ex (MXFP4_ERR_UNSUPPORTED also when one
 * expert's prepared codes reach 2^31 bytes).
 */
int mxfp4_mx_prepared_size(int64_t E, int64_t O, int64_t G, size_t* bytes);
int mxfp4_prepare_mx(const uint8_t* packed, const uint8_t* scales, int64_t E, int64_t O, int64_t G, void* prepared,
                     size_t bytes, hipStream_t stream);
int mxfp4_moe_linear_mxfp8_prepared_ex(const uint16_t* x, const void* prepared, const int32_t* sel, const float* p,
                                       const uint16_t* shared, uint16_t* y, int64_t T, int64_t E, int64_t O,
                                       int64_t G, int64_t K, uint32_t flags, void* workspace, size_t workspace_bytes,
                                       hipStream_t stream);

/*
 * The block-scaled variant with MXFP4 activations (both operands of the
 * scaled MFMA in E2M1: the FP4 x FP4 form). The pages define MXFP4 for
 * blocks of 32 values (page "MXFP4 Dequant", "Overview") without saying how
 * activations would be quantised to it; readings as for MXFP8: per token and
 * block of 32 inputs the smallest power of two 2^X with max|block| <= 6 * 2^X
 * (scale byte X + 127, X clamped to [-127, 127], an all-zero block -127), each
 * element x / 2^X rounded to the nearest E2M1 magnitude (0, .5, 1, 1.5, 2, 3,
 * 4, 6), ties to the even code, sign kept (code sign << 3 | magnitude index).
 *   mxfp4_quantize_mxfp4: x (T, I) bf16 raw bits, I a positive multiple of
 *     32, 8-byte aligned, finite as for MXFP8 -> codes (T, ld / 2) bytes, two codes per byte, the
 *     first in the low nibble (the weights' order), and scale_bytes
 *     (T, ld / 32); ld >= I a multiple of 32, codes 4-byte aligned; columns
 *     [I, ld) get zero codes and scale bytes 0. T * ld < 2^31; no overlap.
 *     MXFP4_ERR_INVALID_ARG otherwise. Enqueued on `stream`, no allocation.
 *   mxfp4_moe_linear_mxfp4act_ex: mxfp4_moe_linear_mxfp8_ex with the
 *     activations quantised by mxfp4_quantize_mxfp4 instead: the routed linear
 *     of the quantised activations, an approximation of mxfp4_moe_linear_ex
 *     (the E2M1 rounding of the activations, relative L2 around 0.1 on
 *     normally distributed activations), reported separately. Sizes, flags,
 *     errors, aliasing and the 255 rule as mxfp4_moe_linear_mxfp8_ex;
 *     workspace of mxfp4_moe_mxfp4act_workspace_size bytes.
 *   mxfp4_moe_linear_mxfp4act_prepared_ex: the same on the buffer of
 *     mxfp4_prepare_mx; results bit for bit those of the canonical call.
 */
int mxfp4_quantize_mxfp4(const uint16_t* x, int64_t T, int64_t I, int64_t ld, uint8_t* codes, uint8_t* scale_bytes,
                         hipStream_t stream);
int mxfp4_moe_mxfp4act_workspace_size(int64_t T, int64_t E, int64_t O, int64_t G, int64_t K, size_t* bytes);
int mxfp4_moe_linear_mxfp4act_ex(const uint16_t* x, const uint8_t* packed, const uint8_t* scales, const int32_t* sel,
                                 const float* p, const uint16_t* shared, uint16_t* y, int64_t T, int64_t E, int64_t O,
                                 int64_t G, int64_t K, uint32_t flags, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream);
int mxfp4_moe_linear_mxfp4act_prepared_ex(const uint16_t* x, const void* prepared, const int32_t* sel,
                                          const float* p, const uint16_t* shared, uint16_t* y, int64_t T, int64_t E,
                                          int64_t O, int64_t G, int64_t K, uint32_t flags, void* workspace,
                                          size_t workspace_bytes, hipStream_t stream);

/*
 * The decode-shaped path (routing, dequant-GEMV and combine in one launch per
 * token chunk; page "MXFP4 Routed Expert Linear", "Route, weight, and add the
 * shared path") on weights repacked by mxfp4_prepare_mx: the MFMA decode
 * kernel, each workgroup's 16 rows being one prepared fragment whose 1 KB
 * blocks are loaded straight into the MFMA operand.
 *   mxfp4_moe_decode_prepared_ex: arguments, dtypes (MXFP4_DTYPE_F32 or
 *     MXFP4_DTYPE_BF16), results, bars and errors as mxfp4_moe_linear_ex with
 *     MXFP4_FLAG_FORCE_GEMV | MXFP4_FLAG_GEMV_MFMA, with `prepared` in place
 *     of packed and scales; the workspace is mxfp4_moe_workspace_size(T, E,
 *     O, G, K, dtype, MXFP4_FLAG_FORCE_GEMV, ...) bytes; flags 0 or
 *     MXFP4_FLAG_CHECK. Allocates nothing; may be captured in a graph.
 */
int mxfp4_moe_decode_prepared_ex(const void* x, const void* prepared, const int32_t* sel, const float* p,
                                 const void* shared, void* y, int64_t T, int64_t E, int64_t O, int64_t G, int64_t K,
                                 int dtype, uint32_t flags, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream);

/*
 * The bf16 routed linear on prepared weights (page "MXFP4 Routed
 * Expert Linear", "Reconstruct the matrix in the right orientation", for the
 * product): the prefill-shaped path - bucketing, a grouped GEMM that brings
 * each 1 KB block of prepared codes into LDS with one request, decodes it in
 * registers and multiplies on bf16 MFMA with fp32 accumulation, and the
 * combine.
 *   mxfp4_prepare_bf16: the repack of mxfp4_prepare_mx (same slots, scale
 *     array, size, arguments and errors) with the code blocks of each tile
 *     and chunk in dword-interleaved order: block 4 h + s holds, at bytes
 *     16 l + 4 (f mod 4) .. +3, bytes 4 s .. 4 s + 3 of slot l of fragment f
 *     (f = 4 h .. 4 h + 3), so that one 16-byte read gives a lane one MFMA
 *     step's codes of four fragments.
 *   mxfp4_moe_linear_prepared_ex: reads a buffer of mxfp4_prepare_bf16;
 *     x (T, 32G), shared and y (T, O) bf16 as
 *     mxfp4_moe_linear_ex with MXFP4_DTYPE_BF16; the workspace is
 *     mxfp4_moe_workspace_size(T, E, O, G, K, MXFP4_DTYPE_BF16,
 *     MXFP4_FLAG_FORCE_GEMM, ...) bytes; flags 0 or MXFP4_FLAG_CHECK; errors
 *     as mxfp4_moe_linear_ex. Results within the bf16 bar of the exact layer
 *     (the same products as the canonical path, summed in another order).
 *   mxfp4_moe_gemm_stage_prepared: the grouped GEMM of that path alone, on
 *     the bucketing a previous mxfp4_moe_linear_prepared_ex call with the
 *     same sizes left in `workspace` (as mxfp4_moe_gemm_stage).
 * MXFP4_ERR_UNSUPPORTED unless O % 4 == 0, T * 64G < 2^31 and one expert's
 * prepared codes stay below 2^31 bytes. Allocates nothing; may be captured
 * in a graph.
 */
int mxfp4_prepare_bf16(const uint8_t* packed, const uint8_t* scales, int64_t E, int64_t O, int64_t G, void* prepared,
                       size_t bytes, hipStream_t stream);
int mxfp4_moe_linear_prepared_ex(const uint16_t* x, const void* prepared, const int32_t* sel, const float* p,
                                  const uint16_t* shared, uint16_t* y, int64_t T, int64_t E, int64_t O, int64_t G,
                                  int64_t K, uint32_t flags, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream);
int mxfp4_moe_gemm_stage_prepared(const uint16_t* x, const void* prepared, int64_t T, int64_t E, int64_t O,
                                  int64_t G, int64_t K, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * The SwiGLU expert block on prepared weights (page "MoE Expert Kernels:
 * Grouped Prefill and Mixed-Quant Compact Experts", section 1; the weights
 * repacked once at load time, nothing decoded).
 *   mxfp4_prepare_swiglu: gate/up packed (E, 2F, G, 16) and scales (E, 2F, G)
 *     (gate rows [0, F) over up rows [F, 2F)) -> the prepared layout of
 *     mxfp4_prepare_bf16 with the rows reordered so that each 128-row tile holds
 *     the gate rows of 64 features followed by their up rows. Size:
 *     mxfp4_mx_prepared_size(E, 2F, G). Alignment, overlap and errors as
 *     mxfp4_prepare_mx; F a multiple of 32.
 *   mxfp4_moe_swiglu_prepared_ex: mxfp4_moe_swiglu_ex with gu_prepared from
 *     mxfp4_prepare_swiglu and dn_prepared from mxfp4_prepare_bf16(dn_packed,
 *     dn_scales, E, O, F / 32, ...); the same workspace size, flags, errors
 *     and bar (both GEMMs on the register-decode kernel). Also
 *     MXFP4_ERR_UNSUPPORTED unless O % 4 == 0 and one expert's prepared codes
 *     stay below 2^31 bytes. Allocates nothing; may be captured in a graph.
 */
int mxfp4_prepare_swiglu(const uint8_t* gu_packed, const uint8_t* gu_scales, int64_t E, int64_t F, int64_t G,
                         void* prepared, size_t bytes, hipStream_t stream);
int mxfp4_moe_swiglu_prepared_ex(const uint16_t* x, const void* gu_prepared, const void* dn_prepared,
                                 const int32_t* sel, const float* p, const uint16_t* shared, uint16_t* y, int64_t T,
                                 int64_t E, int64_t F, int64_t G, int64_t O, int64_t K, uint32_t flags,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * mxfp4_moe_route - the router that produces sel and p from router logits
 * (page "MoE Expert Kernels: Grouped Prefill and Mixed-Quant Compact
 * Experts", section 1, for both router kinds and the floor on the selected
 * mass; the exo pull request page, router bullets, for the tie order, the
 * left-to-right sum, the 1e-20 addend and the scale).
 *   logits (T, E) fp32 device, row-major; bias (E) fp32 device or NULL;
 *   sel (T, K) int32 and p (T, K) fp32 device outputs, row-major.
 * mode MXFP4_ROUTE_SOFTMAX: prob = softmax(logits[t]) over all E experts;
 *   the K experts with the largest logits are chosen (the same order as
 *   their probabilities); p[t,k] = prob[sel] / max(sum of the K chosen probs,
 *   2^-14) * scale. bias must be NULL.
 * mode MXFP4_ROUTE_SIGMOID: s = 1 / (1 + e^-logits[t]); the K experts with
 *   the largest s + bias are chosen (bias NULL reads as zeros); p[t,k] =
 *   s[sel] / (s[sel_0] + ... + s[sel_{K-1}] + 1e-20) * scale, summed left to
 *   right. The bias steers the choice only, never the weights.
 * In both modes sel[t] lists K distinct experts by descending key, equal keys
 * in ascending index order; a NaN key counts as -inf and -0 as +0. Without a
 * bias the sigmoid router ranks by the logits (the same order as the exact
 * scores). Arithmetic is fp32; the sigmoid uses the hardware reciprocal. Needs 1 <= K <= min(E, MXFP4_ROUTE_MAX_K), E <= MXFP4_ROUTE_MAX_EXPERTS,
 * T < 2^30, scale finite, 4-byte aligned buffers and outputs that overlap
 * neither each other nor the inputs; anything else is MXFP4_ERR_INVALID_ARG.
 * T = 0 does nothing. Enqueued on `stream`, no synchronisation, no
 * allocation; may be captured in a graph.
 */
#define MXFP4_ROUTE_SOFTMAX 0
#define MXFP4_ROUTE_SIGMOID 1
#define MXFP4_ROUTE_MAX_EXPERTS 1024
#define MXFP4_ROUTE_MAX_K 64
int mxfp4_moe_route(const float* logits, const float* bias, int64_t T, int64_t E, int64_t K, int mode, float scale,
                    int32_t* sel, float* p, hipStream_t stream);

/*
 * mxfp4_stream_read - a measurement helper, not a step of the layer: read
 * `bytes` bytes of the device buffer `buf` once, in 16-byte pieces spread
 * over `blocks` workgroups of 256 threads (0: min(bytes / 4096, 2048)), and
 * write nothing except, with a chance of about 2^-32, one word of `sink`
 * (a device array of at least `blocks` (or 2048) uint32). Its time is the
 * practical read ceiling the decode-shaped path is compared with (the
 * benchmark's stream workload). buf 16-byte aligned, bytes a multiple of 16
 * below 2^40; MXFP4_ERR_INVALID_ARG otherwise. Enqueued on `stream`.
 */
int mxfp4_stream_read(const void* buf, size_t bytes, int blocks, uint32_t* sink, hipStream_t stream);

/*
 * mxfp4_moe_route_grouped - the group-limited sigmoid router (page "MoE
 * Expert Kernels: Grouped Prefill and Mixed-Quant Compact Experts", section
 * 1, the first of its two routers):
 *   choice score c_e = sigmoid(logits[t, e]) + bias[e] (bias NULL reads as
 *     zeros; a NaN score counts as -inf);
 *   the E experts form n_group groups of E / n_group consecutive experts; a
 *     group's score is the sum of its two largest choice scores;
 *   the topk_group groups with the largest scores are kept (equal scores:
 *     the lower group first);
 *   sel[t] = the K experts of the kept groups with the largest choice
 *     scores, in descending order (equal scores: the lower index first);
 *   p[t, k] = sigmoid(logits[t, sel[t, k]]) (the bias steers the choice
 *     only), divided by (the chosen scores summed left to right + 1e-20) when
 *     renormalize is 1 (as mxfp4_moe_route's sigmoid mode; 0 keeps the
 *     gathered scores), times scale.
 * Arithmetic is fp32 (the sigmoid with the hardware reciprocal). Shapes,
 * alignment, overlap rules and errors as mxfp4_moe_route, and: 2 <= E <=
 * MXFP4_ROUTE_MAX_EXPERTS, 1 <= n_group <= MXFP4_ROUTE_MAX_GROUPS dividing E
 * with E / n_group >= 2, 1 <= topk_group <= n_group, 1 <= K <=
 * min(MXFP4_ROUTE_MAX_K, topk_group * E / n_group), renormalize 0 or 1;
 * anything else is MXFP4_ERR_INVALID_ARG. Enqueued on `stream`, no
 * synchronisation, no allocation; may be captured in a graph.
 */
#define MXFP4_ROUTE_MAX_GROUPS 64
int mxfp4_moe_route_grouped(const float* logits, const float* bias, int64_t T, int64_t E, int64_t K,
                            int64_t n_group, int64_t topk_group, int renormalize, float scale, int32_t* sel,
                            float* p, hipStream_t stream);

/* A static, human-readable name of a status code. */
const char* mxfp4_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MXFP4_MOE_H */
