// C ABI of the MXFP4 routed-expert linear (declarations and conventions in
// include/mxfp4_moe.h). This file holds the host side only: argument checks
// that need no GPU, the workspace layout, the gfx950 check, the choice
// between the decode-shaped and the prefill-shaped path, and the launches.
#include "mxfp4_moe.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cmath>
#include <cstring>

#include "launch.h"

namespace {

using namespace mxfp4;

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct Dims {
  int64_t T, E, O, G, K, P, I;
};

bool mul_ok(int64_t a, int64_t b, int64_t* out) { return !__builtin_mul_overflow(a, b, out) && *out >= 0; }

int check_dims(int64_t T, int64_t E, int64_t O, int64_t G, int64_t K, Dims* d) {
  if (T < 0 || E < 1 || O < 1 || G < 1 || K < 1) return MXFP4_ERR_INVALID_ARG;
  if (E > MXFP4_MAX_EXPERTS || O > (int64_t(1) << 30) || G > (int64_t(1) << 24)) return MXFP4_ERR_INVALID_ARG;
  int64_t P = 0, t = 0;
  if (!mul_ok(T, K, &P) || P > MXFP4_MAX_PAIRS) return MXFP4_ERR_INVALID_ARG;
  // the packed tensor's byte size and the partial buffer must be addressable
  if (!mul_ok(E, O, &t) || !mul_ok(t, G, &t) || !mul_ok(t, 16, &t)) return MXFP4_ERR_INVALID_ARG;
  if (!mul_ok(P, O, &t) || !mul_ok(t, 4, &t)) return MXFP4_ERR_INVALID_ARG;
  if (!mul_ok(T, 32 * G, &t) || !mul_ok(t, 4, &t)) return MXFP4_ERR_INVALID_ARG;
  *d = Dims{T, E, O, G, K, P, 32 * G};
  return MXFP4_OK;
}

int dtype_size(int dtype) { return dtype == MXFP4_DTYPE_F32 ? 4 : (dtype == MXFP4_DTYPE_BF16 ? 2 : 0); }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (na == 0 || nb == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + nb && b0 < a0 + na;
}

// Prefill-shaped grouped GEMM on canonical weights with bf16 activations: the
// register-decode kernel (weights brought into LDS by DMA, 8-wave workgroups
// over 128 pairs x 512 rows) where it applies (O % 4 == 0), else the
// LDS-staged kernel of gemm.hip. Both give the same results contract.
bool regdec_canon_ok(int64_t T, int64_t O, int64_t G) { return gemm_regdec_canon_supported(T, O, G); }

hipError_t launch_canonical_gemm(const uint16_t* x, const uint8_t* packed, const uint8_t* scales, const int32_t* perm,
                                 const GemmTile* tiles, const int32_t* n_tiles, int64_t max_tiles, float* part,
                                 int64_t T, int64_t K, int64_t O, int64_t G, hipStream_t stream) {
  if (regdec_canon_ok(T, O, G))
    return launch_gemm_regdec_canon(x, packed, scales, perm, tiles, n_tiles, max_tiles, part, (int)T, (int)K, (int)O,
                                    (int)G, stream);
  return launch_gemm_bf16(x, packed, scales, perm, tiles, n_tiles, max_tiles, part, (int)T, (int)K, (int)O, (int)G,
                          stream);
}

// Decode-shaped kernel: the row-contiguous one unless the MFMA one is asked
// for. Both address an expert's packed bytes with 32-bit buffer offsets, so
// the decode-shaped path needs O * G * 16 < 2^31.
bool use_rows_kernel(uint32_t flags) { return !(flags & MXFP4_FLAG_GEMV_MFMA); }

int64_t gemv_tokens_per_launch(const Dims& d, int dtype, uint32_t flags) {
  if (!gemv_rows_supported((int)d.O, (int)d.G)) return 0;
  return use_rows_kernel(flags) ? gemv_rows_tokens_per_launch((int)d.K, (int)d.E, (int)d.G, dtype)
                                : decode_tokens_per_launch((int)d.K, (int)d.E, (int)d.G, dtype);
}

// Activation planes the grouped GEMM reads: bf16 x as is, fp32 x as its
// exact three-piece bf16 split.
int gemm_planes(int dtype) { return dtype == MXFP4_DTYPE_F32 ? 3 : 1; }

int select_path(const Dims& d, int dtype, uint32_t flags) {
  if (dtype_size(dtype) == 0) return MXFP4_ERR_INVALID_ARG;
  const bool fv = flags & MXFP4_FLAG_FORCE_GEMV, fm = flags & MXFP4_FLAG_FORCE_GEMM;
  if (fv && fm) return MXFP4_ERR_INVALID_ARG;
  // tokens one fused decode-shaped launch takes: at most 64 pairs, and the
  // tokens' activations and partial rows must fit LDS
  const int64_t tpl = gemv_tokens_per_launch(d, dtype, flags);
  const bool gemv_ok = tpl >= 1;
  const bool gemm_ok = gemm_supported(d.T, d.O, d.G, gemm_planes(dtype));
  if (fv) return gemv_ok ? MXFP4_PATH_GEMV : MXFP4_ERR_UNSUPPORTED;
  if (fm) return gemm_ok ? MXFP4_PATH_GEMM : MXFP4_ERR_UNSUPPORTED;
  // The decode-shaped path when one launch takes every pair: each selected
  // expert's bytes are then read once. Past that, successive launches would
  // read a selected expert once per launch, while the grouped GEMM reads it
  // once per 128 of its pairs.
  if (gemv_ok && (d.T <= tpl || !gemm_ok)) return MXFP4_PATH_GEMV;
  return gemm_ok ? MXFP4_PATH_GEMM : MXFP4_ERR_UNSUPPORTED;
}

// Workspace layout. GEMV: n_invalid only. GEMM: bucketing arrays, the M-tile
// list, the fp32 partial rows [P, O] and, for fp32 activations, their
// three bf16 planes [3, T, I].
struct Layout {
  size_t n_invalid, count, offsets, perm, slot, bcount, tiles, n_tiles, part, xs, total;
};

Layout layout(const Dims& d, int path, int dtype = MXFP4_DTYPE_BF16) {
  Layout L{};
  size_t off = 0;
  L.n_invalid = off;
  off += kAlign;
  if (path == MXFP4_PATH_GEMM) {
    const int64_t nch = bucket_chunks(d.P);
    L.count = off;
    off = align_up(off + d.E * 4);
    L.offsets = off;
    off = align_up(off + (d.E + 1) * 4);
    L.perm = off;
    off = align_up(off + d.P * 4);
    L.slot = off;
    off = align_up(off + d.P * 4);
    L.bcount = off;
    off = align_up(off + (nch * d.E + nch) * 4);
    L.tiles = off;
    off = align_up(off + gemm_max_tiles(d.P, d.E) * sizeof(GemmTile));
    L.n_tiles = off;
    off += kAlign;
    L.part = off;
    off = align_up(off + (size_t)d.P * d.O * 4);
    if (dtype == MXFP4_DTYPE_F32) {
      L.xs = off;
      off = align_up(off + (size_t)3 * d.T * d.I * 2);
    }
  }
  L.total = off;
  return L;
}

std::atomic<int> g_arch[64];  // 0 unknown, 1 gfx950, -1 another device
std::atomic<int> g_cus[64];   // compute units of the device (0 unknown)

int check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MXFP4_ERR_HIP;
  int v = (dev >= 0 && dev < 64) ? g_arch[dev].load(std::memory_order_relaxed) : 0;
  if (v == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MXFP4_ERR_HIP;
    v = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 && (prop.gcnArchName[6] == '\0' || prop.gcnArchName[6] == ':'))
            ? 1
            : -1;
    if (dev >= 0 && dev < 64) {
      g_cus[dev].store(prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 1, std::memory_order_relaxed);
      g_arch[dev].store(v, std::memory_order_relaxed);
    }
  }
  return v == 1 ? MXFP4_OK : MXFP4_ERR_UNSUPPORTED_DEVICE;
}

// compute units of the current device (after check_device)
int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  const int n = g_cus[dev].load(std::memory_order_relaxed);
  return n > 0 ? n : 256;
}

int check_linear_args(const void* x, const uint8_t* packed, const uint8_t* scales, const int32_t* sel, const float* p,
                      const void* shared, void* y, const Dims& d, int dtype) {
  const int es = dtype_size(dtype);
  if (es == 0) return MXFP4_ERR_INVALID_ARG;
  if (d.T == 0) return MXFP4_OK;
  if (!x || !packed || !scales || !sel || !p || !shared || !y) return MXFP4_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(packed, 16) || !aligned(sel, 4) || !aligned(p, 4) || !aligned(shared, es) ||
      !aligned(y, es))
    return MXFP4_ERR_INVALID_ARG;
  const size_t ny = (size_t)d.T * d.O * es;
  const size_t sizes[6] = {(size_t)d.T * d.I * es, (size_t)d.E * d.O * d.G * 16, (size_t)d.E * d.O * d.G,
                           (size_t)d.P * 4, (size_t)d.P * 4, ny};
  const void* ptrs[6] = {x, packed, scales, sel, p, shared};
  for (int i = 0; i < 6; i++) {
    if (i == 5 && ptrs[i] == y) continue;  // in place on shared is allowed
    if (overlap(y, ny, ptrs[i], sizes[i])) return MXFP4_ERR_INVALID_ARG;
  }
  return MXFP4_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MXFP4_OK : MXFP4_ERR_HIP; }

int run_linear(const void* x, const uint8_t* packed, const uint8_t* scales, const int32_t* sel, const float* p,
               const void* shared, void* y, const Dims& d, int dtype, uint32_t flags, void* ws, size_t ws_bytes,
               hipStream_t stream) {
  const int path = select_path(d, dtype, flags);
  if (path < 0) return path;
  const Layout L = layout(d, path, dtype);
  if (ws_bytes < L.total) return MXFP4_ERR_WORKSPACE_TOO_SMALL;
  if (!ws || !aligned(ws, kAlign)) return MXFP4_ERR_INVALID_ARG;
  int st = check_device();
  if (st != MXFP4_OK) return st;
  char* base = static_cast<char*>(ws);
  int32_t* n_invalid = reinterpret_cast<int32_t*>(base + L.n_invalid);
  hipError_t err = hipSuccess;
  const int es = dtype_size(dtype);
  if (path == MXFP4_PATH_GEMV && d.T == 1 && use_rows_kernel(flags) && gemv_one_supported((int)d.O, (int)d.G, (int)d.K)) {
    // one token: its activations stay in registers for the whole call
    err = launch_gemv_one(x, packed, scales, sel, p, shared, y, (int)d.E, (int)d.O, (int)d.G, (int)d.K, dtype, n_invalid,
                          device_cus(), stream);
  } else if (path == MXFP4_PATH_GEMV) {
    // token chunks whose pairs and activations fit one fused launch
    const int64_t tc = gemv_tokens_per_launch(d, dtype, flags);
    if (tc < 1) return MXFP4_ERR_UNSUPPORTED;
    const auto launch = use_rows_kernel(flags) ? launch_gemv_rows : launch_decode_fused;
    int chunk = 0;
    for (int64_t t0 = 0; t0 < d.T && err == hipSuccess; t0 += tc, chunk++) {
      const int64_t tn = (d.T - t0 < tc) ? d.T - t0 : tc;
      err = launch(static_cast<const char*>(x) + t0 * d.I * es, packed, scales, sel + t0 * d.K,
                   p + t0 * d.K, static_cast<const char*>(shared) + t0 * d.O * es,
                   static_cast<char*>(y) + t0 * d.O * es, (int)tn, (int)d.E, (int)d.O, (int)d.G, (int)d.K, dtype,
                   n_invalid, chunk, stream);
    }
  } else {
    BucketOut b;
    b.count = reinterpret_cast<int32_t*>(base + L.count);
    b.offsets = reinterpret_cast<int32_t*>(base + L.offsets);
    b.perm = reinterpret_cast<int32_t*>(base + L.perm);
    b.slot_of_pair = reinterpret_cast<int32_t*>(base + L.slot);
    b.n_invalid = n_invalid;
    b.tiles = reinterpret_cast<GemmTile*>(base + L.tiles);
    b.n_tiles = reinterpret_cast<int32_t*>(base + L.n_tiles);
    err = launch_bucket_multi(sel, (int)d.P, (int)d.E, reinterpret_cast<int32_t*>(base + L.bcount), b, stream);
    float* part = reinterpret_cast<float*>(base + L.part);
    if (dtype == MXFP4_DTYPE_F32) {
      uint16_t* xs = reinterpret_cast<uint16_t*>(base + L.xs);
      if (err == hipSuccess) err = launch_split3(static_cast<const float*>(x), d.T * d.I, xs, stream);
      if (err == hipSuccess)
        err = launch_gemm_f32(xs, packed, scales, b.perm, b.tiles, b.n_tiles, gemm_max_tiles(d.P, d.E), part,
                              (int)d.T, (int)d.K, (int)d.O, (int)d.G, stream);
    } else if (err == hipSuccess) {
      err = launch_canonical_gemm(static_cast<const uint16_t*>(x), packed, scales, b.perm, b.tiles, b.n_tiles,
                                  gemm_max_tiles(d.P, d.E), part, d.T, d.K, d.O, d.G, stream);
    }
    if (err == hipSuccess)
      err = launch_combine(reinterpret_cast<const float*>(base + L.part), b.slot_of_pair, p, shared, y, (int)d.T,
                           (int)d.K, (int)d.O, dtype, stream);
  }
  if (err != hipSuccess) return MXFP4_ERR_HIP;
  if (flags & MXFP4_FLAG_CHECK) {
    if (hipStreamSynchronize(stream) != hipSuccess) return MXFP4_ERR_HIP;
    int32_t inv = 0;
    if (hipMemcpy(&inv, n_invalid, 4, hipMemcpyDeviceToHost) != hipSuccess) return MXFP4_ERR_HIP;
    if (inv != 0) return MXFP4_ERR_INVALID_INDEX;
  }
  return MXFP4_OK;
}

int linear_alloc(const void* x, const uint8_t* packed, const uint8_t* scales, const int32_t* sel, const float* p,
                 const void* shared, void* y, int64_t T, int64_t E, int64_t O, int64_t G, int64_t K, int dtype,
                 hipStream_t stream) {
  Dims d;
  int st = check_dims(T, E, O, G, K, &d);
  if (st != MXFP4_OK) return st;
  st = check_linear_args(x, packed, scales, sel, p, shared, y, d, dtype);
  if (st != MXFP4_OK || d.T == 0) return st;
  const int path = select_path(d, dtype, 0);
  if (path < 0) return path;
  const size_t bytes = layout(d, path, dtype).total;
  st = check_device();
  if (st != MXFP4_OK) return st;
  void* ws = nullptr;
  if (hipMallocAsync(&ws, bytes, stream) != hipSuccess) return MXFP4_ERR_HIP;
  st = run_linear(x, packed, scales, sel, p, shared, y, d, dtype, 0, ws, bytes, stream);
  if (hipFreeAsync(ws, stream) != hipSuccess && st == MXFP4_OK) st = MXFP4_ERR_HIP;
  return st;
}

// ---- SwiGLU expert block: two grouped GEMMs over one bucketing.
struct SwDims {
  Dims gu, dn;  // gate/up: (T, E, 2F, G, K); down: (T, E, O, F/32, K)
  int64_t F;
};

int check_swiglu_dims(int64_t T, int64_t E, int64_t F, int64_t G, int64_t O, int64_t K, SwDims* d) {
  if (F < 32 || F % 32 != 0 || F > (int64_t(1) << 29)) return MXFP4_ERR_INVALID_ARG;
  int st = check_dims(T, E, 2 * F, G, K, &d->gu);
  if (st != MXFP4_OK) return st;
  st = check_dims(T, E, O, F / 32, K, &d->dn);
  if (st != MXFP4_OK) return st;
  int64_t t = 0;
  if (!mul_ok(d->gu.P, F, &t) || !mul_ok(t, 2, &t)) return MXFP4_ERR_INVALID_ARG;
  d->F = F;
  return MXFP4_OK;
}

// The down stage's GEMM layout (bucketing arrays, tiles, fp32 part [P, O]),
// then h [P, F] bf16.
struct SwLayout {
  Layout L;
  size_t h, total;
};

SwLayout swiglu_layout(const SwDims& d) {
  SwLayout S;
  S.L = layout(d.dn, MXFP4_PATH_GEMM);
  S.h = S.L.total;
  S.total = align_up(S.h + (size_t)d.dn.P * d.F * 2);
  return S;
}

bool swiglu_supported(const SwDims& d) {
  return gemm_supported(d.gu.T, d.gu.O, d.gu.G) && gemm_supported(d.dn.P, d.dn.O, d.dn.G);
}

int check_swiglu_args(const uint16_t* x, const uint8_t* gu_packed, const uint8_t* gu_scales, const uint8_t* dn_packed,
                      const uint8_t* dn_scales, const int32_t* sel, const float* p, const uint16_t* shared,
                      const uint16_t* y, const SwDims& d) {
  if (d.gu.T == 0) return MXFP4_OK;
  if (!x || !gu_packed || !gu_scales || !dn_packed || !dn_scales || !sel || !p || !shared || !y)
    return MXFP4_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(gu_packed, 16) || !aligned(dn_packed, 16) || !aligned(sel, 4) || !aligned(p, 4) ||
      !aligned(shared, 2) || !aligned(y, 2))
    return MXFP4_ERR_INVALID_ARG;
  const Dims& a = d.gu;
  const Dims& b = d.dn;
  const size_t ny = (size_t)b.T * b.O * 2;
  const size_t sizes[8] = {(size_t)a.T * a.I * 2, (size_t)a.E * a.O * a.G * 16, (size_t)a.E * a.O * a.G,
                           (size_t)b.E * b.O * b.G * 16, (size_t)b.E * b.O * b.G, (size_t)a.P * 4,
                           (size_t)a.P * 4, ny};
  const void* ptrs[8] = {x, gu_packed, gu_scales, dn_packed, dn_scales, sel, p, shared};
  for (int i = 0; i < 8; i++) {
    if (i == 7 && ptrs[i] == y) continue;  // in place on shared is allowed
    if (overlap(y, ny, ptrs[i], sizes[i])) return MXFP4_ERR_INVALID_ARG;
  }
  return MXFP4_OK;
}

// the block-scaled variant: the bucketing and partial rows of the prefill
// layout, then the MXFP8 codes (T, Kp) and scale bytes (T, Kp / 32)
struct MxLayout {
  Layout L;
  int Kp;
  size_t xq, xs, total;
};

MxLayout mx_layout(const Dims& d, bool act_fp4 = false) {
  MxLayout M;
  M.L = layout(d, MXFP4_PATH_GEMM);
  M.Kp = mx_row_bytes(d.I);
  M.xq = M.L.total;
  M.xs = align_up(M.xq + (size_t)d.T * M.Kp / (act_fp4 ? 2 : 1));
  M.total = align_up(M.xs + (size_t)d.T * M.Kp / 32);
  return M;
}

// act_fp4: activations quantised to MXFP4 instead of MXFP8
int run_mx(const uint16_t* x, const uint8_t* packed, const uint8_t* scales, bool prepared, bool act_fp4,
           const int32_t* sel, const float* p, const uint16_t* shared, uint16_t* y, int64_t T, int64_t E, int64_t O,
           int64_t G, int64_t K, uint32_t flags, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  Dims d;
  int st = check_dims(T, E, O, G, K, &d);
  if (st != MXFP4_OK) return st;
  if (flags & ~MXFP4_FLAG_CHECK) return MXFP4_ERR_INVALID_ARG;
  st = check_linear_args(x, packed, scales, sel, p, shared, y, d, MXFP4_DTYPE_BF16);
  if (st != MXFP4_OK) return st;
  if (!gemm_mx_supported(T, O, G)) return MXFP4_ERR_UNSUPPORTED;
  if (d.T == 0) return MXFP4_OK;
  const MxLayout M = mx_layout(d, act_fp4);
  if (workspace_bytes < M.total) return MXFP4_ERR_WORKSPACE_TOO_SMALL;
  if (!workspace || !aligned(workspace, kAlign)) return MXFP4_ERR_INVALID_ARG;
  st = check_device();
  if (st != MXFP4_OK) return st;
  char* base = static_cast<char*>(workspace);
  const Layout& L = M.L;
  BucketOut b;
  b.count = reinterpret_cast<int32_t*>(base + L.count);
  b.offsets = reinterpret_cast<int32_t*>(base + L.offsets);
  b.perm = reinterpret_cast<int32_t*>(base + L.perm);
  b.slot_of_pair = reinterpret_cast<int32_t*>(base + L.slot);
  b.n_invalid = reinterpret_cast<int32_t*>(base + L.n_invalid);
  b.tiles = reinterpret_cast<GemmTile*>(base + L.tiles);
  b.n_tiles = reinterpret_cast<int32_t*>(base + L.n_tiles);
  uint8_t* xq = reinterpret_cast<uint8_t*>(base + M.xq);
  uint8_t* xs = reinterpret_cast<uint8_t*>(base + M.xs);
  float* part = reinterpret_cast<float*>(base + L.part);
  hipError_t err = launch_bucket_multi(sel, (int)d.P, (int)d.E, reinterpret_cast<int32_t*>(base + L.bcount), b, stream);
  if (err == hipSuccess)
    err = act_fp4 ? launch_quant_mxfp4(x, (int)d.T, (int)d.I, M.Kp, xq, xs, stream)
                  : launch_quant_mxfp8(x, (int)d.T, (int)d.I, M.Kp, xq, xs, stream);
  if (err == hipSuccess)
    err = launch_gemm_mx(xq, xs, packed, scales, b.perm, b.tiles, b.n_tiles, gemm_max_tiles(d.P, d.E), part, (int)d.T,
                         (int)d.K, (int)d.O, (int)d.G, stream, prepared, act_fp4);
  if (err == hipSuccess)
    err = launch_combine(part, b.slot_of_pair, p, shared, y, (int)d.T, (int)d.K, (int)d.O, MXFP4_DTYPE_BF16, stream);
  if (err != hipSuccess) return MXFP4_ERR_HIP;
  if (flags & MXFP4_FLAG_CHECK) {
    if (hipStreamSynchronize(stream) != hipSuccess) return MXFP4_ERR_HIP;
    int32_t inv = 0;
    if (hipMemcpy(&inv, b.n_invalid, 4, hipMemcpyDeviceToHost) != hipSuccess) return MXFP4_ERR_HIP;
    if (inv != 0) return MXFP4_ERR_INVALID_INDEX;
  }
  return MXFP4_OK;
}

}  // namespace

extern "C" {

int mxfp4_moe_swiglu_workspace_size(int64_t T, int64_t E, int64_t F, int64_t G, int64_t O, int64_t K,
                                    size_t* bytes) {
  if (!bytes) return MXFP4_ERR_INVALID_ARG;
  SwDims d;
  int st = check_swiglu_dims(T, E, F, G, O, K, &d);
  if (st != MXFP4_OK) return st;
  if (!swiglu_supported(d)) return MXFP4_ERR_UNSUPPORTED;
  *bytes = (T == 0) ? 0 : swiglu_layout(d).total;
  return MXFP4_OK;
}

int mxfp4_moe_swiglu_ex(const uint16_t* x, const uint8_t* gu_packed, const uint8_t* gu_scales,
                        const uint8_t* dn_packed, const uint8_t* dn_scales, const int32_t* sel, const float* p,
                        const uint16_t* shared, uint16_t* y, int64_t T, int64_t E, int64_t F, int64_t G, int64_t O,
                        int64_t K, uint32_t flags, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  SwDims d;
  int st = check_swiglu_dims(T, E, F, G, O, K, &d);
  if (st != MXFP4_OK) return st;
  if (flags & ~MXFP4_FLAG_CHECK) return MXFP4_ERR_INVALID_ARG;
  st = check_swiglu_args(x, gu_packed, gu_scales, dn_packed, dn_scales, sel, p, shared, y, d);
  if (st != MXFP4_OK) return st;
  if (!swiglu_supported(d)) return MXFP4_ERR_UNSUPPORTED;
  if (d.gu.T == 0) return MXFP4_OK;
  const SwLayout S = swiglu_layout(d);
  if (workspace_bytes < S.total) return MXFP4_ERR_WORKSPACE_TOO_SMALL;
  if (!workspace || !aligned(workspace, kAlign)) return MXFP4_ERR_INVALID_ARG;
  st = check_device();
  if (st != MXFP4_OK) return st;
  char* base = static_cast<char*>(workspace);
  const Layout& L = S.L;
  BucketOut b;
  b.count = reinterpret_cast<int32_t*>(base + L.count);
  b.offsets = reinterpret_cast<int32_t*>(base + L.offsets);
  b.perm = reinterpret_cast<int32_t*>(base + L.perm);
  b.slot_of_pair = reinterpret_cast<int32_t*>(base + L.slot);
  b.n_invalid = reinterpret_cast<int32_t*>(base + L.n_invalid);
  b.tiles = reinterpret_cast<GemmTile*>(base + L.tiles);
  b.n_tiles = reinterpret_cast<int32_t*>(base + L.n_tiles);
  uint16_t* h = reinterpret_cast<uint16_t*>(base + S.h);
  float* part = reinterpret_cast<float*>(base + L.part);
  const int64_t max_tiles = gemm_max_tiles(d.gu.P, d.gu.E);
  hipError_t err = launch_bucket_multi(sel, (int)d.gu.P, (int)d.gu.E, reinterpret_cast<int32_t*>(base + L.bcount), b,
                                       stream);
  if (err == hipSuccess)
    err = regdec_canon_ok(d.gu.T, 2 * d.F, d.gu.G) && d.F % 4 == 0
              ? launch_gemm_regdec_canon_swiglu(x, gu_packed, gu_scales, b.perm, b.tiles, b.n_tiles, max_tiles, h,
                                                (int)d.gu.T, (int)d.gu.K, (int)d.F, (int)d.gu.G, stream)
              : launch_gemm_swiglu(x, gu_packed, gu_scales, b.perm, b.tiles, b.n_tiles, max_tiles, h, (int)d.gu.T,
                                   (int)d.gu.K, (int)d.F, (int)d.gu.G, stream);
  if (err == hipSuccess)
    err = regdec_canon_ok(d.dn.P, d.dn.O, d.dn.G)
              ? launch_gemm_regdec_canon_direct(h, dn_packed, dn_scales, b.tiles, b.n_tiles, max_tiles, part, d.dn.P,
                                                (int)d.dn.O, (int)d.dn.G, stream)
              : launch_gemm_direct(h, dn_packed, dn_scales, b.tiles, b.n_tiles, max_tiles, part, d.dn.P,
                                   (int)d.dn.O, (int)d.dn.G, stream);
  if (err == hipSuccess)
    err = launch_combine(part, b.slot_of_pair, p, shared, y, (int)d.dn.T, (int)d.dn.K, (int)d.dn.O, MXFP4_DTYPE_BF16,
                         stream);
  if (err != hipSuccess) return MXFP4_ERR_HIP;
  if (flags & MXFP4_FLAG_CHECK) {
    if (hipStreamSynchronize(stream) != hipSuccess) return MXFP4_ERR_HIP;
    int32_t inv = 0;
    if (hipMemcpy(&inv, b.n_invalid, 4, hipMemcpyDeviceToHost) != hipSuccess) return MXFP4_ERR_HIP;
    if (inv != 0) return MXFP4_ERR_INVALID_INDEX;
  }
  return MXFP4_OK;
}

int mxfp4_prepare_swiglu(const uint8_t* gu_packed, const uint8_t* gu_scales, int64_t E, int64_t F, int64_t G,
                         void* prepared, size_t bytes, hipStream_t stream) {
  if (F < 32 || F % 32 != 0 || F > (int64_t(1) << 29)) return MXFP4_ERR_INVALID_ARG;
  Dims d;
  int st = check_dims(1, E, 2 * F, G, 1, &d);
  if (st != MXFP4_OK) return st;
  if (!gemm_mx_supported(1, 2 * F, G)) return MXFP4_ERR_UNSUPPORTED;
  const size_t need = mx_prepared_bytes(E, 2 * F, G);
  if (bytes < need) return MXFP4_ERR_WORKSPACE_TOO_SMALL;
  if (!gu_packed || !gu_scales || !prepared || !aligned(gu_packed, 16) || !aligned(prepared, 16))
    return MXFP4_ERR_INVALID_ARG;
  if (overlap(prepared, need, gu_packed, (size_t)E * 2 * F * G * 16) ||
      overlap(prepared, need, gu_scales, (size_t)E * 2 * F * G))
    return MXFP4_ERR_INVALID_ARG;
  st = check_device();
  if (st != MXFP4_OK) return st;
  return hip_status(launch_prepare_mx(gu_packed, gu_scales, E, (int)(2 * F), (int)G, static_cast<uint8_t*>(prepared),
                                      stream, (int)F, true));
}

int mxfp4_moe_swiglu_prepared_ex(const uint16_t* x, const void* gu_prepared, const void* dn_prepared,
                                 const int32_t* sel, const float* p, const uint16_t* shared, uint16_t* y, int64_t T,
                                 int64_t E, int64_t F, int64_t G, int64_t O, int64_t K, uint32_t flags,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  SwDims d;
  int st = check_swiglu_dims(T, E, F, G, O, K, &d);
  if (st != MXFP4_OK) return st;
  if (flags & ~MXFP4_FLAG_CHECK) return MXFP4_ERR_INVALID_ARG;
  if (!swiglu_supported(d) || !gemm_mx_supported(d.gu.T, d.gu.O, d.gu.G) ||
      !gemm_regdec_supported(d.gu.T, d.gu.O, d.gu.G) || !gemm_mx_supported(d.dn.P, d.dn.O, d.dn.G) ||
      !gemm_regdec_supported(d.dn.P, d.dn.O, d.dn.G))
    return MXFP4_ERR_UNSUPPORTED;
  const uint8_t* gp = static_cast<const uint8_t*>(gu_prepared);
  const uint8_t* dp = static_cast<const uint8_t*>(dn_prepared);
  const size_t gbytes = mx_prepared_bytes(E, 2 * F, G), dbytes = mx_prepared_bytes(E, O, F / 32);
  st = check_swiglu_args(x, gp, gp ? gp + gbytes / 17 * 16 : nullptr, dp, dp ? dp + dbytes / 17 * 16 : nullptr, sel,
                         p, shared, y, d);
  if (st != MXFP4_OK) return st;
  if (d.gu.T == 0) return MXFP4_OK;
  if (overlap(y, (size_t)T * O * 2, gp, gbytes) || overlap(y, (size_t)T * O * 2, dp, dbytes))
    return MXFP4_ERR_INVALID_ARG;
  const SwLayout S = swiglu_layout(d);
  if (workspace_bytes < S.total) return MXFP4_ERR_WORKSPACE_TOO_SMALL;
  if (!workspace || !aligned(workspace, kAlign)) return MXFP4_ERR_INVALID_ARG;
  st = check_device();
  if (st != MXFP4_OK) return st;
  char* base = static_cast<char*>(workspace);
  const Layout& L = S.L;
  BucketOut b;
  b.count = reinterpret_cast<int32_t*>(base + L.count);
  b.offsets = reinterpret_cast<int32_t*>(base + L.offsets);
  b.perm = reinterpret_cast<int32_t*>(base + L.perm);
  b.slot_of_pair = reinterpret_cast<int32_t*>(base + L.slot);
  b.n_invalid = reinterpret_cast<int32_t*>(base + L.n_invalid);
  b.tiles = reinterpret_cast<GemmTile*>(base + L.tiles);
  b.n_tiles = reinterpret_cast<int32_t*>(base + L.n_tiles);
  uint16_t* h = reinterpret_cast<uint16_t*>(base + S.h);
  float* part = reinterpret_cast<float*>(base + L.part);
  const int64_t max_tiles = gemm_max_tiles(d.gu.P, d.gu.E);
  hipError_t err = launch_bucket_multi(sel, (int)d.gu.P, (int)d.gu.E, reinterpret_cast<int32_t*>(base + L.bcount), b,
                                       stream);
  if (err == hipSuccess)
    err = launch_gemm_regdec_swiglu(x, gp, gp + gbytes / 17 * 16, b.perm, b.tiles, b.n_tiles, max_tiles, h,
                                    (int)d.gu.T, (int)d.gu.K, (int)d.F, (int)d.gu.G, stream);
  if (err == hipSuccess)
    err = launch_gemm_regdec_direct(h, dp, dp + dbytes / 17 * 16, b.tiles, b.n_tiles, max_tiles, part, d.dn.P,
                                    (int)d.dn.O, (int)d.dn.G, stream);
  if (err == hipSuccess)
    err = launch_combine(part, b.slot_of_pair, p, shared, y, (int)d.dn.T, (int)d.dn.K, (int)d.dn.O, MXFP4_DTYPE_BF16,
                         stream);
  if (err != hipSuccess) return MXFP4_ERR_HIP;
  if (flags & MXFP4_FLAG_CHECK) {
    if (hipStreamSynchronize(stream) != hipSuccess) return MXFP4_ERR_HIP;
    int32_t inv = 0;
    if (hipMemcpy(&inv, b.n_invalid, 4, hipMemcpyDeviceToHost) != hipSuccess) return MXFP4_ERR_HIP;
    if (inv != 0) return MXFP4_ERR_INVALID_INDEX;
  }
  return MXFP4_OK;
}

int mxfp4_quantize_mxfp8(const uint16_t* x, int64_t T, int64_t I, int64_t ld, uint8_t* codes, uint8_t* scale_bytes,
                         hipStream_t stream) {
  if (T < 0 || I < 32 || I % 32 || ld < I || ld % 32 || T * ld >= (int64_t(1) << 31)) return MXFP4_ERR_INVALID_ARG;
  if (T == 0) return MXFP4_OK;
  if (!x || !codes || !scale_bytes || !aligned(x, 8) || !aligned(codes, 4)) return MXFP4_ERR_INVALID_ARG;
  const size_t nx = size_t(T) * I * 2, nc = size_t(T) * ld, ns = nc / 32;
  if (overlap(codes, nc, x, nx) || overlap(scale_bytes, ns, x, nx) || overlap(codes, nc, scale_bytes, ns))
    return MXFP4_ERR_INVALID_ARG;
  const int st = check_device();
  if (st != MXFP4_OK) return st;
  return hip_status(launch_quant_mxfp8(x, (int)T, (int)I, (int)ld, codes, scale_bytes, stream));
}

int mxfp4_moe_mxfp8_workspace_size(int64_t T, int64_t E, int64_t O, int64_t G, int64_t K, size_t* bytes) {
  if (!bytes) return MXFP4_ERR_INVALID_ARG;
  Dims d;
  const int st = check_dims(T, E, O, G, K, &d);
  if (st != MXFP4_OK) return st;
  if (!gemm_mx_supported(T, O, G)) return MXFP4_ERR_UNSUPPORTED;
  *bytes = (T == 0) ? 0 : mx_layout(d).total;
  return MXFP4_OK;
}

int mxfp4_moe_linear_mxfp8_ex(const uint16_t* x, const uint8_t* packed, const uint8_t* scales, const int32_t* sel,
                              const float* p, const uint16_t* shared, uint16_t* y, int64_t T, int64_t E, int64_t O,
                              int64_t G, int64_t K, uint32_t flags, void* workspace, size_t workspace_bytes,
                              hipStream_t stream) {
  return run_mx(x, packed, scales, false, false, sel, p, shared, y, T, E, O, G, K, flags, workspace, workspace_bytes,
                stream);
}

int mxfp4_mx_prepared_size(int64_t E, int64_t O, int64_t G, size_t* bytes) {
  if (!bytes) return MXFP4_ERR_INVALID_ARG;
  Dims d;
  const int st = check_dims(1, E, O, G, 1, &d);
  if (st != MXFP4_OK) return st;
  if (!gemm_mx_supported(1, O, G)) return MXFP4_ERR_UNSUPPORTED;
  *bytes = mx_prepared_bytes(E, O, G);
  return MXFP4_OK;
}

namespace {
int prepare(const uint8_t* packed, const uint8_t* scales, int64_t E, int64_t O, int64_t G, void* prepared,
            size_t bytes, hipStream_t stream, bool interleaved) {
  Dims d;
  int st = check_dims(1, E, O, G, 1, &d);
  if (st != MXFP4_OK) return st;
  if (!gemm_mx_supported(1, O, G)) return MXFP4_ERR_UNSUPPORTED;
  const size_t need = mx_prepared_bytes(E, O, G);
  if (bytes < need) return MXFP4_ERR_WORKSPACE_TOO_SMALL;
  if (!packed || !scales || !prepared || !aligned(packed, 16) || !aligned(prepared, 16)) return MXFP4_ERR_INVALID_ARG;
  if (overlap(prepared, need, packed, (size_t)E * O * G * 16) || overlap(prepared, need, scales, (size_t)E * O * G))
    return MXFP4_ERR_INVALID_ARG;
  st = check_device();
  if (st != MXFP4_OK) return st;
  return hip_status(launch_prepare_mx(packed, scales, E, (int)O, (int)G, static_cast<uint8_t*>(prepared), stream, 0,
                                      interleaved));
}
}  // namespace

int mxfp4_prepare_mx(const uint8_t* packed, const uint8_t* scales, int64_t E, int64_t O, int64_t G, void* prepared,
                     size_t bytes, hipStream_t stream) {
  return prepare(packed, scales, E, O, G, prepared, bytes, stream, false);
}

int mxfp4_prepare_bf16(const uint8_t* packed, const uint8_t* scales, int64_t E, int64_t O, int64_t G, void* prepared,
                       size_t bytes, hipStream_t stream) {
  return prepare(packed, scales, E, O, G, prepared, bytes, stream, true);
}

int mxfp4_moe_linear_prepared_ex(const uint16_t* x, const void* prepared, const int32_t* sel, const float* p,
                                  const uint16_t* shared, uint16_t* y, int64_t T, int64_t E, int64_t O, int64_t G,
                                  int64_t K, uint32_t flags, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream) {
  Dims d;
  int st = check_dims(T, E, O, G, K, &d);
  if (st != MXFP4_OK) return st;
  if (flags & ~MXFP4_FLAG_CHECK) return MXFP4_ERR_INVALID_ARG;
  if (!gemm_mx_supported(T, O, G) || !gemm_regdec_supported(T, O, G)) return MXFP4_ERR_UNSUPPORTED;
  const uint8_t* pp = static_cast<const uint8_t*>(prepared);
  const size_t pbytes = mx_prepared_bytes(E, O, G);
  const uint8_t* ps = pp ? pp + pbytes / 17 * 16 : nullptr;
  st = check_linear_args(x, pp, ps, sel, p, shared, y, d, MXFP4_DTYPE_BF16);
  if (st != MXFP4_OK) return st;
  if (d.T == 0) return MXFP4_OK;
  if (overlap(y, (size_t)T * O * 2, pp, pbytes)) return MXFP4_ERR_INVALID_ARG;
  const Layout L = layout(d, MXFP4_PATH_GEMM);
  if (workspace_bytes < L.total) return MXFP4_ERR_WORKSPACE_TOO_SMALL;
  if (!workspace || !aligned(workspace, kAlign)) return MXFP4_ERR_INVALID_ARG;
  st = check_device();
  if (st != MXFP4_OK) return st;
  char* base = static_cast<char*>(workspace);
  BucketOut b;
  b.count = reinterpret_cast<int32_t*>(base + L.count);
  b.offsets = reinterpret_cast<int32_t*>(base + L.offsets);
  b.perm = reinterpret_cast<int32_t*>(base + L.perm);
  b.slot_of_pair = reinterpret_cast<int32_t*>(base + L.slot);
  b.n_invalid = reinterpret_cast<int32_t*>(base + L.n_invalid);
  b.tiles = reinterpret_cast<GemmTile*>(base + L.tiles);
  b.n_tiles = reinterpret_cast<int32_t*>(base + L.n_tiles);
  float* part = reinterpret_cast<float*>(base + L.part);
  hipError_t err = launch_bucket_multi(sel, (int)d.P, (int)d.E, reinterpret_cast<int32_t*>(base + L.bcount), b, stream);
  if (err == hipSuccess)
    err = launch_gemm_regdec(x, pp, ps, b.perm, b.tiles, b.n_tiles, gemm_max_tiles(d.P, d.E), part, (int)d.T, (int)d.K,
                             (int)d.O, (int)d.G, stream);
  if (err == hipSuccess)
    err = launch_combine(part, b.slot_of_pair, p, shared, y, (int)d.T, (int)d.K, (int)d.O, MXFP4_DTYPE_BF16, stream);
  if (err != hipSuccess) return MXFP4_ERR_HIP;
  if (flags & MXFP4_FLAG_CHECK) {
    if (hipStreamSynchronize(stream) != hipSuccess) return MXFP4_ERR_HIP;
    int32_t inv = 0;
    if (hipMemcpy(&inv, b.n_invalid, 4, hipMemcpyDeviceToHost) != hipSuccess) return MXFP4_ERR_HIP;
    if (inv != 0) return MXFP4_ERR_INVALID_INDEX;
  }
  return MXFP4_OK;
}

int mxfp4_moe_gemm_stage_prepared(const uint16_t* x, const void* prepared, int64_t T, int64_t E, int64_t O,
                                  int64_t G, int64_t K, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  Dims d;
  int st = check_dims(T, E, O, G, K, &d);
  if (st != MXFP4_OK) return st;
  if (d.T == 0) return MXFP4_OK;
  if (!x || !prepared) return MXFP4_ERR_INVALID_ARG;
  if (!gemm_mx_supported(T, O, G) || !gemm_regdec_supported(T, O, G)) return MXFP4_ERR_UNSUPPORTED;
  const Layout L = layout(d, MXFP4_PATH_GEMM);
  if (workspace_bytes < L.total) return MXFP4_ERR_WORKSPACE_TOO_SMALL;
  if (!workspace || !aligned(workspace, kAlign)) return MXFP4_ERR_INVALID_ARG;
  st = check_device();
  if (st != MXFP4_OK) return st;
  char* base = static_cast<char*>(workspace);
  const uint8_t* pp = static_cast<const uint8_t*>(prepared);
  const size_t pbytes = mx_prepared_bytes(E, O, G);
  return hip_status(launch_gemm_regdec(x, pp, pp + pbytes / 17 * 16, reinterpret_cast<const int32_t*>(base + L.perm),
                                       reinterpret_cast<const GemmTile*>(base + L.tiles),
                                       reinterpret_cast<const int32_t*>(base + L.n_tiles), gemm_max_tiles(d.P, d.E),
                                       reinterpret_cast<float*>(base + L.part), (int)d.T, (int)d.K, (int)d.O, (int)d.G,
                                       stream));
}

int mxfp4_moe_decode_prepared_ex(const void* x, const void* prepared, const int32_t* sel, const float* p,
                                 const void* shared, void* y, int64_t T, int64_t E, int64_t O, int64_t G, int64_t K,
                                 int dtype, uint32_t flags, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream) {
  Dims d;
  int st = check_dims(T, E, O, G, K, &d);
  if (st != MXFP4_OK) return st;
  if (flags & ~MXFP4_FLAG_CHECK) return MXFP4_ERR_INVALID_ARG;
  if (dtype_size(dtype) == 0) return MXFP4_ERR_INVALID_ARG;
  if (!gemm_mx_supported(1, O, G) || !gemv_rows_supported((int)O, (int)G)) return MXFP4_ERR_UNSUPPORTED;
  const int64_t tc = decode_tokens_per_launch((int)K, (int)E, (int)G, dtype);
  if (tc < 1) return MXFP4_ERR_UNSUPPORTED;
  const uint8_t* pp = static_cast<const uint8_t*>(prepared);
  const size_t pbytes = mx_prepared_bytes(E, O, G);
  const uint8_t* ps = pp ? pp + pbytes / 17 * 16 : nullptr;
  st = check_linear_args(x, pp, ps, sel, p, shared, y, d, dtype);
  if (st != MXFP4_OK) return st;
  if (d.T == 0) return MXFP4_OK;
  const int es = dtype_size(dtype);
  if (overlap(y, (size_t)T * O * es, pp, pbytes)) return MXFP4_ERR_INVALID_ARG;
  const Layout L = layout(d, MXFP4_PATH_GEMV);
  if (workspace_bytes < L.total) return MXFP4_ERR_WORKSPACE_TOO_SMALL;
  if (!workspace || !aligned(workspace, kAlign)) return MXFP4_ERR_INVALID_ARG;
  st = check_device();
  if (st != MXFP4_OK) return st;
  int32_t* n_invalid = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + L.n_invalid);
  hipError_t err = hipSuccess;
  int chunk = 0;
  for (int64_t t0 = 0; t0 < d.T && err == hipSuccess; t0 += tc, chunk++) {
    const int64_t tn = (d.T - t0 < tc) ? d.T - t0 : tc;
    err = launch_decode_prepared(static_cast<const char*>(x) + t0 * d.I * es, pp, ps, sel + t0 * d.K, p + t0 * d.K,
                                 static_cast<const char*>(shared) + t0 * d.O * es, static_cast<char*>(y) + t0 * d.O * es,
                                 (int)tn, (int)d.E, (int)d.O, (int)d.G, (int)d.K, dtype, n_invalid, chunk, stream);
  }
  if (err != hipSuccess) return MXFP4_ERR_HIP;
  if (flags & MXFP4_FLAG_CHECK) {
    if (hipStreamSynchronize(stream) != hipSuccess) return MXFP4_ERR_HIP;
    int32_t inv = 0;
    if (hipMemcpy(&inv, n_invalid, 4, hipMemcpyDeviceToHost) != hipSuccess) return MXFP4_ERR_HIP;
    if (inv != 0) return MXFP4_ERR_INVALID_INDEX;
  }
  return MXFP4_OK;
}

int mxfp4_moe_linear_mxfp8_prepared_ex(const uint16_t* x, const void* prepared, const int32_t* sel, const float* p,
                                       const uint16_t* shared, uint16_t* y, int64_t T, int64_t E, int64_t O,
                                       int64_t G, int64_t K, uint32_t flags, void* workspace, size_t workspace_bytes,
                                       hipStream_t stream) {
  Dims d;
  const int st = check_dims(T, E, O, G, K, &d);
  if (st != MXFP4_OK) return st;
  if (!gemm_mx_supported(T, O, G)) return MXFP4_ERR_UNSUPPORTED;
  const uint8_t* pp = static_cast<const uint8_t*>(prepared);
  const size_t pbytes = mx_prepared_bytes(E, O, G);
  if (T > 0 && pp && y && overlap(y, (size_t)T * O * 2, pp, pbytes)) return MXFP4_ERR_INVALID_ARG;
  return run_mx(x, pp, pp ? pp + pbytes / 17 * 16 : nullptr, true, false, sel, p, shared, y, T, E, O, G, K, flags,
                workspace, workspace_bytes, stream);
}

int mxfp4_quantize_mxfp4(const uint16_t* x, int64_t T, int64_t I, int64_t ld, uint8_t* codes, uint8_t* scale_bytes,
                         hipStream_t stream) {
  if (T < 0 || I < 32 || I % 32 || ld < I || ld % 32 || T * ld >= (int64_t(1) << 31)) return MXFP4_ERR_INVALID_ARG;
  if (T == 0) return MXFP4_OK;
  if (!x || !codes || !scale_bytes || !aligned(x, 8) || !aligned(codes, 4)) return MXFP4_ERR_INVALID_ARG;
  const size_t nx = size_t(T) * I * 2, nc = size_t(T) * ld / 2, ns = size_t(T) * ld / 32;
  if (overlap(codes, nc, x, nx) || overlap(scale_bytes, ns, x, nx) || overlap(codes, nc, scale_bytes, ns))
    return MXFP4_ERR_INVALID_ARG;
  const int st = check_device();
  if (st != MXFP4_OK) return st;
  return hip_status(launch_quant_mxfp4(x, (int)T, (int)I, (int)ld, codes, scale_bytes, stream));
}

int mxfp4_moe_mxfp4act_workspace_size(int64_t T, int64_t E, int64_t O, int64_t G, int64_t K, size_t* bytes) {
  if (!bytes) return MXFP4_ERR_INVALID_ARG;
  Dims d;
  const int st = check_dims(T, E, O, G, K, &d);
  if (st != MXFP4_OK) return st;
  if (!gemm_mx_supported(T, O, G)) return MXFP4_ERR_UNSUPPORTED;
  *bytes = (T == 0) ? 0 : mx_layout(d, true).total;
  return MXFP4_OK;
}

int mxfp4_moe_linear_mxfp4act_ex(const uint16_t* x, const uint8_t* packed, const uint8_t* scales, const int32_t* sel,
                                 const float* p, const uint16_t* shared, uint16_t* y, int64_t T, int64_t E, int64_t O,
                                 int64_t G, int64_t K, uint32_t flags, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream) {
  return run_mx(x, packed, scales, false, true, sel, p, shared, y, T, E, O, G, K, flags, workspace, workspace_bytes,
                stream);
}

int mxfp4_moe_linear_mxfp4act_prepared_ex(const uint16_t* x, const void* prepared, const int32_t* sel,
                                          const float* p, const uint16_t* shared, uint16_t* y, int64_t T, int64_t E,
                                          int64_t O, int64_t G, int64_t K, uint32_t flags, void* workspace,
                                          size_t workspace_bytes, hipStream_t stream) {
  Dims d;
  const int st = check_dims(T, E, O, G, K, &d);
  if (st != MXFP4_OK) return st;
  if (!gemm_mx_supported(T, O, G)) return MXFP4_ERR_UNSUPPORTED;
  const uint8_t* pp = static_cast<const uint8_t*>(prepared);
  const size_t pbytes = mx_prepared_bytes(E, O, G);
  if (T > 0 && pp && y && overlap(y, (size_t)T * O * 2, pp, pbytes)) return MXFP4_ERR_INVALID_ARG;
  return run_mx(x, pp, pp ? pp + pbytes / 17 * 16 : nullptr, true, true, sel, p, shared, y, T, E, O, G, K, flags,
                workspace, workspace_bytes, stream);
}

int mxfp4_moe_route(const float* logits, const float* bias, int64_t T, int64_t E, int64_t K, int mode, float scale,
                    int32_t* sel, float* p, hipStream_t stream) {
  if (T < 0 || T > (int64_t(1) << 30) || E < 1 || E > MXFP4_ROUTE_MAX_EXPERTS || K < 1 || K > E ||
      K > MXFP4_ROUTE_MAX_K)
    return MXFP4_ERR_INVALID_ARG;
  if (mode != MXFP4_ROUTE_SOFTMAX && mode != MXFP4_ROUTE_SIGMOID) return MXFP4_ERR_INVALID_ARG;
  if (mode == MXFP4_ROUTE_SOFTMAX && bias) return MXFP4_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return MXFP4_ERR_INVALID_ARG;
  if (T == 0) return MXFP4_OK;
  if (!logits || !sel || !p) return MXFP4_ERR_INVALID_ARG;
  if (!aligned(logits, 4) || !aligned(sel, 4) || !aligned(p, 4) || (bias && !aligned(bias, 4)))
    return MXFP4_ERR_INVALID_ARG;
  const size_t nl = size_t(T) * size_t(E) * 4, no = size_t(T) * size_t(K) * 4, nb = size_t(E) * 4;
  if (overlap(sel, no, p, no) || overlap(sel, no, logits, nl) || overlap(p, no, logits, nl)) return MXFP4_ERR_INVALID_ARG;
  if (bias && (overlap(sel, no, bias, nb) || overlap(p, no, bias, nb))) return MXFP4_ERR_INVALID_ARG;
  const int st = check_device();
  if (st != MXFP4_OK) return st;
  return hip_status(launch_route(logits, bias, (int)T, (int)E, (int)K, mode, scale, sel, p, stream));
}

int mxfp4_moe_route_grouped(const float* logits, const float* bias, int64_t T, int64_t E, int64_t K, int64_t n_group,
                            int64_t topk_group, int renormalize, float scale, int32_t* sel, float* p,
                            hipStream_t stream) {
  if (T < 0 || T > (int64_t(1) << 30) || E < 2 || E > MXFP4_ROUTE_MAX_EXPERTS || n_group < 1 ||
      n_group > MXFP4_ROUTE_MAX_GROUPS || E % n_group != 0 || E / n_group < 2 || topk_group < 1 ||
      topk_group > n_group || K < 1 || K > MXFP4_ROUTE_MAX_K || K > topk_group * (E / n_group))
    return MXFP4_ERR_INVALID_ARG;
  if (renormalize != 0 && renormalize != 1) return MXFP4_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return MXFP4_ERR_INVALID_ARG;
  if (T == 0) return MXFP4_OK;
  if (!logits || !sel || !p) return MXFP4_ERR_INVALID_ARG;
  if (!aligned(logits, 4) || !aligned(sel, 4) || !aligned(p, 4) || (bias && !aligned(bias, 4)))
    return MXFP4_ERR_INVALID_ARG;
  const size_t nl = size_t(T) * size_t(E) * 4, no = size_t(T) * size_t(K) * 4, nb = size_t(E) * 4;
  if (overlap(sel, no, p, no) || overlap(sel, no, logits, nl) || overlap(p, no, logits, nl)) return MXFP4_ERR_INVALID_ARG;
  if (bias && (overlap(sel, no, bias, nb) || overlap(p, no, bias, nb))) return MXFP4_ERR_INVALID_ARG;
  const int st = check_device();
  if (st != MXFP4_OK) return st;
  return hip_status(launch_route_grouped(logits, bias, (int)T, (int)E, (int)K, (int)n_group, (int)topk_group,
                                         renormalize, scale, sel, p, stream));
}

int mxfp4_moe_linear(const float* x, const uint8_t* packed, const uint8_t* scales, const int32_t* sel, const float* p,
                     const float* shared, float* y, int64_t T, int64_t E, int64_t O, int64_t G, int64_t K,
                     hipStream_t stream) {
  return linear_alloc(x, packed, scales, sel, p, shared, y, T, E, O, G, K, MXFP4_DTYPE_F32, stream);
}

int mxfp4_moe_linear_bf16(const uint16_t* x, const uint8_t* packed, const uint8_t* scales, const int32_t* sel,
                          const float* p, const uint16_t* shared, uint16_t* y, int64_t T, int64_t E, int64_t O,
                          int64_t G, int64_t K, hipStream_t stream) {
  return linear_alloc(x, packed, scales, sel, p, shared, y, T, E, O, G, K, MXFP4_DTYPE_BF16, stream);
}

int mxfp4_moe_workspace_size(int64_t T, int64_t E, int64_t O, int64_t G, int64_t K, int dtype, uint32_t flags,
                             size_t* bytes) {
  if (!bytes) return MXFP4_ERR_INVALID_ARG;
  Dims d;
  int st = check_dims(T, E, O, G, K, &d);
  if (st != MXFP4_OK) return st;
  const int path = select_path(d, dtype, flags);
  if (path < 0) return path;
  *bytes = (T == 0) ? 0 : layout(d, path, dtype).total;
  return MXFP4_OK;
}

int mxfp4_moe_select_path(int64_t T, int64_t E, int64_t O, int64_t G, int64_t K, int dtype, uint32_t flags) {
  Dims d;
  int st = check_dims(T, E, O, G, K, &d);
  if (st != MXFP4_OK) return st;
  return select_path(d, dtype, flags);
}

int mxfp4_moe_linear_ex(const void* x, const uint8_t* packed, const uint8_t* scales, const int32_t* sel, const float* p,
                        const void* shared, void* y, int64_t T, int64_t E, int64_t O, int64_t G, int64_t K, int dtype,
                        uint32_t flags, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  Dims d;
  int st = check_dims(T, E, O, G, K, &d);
  if (st != MXFP4_OK) return st;
  if (flags & ~(MXFP4_FLAG_FORCE_GEMV | MXFP4_FLAG_FORCE_GEMM | MXFP4_FLAG_CHECK | MXFP4_FLAG_GEMV_MFMA))
    return MXFP4_ERR_INVALID_ARG;
  st = check_linear_args(x, packed, scales, sel, p, shared, y, d, dtype);
  if (st != MXFP4_OK) return st;
  const int path = select_path(d, dtype, flags);
  if (path < 0) return path;
  if (d.T == 0) return MXFP4_OK;
  return run_linear(x, packed, scales, sel, p, shared, y, d, dtype, flags, workspace, workspace_bytes, stream);
}

int mxfp4_moe_gemm_stage(const void* x, const uint8_t* packed, const uint8_t* scales, int64_t T, int64_t E, int64_t O,
                         int64_t G, int64_t K, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  Dims d;
  int st = check_dims(T, E, O, G, K, &d);
  if (st != MXFP4_OK) return st;
  if (d.T == 0) return MXFP4_OK;
  if (!x || !packed || !scales) return MXFP4_ERR_INVALID_ARG;
  if (!gemm_supported(d.T, d.O, d.G)) return MXFP4_ERR_UNSUPPORTED;
  const Layout L = layout(d, MXFP4_PATH_GEMM);
  if (workspace_bytes < L.total) return MXFP4_ERR_WORKSPACE_TOO_SMALL;
  if (!workspace || !aligned(workspace, kAlign)) return MXFP4_ERR_INVALID_ARG;
  st = check_device();
  if (st != MXFP4_OK) return st;
  char* base = static_cast<char*>(workspace);
  const hipError_t err = launch_canonical_gemm(
      static_cast<const uint16_t*>(x), packed, scales, reinterpret_cast<const int32_t*>(base + L.perm),
      reinterpret_cast<const GemmTile*>(base + L.tiles), reinterpret_cast<const int32_t*>(base + L.n_tiles),
      gemm_max_tiles(d.P, d.E), reinterpret_cast<float*>(base + L.part), d.T, d.K, d.O, d.G, stream);
  return hip_status(err);
}

int mxfp4_moe_bucket_workspace_size(int64_t T, int64_t K, int64_t E, uint32_t flags, size_t* bytes) {
  if (!bytes || T < 0 || K < 1 || E < 1 || E > MXFP4_MAX_EXPERTS) return MXFP4_ERR_INVALID_ARG;
  if ((flags & MXFP4_FLAG_BUCKET_ONE_BLOCK) && (flags & MXFP4_FLAG_BUCKET_MULTI_BLOCK)) return MXFP4_ERR_INVALID_ARG;
  int64_t P = 0;
  if (!mul_ok(T, K, &P) || P > MXFP4_MAX_PAIRS) return MXFP4_ERR_INVALID_ARG;
  const int64_t nch = bucket_chunks(P);
  *bytes = align_up((size_t)(nch * E + nch) * 4);
  return MXFP4_OK;
}

int mxfp4_moe_bucket(const int32_t* sel, int64_t T, int64_t K, int64_t E, int32_t* count, int32_t* offsets,
                     int32_t* perm, int32_t* slot_of_pair, int32_t* n_invalid, uint32_t flags, void* workspace,
                     size_t workspace_bytes, hipStream_t stream) {
  size_t need = 0;
  int st = mxfp4_moe_bucket_workspace_size(T, K, E, flags, &need);
  if (st != MXFP4_OK) return st;
  if (flags & ~(MXFP4_FLAG_BUCKET_ONE_BLOCK | MXFP4_FLAG_BUCKET_MULTI_BLOCK)) return MXFP4_ERR_INVALID_ARG;
  if (!count || !offsets || !n_invalid) return MXFP4_ERR_INVALID_ARG;
  const int64_t P = T * K;
  if (P > 0 && (!sel || !perm || !slot_of_pair)) return MXFP4_ERR_INVALID_ARG;
  const bool one = (flags & MXFP4_FLAG_BUCKET_ONE_BLOCK) || (!(flags & MXFP4_FLAG_BUCKET_MULTI_BLOCK) && P <= 4096);
  if (!one && (!workspace || workspace_bytes < need || !aligned(workspace, 4))) return MXFP4_ERR_WORKSPACE_TOO_SMALL;
  st = check_device();
  if (st != MXFP4_OK) return st;
  BucketOut b{count, offsets, perm, slot_of_pair, n_invalid, nullptr, nullptr};
  hipError_t err = one ? launch_bucket_one_block(sel, (int)P, (int)E, b, stream)
                       : (P == 0 ? launch_bucket_one_block(sel, 0, (int)E, b, stream)
                                 : launch_bucket_multi(sel, (int)P, (int)E, static_cast<int32_t*>(workspace), b, stream));
  return hip_status(err);
}

int mxfp4_decode_rows(const uint8_t* packed, const uint8_t* scales, int64_t E, int64_t O, int64_t G, int64_t e,
                      int64_t row0, int64_t nrows, int dtype, void* out, hipStream_t stream) {
  Dims d;
  int st = check_dims(0, E, O, G, 1, &d);
  if (st != MXFP4_OK) return st;
  if (dtype_size(dtype) == 0 || e < 0 || e >= E || row0 < 0 || nrows < 0 || row0 + nrows > O)
    return MXFP4_ERR_INVALID_ARG;
  if (nrows == 0) return MXFP4_OK;
  if (!packed || !scales || !out || !aligned(packed, 16) || !aligned(out, 16)) return MXFP4_ERR_INVALID_ARG;
  st = check_device();
  if (st != MXFP4_OK) return st;
  const int64_t row = e * O + row0;
  return hip_status(launch_decode_rows(packed + row * G * 16, scales + row * G, nrows, G, dtype, out, stream));
}

int mxfp4_stream_read(const void* buf, size_t bytes, int blocks, uint32_t* sink, hipStream_t stream) {
  if (bytes == 0) return MXFP4_OK;
  if (!buf || !sink || !aligned(buf, 16) || bytes % 16 != 0 || blocks < 0 || blocks > 65536 ||
      bytes > ((size_t)1 << 40))
    return MXFP4_ERR_INVALID_ARG;
  const int st = check_device();
  if (st != MXFP4_OK) return st;
  return hip_status(launch_stream_read(buf, (int64_t)bytes, blocks, sink, stream));
}

const char* mxfp4_status_string(int status) {
  switch (status) {
    case MXFP4_OK: return "ok";
    case MXFP4_ERR_INVALID_ARG: return "invalid argument";
    case MXFP4_ERR_UNSUPPORTED_DEVICE: return "unsupported device (gfx950 required)";
    case MXFP4_ERR_HIP: return "HIP runtime error";
    case MXFP4_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MXFP4_ERR_INVALID_INDEX: return "selected expert index out of range";
    case MXFP4_ERR_UNSUPPORTED: return "unsupported path for this dtype or shape";
    default: return "unknown status";
  }
}

}  // extern "C"
