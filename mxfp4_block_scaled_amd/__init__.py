"""MXFP4 routed-expert linear on AMD MI355X (gfx950).

    y_t = y_t^shared + sum_k p[t,k] W_{sel[t,k]} x_t

with every W_e stored as packed E2M1 codes [E, O, G, 16] and E8M0 scale
bytes [E, O, G] (page "MXFP4 Routed Expert Linear", Kimi K3). All the work
runs in the HIP kernels of ``libmxfp4_moe.so`` behind the C ABI declared in
include/mxfp4_moe.h; this module only checks tensor arguments, allocates the
output and the workspace with PyTorch, and passes pointers and the current
HIP stream through ctypes. It has no other implementation of any step: when
the library is missing, every call raises.
"""

from __future__ import annotations

import ctypes

import torch

from . import _abi
from ._abi import (  # noqa: F401
    DTYPE_BF16, DTYPE_F32, FLAG_CHECK, FLAG_FORCE_GEMM, FLAG_FORCE_GEMV, FLAG_GEMV_MFMA, FLAG_BUCKET_MULTI_BLOCK,
    FLAG_BUCKET_ONE_BLOCK, PATH_GEMM, PATH_GEMV, ROUTE_SIGMOID, ROUTE_SOFTMAX, Mxfp4Error, bucket_workspace_size,
    mxfp4act_workspace_size, mxfp8_workspace_size, select_path,
    status_string, swiglu_workspace_size, workspace_size,
)

__all__ = [
    "mxfp4_expert_linear", "moe_linear", "moe_swiglu", "decode_rows", "bucket", "gemm_stage", "workspace_size",
    "swiglu_workspace_size", "select_path", "route", "quantize_mxfp8", "moe_linear_mxfp8", "mxfp8_workspace_size",
    "prepare_mx", "PreparedMx", "moe_linear_mxfp8_prepared", "moe_linear_prepared", "gemm_stage_prepared",
    "prepare_bf16", "moe_decode_prepared", "prepare_swiglu", "PreparedSwiGLU", "moe_swiglu_prepared",
    "route_grouped", "stream_read", "quantize_mxfp4", "moe_linear_mxfp4act", "moe_linear_mxfp4act_prepared",
    "mxfp4act_workspace_size", "Mxfp4Error", "library_path",
]

_DTYPES = {torch.float32: DTYPE_F32, torch.bfloat16: DTYPE_BF16}


def library_path() -> str:
    _abi.lib()
    return _abi.LIB_PATH


def _ptr(t: torch.Tensor | None):
    return ctypes.c_void_p(t.data_ptr() if t is not None else 0)


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t: torch.Tensor, name: str, dtype, ndim: int, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def moe_linear(x: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor, sel: torch.Tensor, p: torch.Tensor,
               shared: torch.Tensor, *, out: torch.Tensor | None = None, flags: int = 0,
               workspace: torch.Tensor | None = None) -> torch.Tensor:
    """y = shared + sum_k p[:,k] * W_{sel[:,k]} x on the current HIP stream.

    x [T, 32G] fp32 or bf16; packed [E, O, G, 16] uint8; scales [E, O, G]
    uint8; sel [T, K] int32; p [T, K] fp32; shared [T, O] in x's dtype. All
    on one gfx950 device and contiguous. Returns ``out`` (allocated when not
    given; it may be ``shared`` itself). ``workspace``, when given, is a
    uint8 device tensor of at least ``workspace_size(...)`` bytes.
    """
    if x.dtype not in _DTYPES:
        raise TypeError(f"x must be float32 or bfloat16, got {x.dtype}")
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("x must be on a HIP device")
    dt = _DTYPES[x.dtype]
    _need(x, "x", x.dtype, 2, dev)
    _need(packed, "packed", torch.uint8, 4, dev)
    _need(scales, "scales", torch.uint8, 3, dev)
    _need(sel, "sel", torch.int32, 2, dev)
    _need(p, "p", torch.float32, 2, dev)
    _need(shared, "shared", x.dtype, 2, dev)
    T, I = x.shape
    E, O, G, B = packed.shape
    K = sel.shape[1]
    if B != 16 or I != 32 * G:
        raise ValueError(f"packed must be [E, O, G, 16] with 32G == x.shape[1]; got {tuple(packed.shape)}, I={I}")
    if tuple(scales.shape) != (E, O, G):
        raise ValueError("scales must have the packed shape without its last axis")
    if tuple(sel.shape) != (T, K) or tuple(p.shape) != (T, K) or tuple(shared.shape) != (T, O):
        raise ValueError("sel and p must be [T, K] and shared [T, O]")
    y = torch.empty_like(shared) if out is None else out
    _need(y, "out", x.dtype, 2, dev)
    if tuple(y.shape) != (T, O):
        raise ValueError("out must be [T, O]")
    need = workspace_size(T, E, O, G, K, dt, flags)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    elif workspace.dtype != torch.uint8 or workspace.device != dev:
        raise ValueError("workspace must be a uint8 tensor on x's device")
    with torch.cuda.device(dev):
        st = _abi.lib().mxfp4_moe_linear_ex(
            _ptr(x), _ptr(packed), _ptr(scales), _ptr(sel), _ptr(p), _ptr(shared), _ptr(y),
            T, E, O, G, K, dt, flags, _ptr(workspace), workspace.numel(), _stream(dev))
    _abi.check(st, "mxfp4_moe_linear_ex")
    return y


def moe_swiglu(x: torch.Tensor, gu_packed: torch.Tensor, gu_scales: torch.Tensor, dn_packed: torch.Tensor,
               dn_scales: torch.Tensor, sel: torch.Tensor, p: torch.Tensor, shared: torch.Tensor, *,
               out: torch.Tensor | None = None, flags: int = 0,
               workspace: torch.Tensor | None = None) -> torch.Tensor:
    """The routed SwiGLU expert block on the current HIP stream (bf16):
    y = shared + sum_k p[:,k] * Down_e(silu(Gate_e x) * Up_e x), e = sel[:,k].

    x [T, 32G] bf16; gu_packed [E, 2F, G, 16] / gu_scales [E, 2F, G] uint8
    (gate rows first, then up); dn_packed [E, O, F/32, 16] / dn_scales
    [E, O, F/32] uint8; sel [T, K] int32; p [T, K] fp32; shared [T, O] bf16.
    Returns ``out`` (allocated when not given; it may be ``shared``).
    """
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("x must be on a HIP device")
    _need(x, "x", torch.bfloat16, 2, dev)
    _need(gu_packed, "gu_packed", torch.uint8, 4, dev)
    _need(gu_scales, "gu_scales", torch.uint8, 3, dev)
    _need(dn_packed, "dn_packed", torch.uint8, 4, dev)
    _need(dn_scales, "dn_scales", torch.uint8, 3, dev)
    _need(sel, "sel", torch.int32, 2, dev)
    _need(p, "p", torch.float32, 2, dev)
    _need(shared, "shared", torch.bfloat16, 2, dev)
    T, I = x.shape
    E, F2, G, B = gu_packed.shape
    K = sel.shape[1]
    O = dn_packed.shape[1]
    if B != 16 or I != 32 * G or F2 % 2 != 0:
        raise ValueError(f"gu_packed must be [E, 2F, G, 16] with 32G == x.shape[1]; got {tuple(gu_packed.shape)}")
    F = F2 // 2
    if tuple(gu_scales.shape) != (E, F2, G):
        raise ValueError("gu_scales must have gu_packed's shape without its last axis")
    if F % 32 != 0 or tuple(dn_packed.shape) != (E, O, F // 32, 16) or tuple(dn_scales.shape) != (E, O, F // 32):
        raise ValueError(f"dn_packed must be [E, O, F/32, 16] with F = {F} a multiple of 32, dn_scales [E, O, F/32]")
    if tuple(sel.shape) != (T, K) or tuple(p.shape) != (T, K) or tuple(shared.shape) != (T, O):
        raise ValueError("sel and p must be [T, K] and shared [T, O]")
    y = torch.empty_like(shared) if out is None else out
    _need(y, "out", torch.bfloat16, 2, dev)
    if tuple(y.shape) != (T, O):
        raise ValueError("out must be [T, O]")
    need = _abi.swiglu_workspace_size(T, E, F, G, O, K)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    elif workspace.dtype != torch.uint8 or workspace.device != dev:
        raise ValueError("workspace must be a uint8 tensor on x's device")
    with torch.cuda.device(dev):
        st = _abi.lib().mxfp4_moe_swiglu_ex(
            _ptr(x), _ptr(gu_packed), _ptr(gu_scales), _ptr(dn_packed), _ptr(dn_scales), _ptr(sel), _ptr(p),
            _ptr(shared), _ptr(y), T, E, F, G, O, K, flags, _ptr(workspace), workspace.numel(), _stream(dev))
    _abi.check(st, "mxfp4_moe_swiglu_ex")
    return y


def quantize_mxfp8(x: torch.Tensor, ld: int | None = None) -> tuple[torch.Tensor, torch.Tensor]:
    """bf16 activations [T, I] -> (E4M3 codes uint8 [T, ld], E8M0 scale
    bytes uint8 [T, ld/32]), one scale per token and block of 32 inputs;
    columns past I hold zeros. ld defaults to I."""
    dev = x.device
    _need(x, "x", torch.bfloat16, 2, dev)
    T, I = x.shape
    ld = I if ld is None else ld
    codes = torch.empty((T, ld), dtype=torch.uint8, device=dev)
    sb = torch.empty((T, ld // 32), dtype=torch.uint8, device=dev)
    with torch.cuda.device(dev):
        st = _abi.lib().mxfp4_quantize_mxfp8(_ptr(x), T, I, ld, _ptr(codes), _ptr(sb), _stream(dev))
    _abi.check(st, "mxfp4_quantize_mxfp8")
    return codes, sb


def quantize_mxfp4(x: torch.Tensor, ld: int | None = None) -> tuple[torch.Tensor, torch.Tensor]:
    """bf16 activations [T, I] -> (E2M1 codes uint8 [T, ld/2], two per byte
    with the first in the low nibble, and E8M0 scale bytes uint8 [T, ld/32]),
    one scale per token and block of 32 inputs; columns past I hold zeros.
    ld defaults to I."""
    dev = x.device
    _need(x, "x", torch.bfloat16, 2, dev)
    T, I = x.shape
    ld = I if ld is None else ld
    codes = torch.empty((T, ld // 2), dtype=torch.uint8, device=dev)
    sb = torch.empty((T, ld // 32), dtype=torch.uint8, device=dev)
    with torch.cuda.device(dev):
        st = _abi.lib().mxfp4_quantize_mxfp4(_ptr(x), T, I, ld, _ptr(codes), _ptr(sb), _stream(dev))
    _abi.check(st, "mxfp4_quantize_mxfp4")
    return codes, sb


def moe_linear_mxfp8(x: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor, sel: torch.Tensor,
                     p: torch.Tensor, shared: torch.Tensor, *, out: torch.Tensor | None = None, flags: int = 0,
                     workspace: torch.Tensor | None = None) -> torch.Tensor:
    """The block-scaled variant of ``moe_linear`` (bf16 only): activations
    quantised to MXFP8, multiplied by the packed weights as stored on the
    block-scaled MFMA. An approximation of ``moe_linear`` (activation
    rounding), reported separately. Shapes as ``moe_linear``."""
    return _moe_linear_mx(x, packed, scales, sel, p, shared, out, flags, workspace, False)


def moe_linear_mxfp4act(x: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor, sel: torch.Tensor,
                        p: torch.Tensor, shared: torch.Tensor, *, out: torch.Tensor | None = None, flags: int = 0,
                        workspace: torch.Tensor | None = None) -> torch.Tensor:
    """``moe_linear_mxfp8`` with the activations quantised to MXFP4 instead
    (both operands of the scaled MFMA in E2M1). Reported separately."""
    return _moe_linear_mx(x, packed, scales, sel, p, shared, out, flags, workspace, True)


def _moe_linear_mx(x, packed, scales, sel, p, shared, out, flags, workspace, act_fp4):
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("x must be on a HIP device")
    _need(x, "x", torch.bfloat16, 2, dev)
    _need(packed, "packed", torch.uint8, 4, dev)
    _need(scales, "scales", torch.uint8, 3, dev)
    _need(sel, "sel", torch.int32, 2, dev)
    _need(p, "p", torch.float32, 2, dev)
    _need(shared, "shared", torch.bfloat16, 2, dev)
    T, I = x.shape
    E, O, G, B = packed.shape
    K = sel.shape[1]
    if B != 16 or I != 32 * G or tuple(scales.shape) != (E, O, G):
        raise ValueError(f"packed must be [E, O, G, 16] with 32G == x.shape[1] and scales [E, O, G]")
    if tuple(sel.shape) != (T, K) or tuple(p.shape) != (T, K) or tuple(shared.shape) != (T, O):
        raise ValueError("sel and p must be [T, K] and shared [T, O]")
    y = torch.empty_like(shared) if out is None else out
    _need(y, "out", torch.bfloat16, 2, dev)
    if tuple(y.shape) != (T, O):
        raise ValueError("out must be [T, O]")
    need = (_abi.mxfp4act_workspace_size if act_fp4 else _abi.mxfp8_workspace_size)(T, E, O, G, K)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    elif workspace.dtype != torch.uint8 or workspace.device != dev:
        raise ValueError("workspace must be a uint8 tensor on x's device")
    name = "mxfp4_moe_linear_mxfp4act_ex" if act_fp4 else "mxfp4_moe_linear_mxfp8_ex"
    with torch.cuda.device(dev):
        st = getattr(_abi.lib(), name)(
            _ptr(x), _ptr(packed), _ptr(scales), _ptr(sel), _ptr(p), _ptr(shared), _ptr(y), T, E, O, G, K, flags,
            _ptr(workspace), workspace.numel(), _stream(dev))
    _abi.check(st, name)
    return y


class PreparedMx:
    """Weights repacked by ``prepare_mx`` (read by the block-scaled variant
    and by the bf16 prepared path): a uint8 device buffer and the (E, O, G)
    it was made from."""

    def __init__(self, buf: torch.Tensor, E: int, O: int, G: int, interleaved: bool = False):
        self.buf, self.E, self.O, self.G, self.interleaved = buf, E, O, G, interleaved


def prepare_mx(packed: torch.Tensor, scales: torch.Tensor, *, interleaved: bool = False) -> PreparedMx:
    """Load-time repack of [E, O, G, 16] codes and [E, O, G] scale bytes into
    the fragment-major layout the block-scaled variant streams (a byte
    permutation plus zero padding); ``interleaved``: the dword-interleaved
    code order of ``prepare_bf16``."""
    dev = packed.device
    _need(packed, "packed", torch.uint8, 4, dev)
    _need(scales, "scales", torch.uint8, 3, dev)
    E, O, G, B = packed.shape
    if B != 16 or tuple(scales.shape) != (E, O, G):
        raise ValueError("packed must be [E, O, G, 16] and scales [E, O, G]")
    n = _abi.mx_prepared_size(E, O, G)
    buf = torch.empty(n, dtype=torch.uint8, device=dev)
    with torch.cuda.device(dev):
        fn = _abi.lib().mxfp4_prepare_bf16 if interleaved else _abi.lib().mxfp4_prepare_mx
        st = fn(_ptr(packed), _ptr(scales), E, O, G, _ptr(buf), n, _stream(dev))
    _abi.check(st, "mxfp4_prepare_bf16" if interleaved else "mxfp4_prepare_mx")
    return PreparedMx(buf, E, O, G, interleaved)


def prepare_bf16(packed: torch.Tensor, scales: torch.Tensor) -> PreparedMx:
    """Load-time repack for the bf16 prepared paths (``moe_linear_prepared``,
    the SwiGLU block's down projection): ``prepare_mx``'s slots with the code
    blocks in dword-interleaved order."""
    return prepare_mx(packed, scales, interleaved=True)


def moe_linear_mxfp8_prepared(x: torch.Tensor, prepared: PreparedMx, sel: torch.Tensor, p: torch.Tensor,
                              shared: torch.Tensor, *, out: torch.Tensor | None = None, flags: int = 0,
                              workspace: torch.Tensor | None = None) -> torch.Tensor:
    """``moe_linear_mxfp8`` on weights repacked by ``prepare_mx`` (the same
    result bit for bit)."""
    return _moe_linear_mx_prepared(x, prepared, sel, p, shared, out, flags, workspace, False)


def moe_linear_mxfp4act_prepared(x: torch.Tensor, prepared: PreparedMx, sel: torch.Tensor, p: torch.Tensor,
                                 shared: torch.Tensor, *, out: torch.Tensor | None = None, flags: int = 0,
                                 workspace: torch.Tensor | None = None) -> torch.Tensor:
    """``moe_linear_mxfp4act`` on weights repacked by ``prepare_mx`` (the same
    result bit for bit)."""
    return _moe_linear_mx_prepared(x, prepared, sel, p, shared, out, flags, workspace, True)


def _moe_linear_mx_prepared(x, prepared, sel, p, shared, out, flags, workspace, act_fp4):
    dev = x.device
    _need(x, "x", torch.bfloat16, 2, dev)
    _need(sel, "sel", torch.int32, 2, dev)
    _need(p, "p", torch.float32, 2, dev)
    _need(shared, "shared", torch.bfloat16, 2, dev)
    if not isinstance(prepared, PreparedMx) or prepared.buf.device != dev or prepared.interleaved:
        raise ValueError("prepared must come from prepare_mx on x's device")
    T, I = x.shape
    E, O, G = prepared.E, prepared.O, prepared.G
    K = sel.shape[1]
    if I != 32 * G:
        raise ValueError(f"x has {I} inputs; the prepared weights have 32 * {G}")
    if tuple(sel.shape) != (T, K) or tuple(p.shape) != (T, K) or tuple(shared.shape) != (T, O):
        raise ValueError("sel and p must be [T, K] and shared [T, O]")
    y = torch.empty_like(shared) if out is None else out
    _need(y, "out", torch.bfloat16, 2, dev)
    if tuple(y.shape) != (T, O):
        raise ValueError("out must be [T, O]")
    need = (_abi.mxfp4act_workspace_size if act_fp4 else _abi.mxfp8_workspace_size)(T, E, O, G, K)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    name = "mxfp4_moe_linear_mxfp4act_prepared_ex" if act_fp4 else "mxfp4_moe_linear_mxfp8_prepared_ex"
    with torch.cuda.device(dev):
        st = getattr(_abi.lib(), name)(
            _ptr(x), _ptr(prepared.buf), _ptr(sel), _ptr(p), _ptr(shared), _ptr(y), T, E, O, G, K, flags,
            _ptr(workspace), workspace.numel(), _stream(dev))
    _abi.check(st, name)
    return y


def _prepared_call_args(x, prepared, sel, p, shared, out):
    dev = x.device
    _need(x, "x", torch.bfloat16, 2, dev)
    _need(sel, "sel", torch.int32, 2, dev)
    _need(p, "p", torch.float32, 2, dev)
    _need(shared, "shared", torch.bfloat16, 2, dev)
    if not isinstance(prepared, PreparedMx) or prepared.buf.device != dev or not prepared.interleaved:
        raise ValueError("prepared must come from prepare_bf16 on x's device")
    T, I = x.shape
    E, O, G = prepared.E, prepared.O, prepared.G
    K = sel.shape[1]
    if I != 32 * G:
        raise ValueError(f"x has {I} inputs; the prepared weights have 32 * {G}")
    if tuple(sel.shape) != (T, K) or tuple(p.shape) != (T, K) or tuple(shared.shape) != (T, O):
        raise ValueError("sel and p must be [T, K] and shared [T, O]")
    y = torch.empty_like(shared) if out is None else out
    _need(y, "out", torch.bfloat16, 2, dev)
    if tuple(y.shape) != (T, O):
        raise ValueError("out must be [T, O]")
    return dev, T, E, O, G, K, y


def moe_linear_prepared(x: torch.Tensor, prepared: PreparedMx, sel: torch.Tensor, p: torch.Tensor,
                        shared: torch.Tensor, *, out: torch.Tensor | None = None, flags: int = 0,
                        workspace: torch.Tensor | None = None) -> torch.Tensor:
    """The bf16 routed linear (prefill-shaped path) on weights repacked by
    ``prepare_bf16``: bucketing, the register-decode grouped GEMM, combine."""
    dev, T, E, O, G, K, y = _prepared_call_args(x, prepared, sel, p, shared, out)
    need = workspace_size(T, E, O, G, K, DTYPE_BF16, FLAG_FORCE_GEMM)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    with torch.cuda.device(dev):
        st = _abi.lib().mxfp4_moe_linear_prepared_ex(
            _ptr(x), _ptr(prepared.buf), _ptr(sel), _ptr(p), _ptr(shared), _ptr(y), T, E, O, G, K, flags,
            _ptr(workspace), workspace.numel(), _stream(dev))
    _abi.check(st, "mxfp4_moe_linear_prepared_ex")
    return y


def gemm_stage_prepared(x: torch.Tensor, prepared: PreparedMx, K: int, workspace: torch.Tensor) -> None:
    """Re-run only the grouped GEMM of ``moe_linear_prepared`` on the bucketing
    its last call with this workspace (same sizes) left there. For timing."""
    dev = x.device
    _need(x, "x", torch.bfloat16, 2, dev)
    T = x.shape[0]
    with torch.cuda.device(dev):
        st = _abi.lib().mxfp4_moe_gemm_stage_prepared(_ptr(x), _ptr(prepared.buf), T, prepared.E, prepared.O,
                                                      prepared.G, K, _ptr(workspace), workspace.numel(),
                                                      _stream(dev))
    _abi.check(st, "mxfp4_moe_gemm_stage_prepared")


class PreparedSwiGLU:
    """SwiGLU expert weights repacked once (``prepare_swiglu``): the gate/up
    buffer, the down buffer and the (E, F, G, O) they were made from."""

    def __init__(self, gu: torch.Tensor, dn: PreparedMx, E: int, F: int, G: int, O: int):
        self.gu, self.dn, self.E, self.F, self.G, self.O = gu, dn, E, F, G, O


def prepare_swiglu(gu_packed: torch.Tensor, gu_scales: torch.Tensor, dn_packed: torch.Tensor,
                   dn_scales: torch.Tensor) -> PreparedSwiGLU:
    """Load-time repack of a SwiGLU block's weights: gate/up [E, 2F, G, 16]
    (gate rows first) in the row order that puts 64 features' gate and up
    rows in one tile, and the down projection [E, O, F/32, 16] as
    ``prepare_mx``. A byte permutation plus zero padding."""
    dev = gu_packed.device
    _need(gu_packed, "gu_packed", torch.uint8, 4, dev)
    _need(gu_scales, "gu_scales", torch.uint8, 3, dev)
    E, F2, G, B = gu_packed.shape
    if B != 16 or F2 % 64 != 0 or tuple(gu_scales.shape) != (E, F2, G):
        raise ValueError("gu_packed must be [E, 2F, G, 16] with F a multiple of 32, gu_scales [E, 2F, G]")
    F = F2 // 2
    dn = prepare_bf16(dn_packed, dn_scales)
    if dn.E != E or dn.G != F // 32:
        raise ValueError("dn_packed must be [E, O, F/32, 16]")
    n = _abi.mx_prepared_size(E, F2, G)
    gu = torch.empty(n, dtype=torch.uint8, device=dev)
    with torch.cuda.device(dev):
        st = _abi.lib().mxfp4_prepare_swiglu(_ptr(gu_packed), _ptr(gu_scales), E, F, G, _ptr(gu), n, _stream(dev))
    _abi.check(st, "mxfp4_prepare_swiglu")
    return PreparedSwiGLU(gu, dn, E, F, G, dn.O)


def moe_swiglu_prepared(x: torch.Tensor, prepared: PreparedSwiGLU, sel: torch.Tensor, p: torch.Tensor,
                        shared: torch.Tensor, *, out: torch.Tensor | None = None, flags: int = 0,
                        workspace: torch.Tensor | None = None) -> torch.Tensor:
    """``moe_swiglu`` on weights repacked by ``prepare_swiglu`` (both GEMMs on
    the register-decode kernel)."""
    dev = x.device
    _need(x, "x", torch.bfloat16, 2, dev)
    _need(sel, "sel", torch.int32, 2, dev)
    _need(p, "p", torch.float32, 2, dev)
    _need(shared, "shared", torch.bfloat16, 2, dev)
    if not isinstance(prepared, PreparedSwiGLU) or prepared.gu.device != dev:
        raise ValueError("prepared must come from prepare_swiglu on x's device")
    T, I = x.shape
    E, F, G, O = prepared.E, prepared.F, prepared.G, prepared.O
    K = sel.shape[1]
    if I != 32 * G:
        raise ValueError(f"x has {I} inputs; the prepared weights have 32 * {G}")
    if tuple(sel.shape) != (T, K) or tuple(p.shape) != (T, K) or tuple(shared.shape) != (T, O):
        raise ValueError("sel and p must be [T, K] and shared [T, O]")
    y = torch.empty_like(shared) if out is None else out
    _need(y, "out", torch.bfloat16, 2, dev)
    if tuple(y.shape) != (T, O):
        raise ValueError("out must be [T, O]")
    need = _abi.swiglu_workspace_size(T, E, F, G, O, K)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    with torch.cuda.device(dev):
        st = _abi.lib().mxfp4_moe_swiglu_prepared_ex(
            _ptr(x), _ptr(prepared.gu), _ptr(prepared.dn.buf), _ptr(sel), _ptr(p), _ptr(shared), _ptr(y), T, E, F, G,
            O, K, flags, _ptr(workspace), workspace.numel(), _stream(dev))
    _abi.check(st, "mxfp4_moe_swiglu_prepared_ex")
    return y


def moe_decode_prepared(x: torch.Tensor, prepared: PreparedMx, sel: torch.Tensor, p: torch.Tensor,
                        shared: torch.Tensor, *, out: torch.Tensor | None = None, flags: int = 0,
                        workspace: torch.Tensor | None = None) -> torch.Tensor:
    """The decode-shaped path (fp32 or bf16 x) on weights repacked by
    ``prepare_mx``: routing, the MFMA dequant-GEMV and the combine in one
    launch per token chunk."""
    dev = x.device
    if x.dtype not in _DTYPES:
        raise ValueError("x must be float32 or bfloat16")
    td = x.dtype
    _need(x, "x", td, 2, dev)
    _need(sel, "sel", torch.int32, 2, dev)
    _need(p, "p", torch.float32, 2, dev)
    _need(shared, "shared", td, 2, dev)
    if not isinstance(prepared, PreparedMx) or prepared.buf.device != dev or prepared.interleaved:
        raise ValueError("prepared must come from prepare_mx on x's device")
    T, I = x.shape
    E, O, G = prepared.E, prepared.O, prepared.G
    K = sel.shape[1]
    if I != 32 * G:
        raise ValueError(f"x has {I} inputs; the prepared weights have 32 * {G}")
    if tuple(sel.shape) != (T, K) or tuple(p.shape) != (T, K) or tuple(shared.shape) != (T, O):
        raise ValueError("sel and p must be [T, K] and shared [T, O]")
    y = torch.empty_like(shared) if out is None else out
    _need(y, "out", td, 2, dev)
    if tuple(y.shape) != (T, O):
        raise ValueError("out must be [T, O]")
    dt = _DTYPES[td]
    need = workspace_size(T, E, O, G, K, dt, FLAG_FORCE_GEMV)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    with torch.cuda.device(dev):
        st = _abi.lib().mxfp4_moe_decode_prepared_ex(
            _ptr(x), _ptr(prepared.buf), _ptr(sel), _ptr(p), _ptr(shared), _ptr(y), T, E, O, G, K, dt, flags,
            _ptr(workspace), workspace.numel(), _stream(dev))
    _abi.check(st, "mxfp4_moe_decode_prepared_ex")
    return y


def mxfp4_expert_linear(latent_tokens: torch.Tensor, packed_weights: torch.Tensor, scale_bytes: torch.Tensor,
                        selected_experts: torch.Tensor, mixture_weights: torch.Tensor,
                        shared_output: torch.Tensor) -> torch.Tensor:
    """The problem page's signature ("Starter Code"): returns a new tensor
    shaped like ``shared_output`` in the latent tokens' dtype and device.

    Marshalling only: the expert indices are passed as int32 and the mixture
    weights as fp32 (copies when they arrive in another integer or float
    type); nothing supplied is modified.
    """
    if shared_output.dtype != latent_tokens.dtype:
        raise TypeError("shared_output must have the latent tokens' dtype")
    sel = selected_experts.to(device=latent_tokens.device, dtype=torch.int32).contiguous()
    p = mixture_weights.to(device=latent_tokens.device, dtype=torch.float32).contiguous()
    return moe_linear(latent_tokens.contiguous(), packed_weights.contiguous(), scale_bytes.contiguous(), sel, p,
                      shared_output.contiguous())


def decode_rows(packed: torch.Tensor, scales: torch.Tensor, e: int, row0: int, nrows: int,
                dtype: torch.dtype = torch.float32) -> torch.Tensor:
    """Rows row0 .. row0+nrows-1 of expert e decoded to [nrows, 32G] (exact)."""
    dev = packed.device
    _need(packed, "packed", torch.uint8, 4, dev)
    _need(scales, "scales", torch.uint8, 3, dev)
    E, O, G, _ = packed.shape
    out = torch.empty((nrows, 32 * G), dtype=dtype, device=dev)
    with torch.cuda.device(dev):
        st = _abi.lib().mxfp4_decode_rows(_ptr(packed), _ptr(scales), E, O, G, e, row0, nrows, _DTYPES[dtype],
                                          _ptr(out), _stream(dev))
    _abi.check(st, "mxfp4_decode_rows")
    return out


def gemm_stage(x: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor, K: int,
               workspace: torch.Tensor) -> None:
    """Re-run only the grouped GEMM of the prefill-shaped path on the
    bucketing that the last ``moe_linear`` call with this workspace (bf16,
    same sizes, prefill-shaped path) left there. For timing."""
    dev = x.device
    _need(x, "x", torch.bfloat16, 2, dev)
    _need(packed, "packed", torch.uint8, 4, dev)
    _need(scales, "scales", torch.uint8, 3, dev)
    T = x.shape[0]
    E, O, G, _ = packed.shape
    with torch.cuda.device(dev):
        st = _abi.lib().mxfp4_moe_gemm_stage(_ptr(x), _ptr(packed), _ptr(scales), T, E, O, G, K, _ptr(workspace),
                                             workspace.numel(), _stream(dev))
    _abi.check(st, "mxfp4_moe_gemm_stage")


def stream_read(buf: torch.Tensor, sink: torch.Tensor, blocks: int = 0) -> None:
    """Read every byte of the device tensor ``buf`` once with the plain
    streaming-read kernel (a measurement helper, not a step of the layer);
    ``sink`` is an int32/uint32 device tensor of at least ``blocks`` (or 2048)
    elements that is practically never written."""
    dev = buf.device
    if not buf.is_contiguous() or sink.device != dev or sink.element_size() != 4:
        raise ValueError("buf must be contiguous and sink a 4-byte tensor on the same device")
    nbytes = buf.numel() * buf.element_size()
    if sink.numel() < (blocks or 2048):
        raise ValueError("sink too small")
    with torch.cuda.device(dev):
        st = _abi.lib().mxfp4_stream_read(_ptr(buf), nbytes, blocks, _ptr(sink), _stream(dev))
    _abi.check(st, "mxfp4_stream_read")


def route(logits: torch.Tensor, K: int, mode: str = "softmax", bias: torch.Tensor | None = None,
          scale: float = 1.0, *, sel: torch.Tensor | None = None,
          p: torch.Tensor | None = None) -> tuple[torch.Tensor, torch.Tensor]:
    """Router: fp32 logits (T, E) -> (sel int32 (T, K), p fp32 (T, K)).
    mode "softmax" (bias must be None) or "sigmoid" (bias (E,) fp32 steers
    the choice only)."""
    modes = {"softmax": ROUTE_SOFTMAX, "sigmoid": ROUTE_SIGMOID}
    if mode not in modes:
        raise ValueError(f"mode must be one of {sorted(modes)}, got {mode!r}")
    dev = logits.device
    _need(logits, "logits", torch.float32, 2, dev)
    if bias is not None:
        _need(bias, "bias", torch.float32, 1, dev)
        if bias.shape[0] != logits.shape[1]:
            raise ValueError(f"bias has {bias.shape[0]} entries, logits have {logits.shape[1]} experts")
    T = logits.shape[0]
    if sel is None:
        sel = torch.empty((T, K), dtype=torch.int32, device=dev)
    if p is None:
        p = torch.empty((T, K), dtype=torch.float32, device=dev)
    _need(sel, "sel", torch.int32, 2, dev)
    _need(p, "p", torch.float32, 2, dev)
    if tuple(sel.shape) != (T, K) or tuple(p.shape) != (T, K):
        raise ValueError(f"sel and p must be ({T}, {K})")
    with torch.cuda.device(dev):
        st = _abi.lib().mxfp4_moe_route(_ptr(logits), _ptr(bias), T, logits.shape[1], K, modes[mode],
                                        float(scale), _ptr(sel), _ptr(p), _stream(dev))
    _abi.check(st, "mxfp4_moe_route")
    return sel, p


def route_grouped(logits: torch.Tensor, K: int, n_group: int, topk_group: int, bias: torch.Tensor | None = None,
                  scale: float = 1.0, renormalize: bool = True, *, sel: torch.Tensor | None = None,
                  p: torch.Tensor | None = None) -> tuple[torch.Tensor, torch.Tensor]:
    """Group-limited sigmoid router (mxfp4_moe_route_grouped): fp32 logits
    (T, E) -> (sel int32 (T, K), p fp32 (T, K)); bias (E,) fp32 or None."""
    dev = logits.device
    _need(logits, "logits", torch.float32, 2, dev)
    if bias is not None:
        _need(bias, "bias", torch.float32, 1, dev)
        if bias.shape[0] != logits.shape[1]:
            raise ValueError(f"bias has {bias.shape[0]} entries, logits have {logits.shape[1]} experts")
    T = logits.shape[0]
    if sel is None:
        sel = torch.empty((T, K), dtype=torch.int32, device=dev)
    if p is None:
        p = torch.empty((T, K), dtype=torch.float32, device=dev)
    _need(sel, "sel", torch.int32, 2, dev)
    _need(p, "p", torch.float32, 2, dev)
    if tuple(sel.shape) != (T, K) or tuple(p.shape) != (T, K):
        raise ValueError(f"sel and p must be ({T}, {K})")
    with torch.cuda.device(dev):
        st = _abi.lib().mxfp4_moe_route_grouped(_ptr(logits), _ptr(bias), T, logits.shape[1], K, n_group, topk_group,
                                                int(bool(renormalize)), float(scale), _ptr(sel), _ptr(p),
                                                _stream(dev))
    _abi.check(st, "mxfp4_moe_route_grouped")
    return sel, p


def bucket(sel: torch.Tensor, E: int, flags: int = 0) -> dict:
    """Stable counting sort of the (token, slot) pairs by expert."""
    dev = sel.device
    _need(sel, "sel", torch.int32, 2, dev)
    T, K = sel.shape
    P = T * K
    i32 = dict(dtype=torch.int32, device=dev)
    count = torch.empty(E, **i32)
    offsets = torch.empty(E + 1, **i32)
    perm = torch.full((P,), -7, **i32)
    slot = torch.empty(P, **i32)
    n_invalid = torch.empty(1, **i32)
    ws = torch.empty(max(bucket_workspace_size(T, K, E, flags), 1), dtype=torch.uint8, device=dev)
    with torch.cuda.device(dev):
        st = _abi.lib().mxfp4_moe_bucket(_ptr(sel), T, K, E, _ptr(count), _ptr(offsets), _ptr(perm), _ptr(slot),
                                         _ptr(n_invalid), flags, _ptr(ws), ws.numel(), _stream(dev))
    _abi.check(st, "mxfp4_moe_bucket")
    return {"count": count, "offsets": offsets, "perm": perm, "slot_of_pair": slot, "n_invalid": n_invalid}
