"""ctypes view of the C ABI in include/mxfp4_moe.h (argument marshalling only).

Loading fails loudly when the shared library has not been built: there is
no fallback implementation of any step.
"""

from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmxfp4_moe.so")

# mirrors of the header's constants
OK = 0
ERR_INVALID_ARG = -1
ERR_UNSUPPORTED_DEVICE = -2
ERR_HIP = -3
ERR_WORKSPACE_TOO_SMALL = -4
ERR_INVALID_INDEX = -5
ERR_UNSUPPORTED = -6

DTYPE_F32 = 0
DTYPE_BF16 = 1

FLAG_FORCE_GEMV = 0x1
FLAG_FORCE_GEMM = 0x2
FLAG_CHECK = 0x4
FLAG_GEMV_MFMA = 0x8
FLAG_BUCKET_ONE_BLOCK = 0x10
FLAG_BUCKET_MULTI_BLOCK = 0x20

NOALLOC_SCRATCH_BYTES = 32 << 20

MAX_EXPERTS = 8192
MAX_PAIRS = 1 << 26

PATH_GEMV = 1
PATH_GEMM = 2

ROUTE_SOFTMAX = 0
ROUTE_SIGMOID = 1
ROUTE_MAX_EXPERTS = 1024
ROUTE_MAX_K = 64
ROUTE_MAX_GROUPS = 64

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_int = ctypes.c_int
_u32 = ctypes.c_uint32
_sz = ctypes.c_size_t

# name -> (restype, argtypes), in the header's order
SIGNATURES = {
    "mxfp4_moe_linear": (_int, [_vp] * 7 + [_i64] * 5 + [_vp]),
    "mxfp4_moe_linear_bf16": (_int, [_vp] * 7 + [_i64] * 5 + [_vp]),
    "mxfp4_moe_workspace_size": (_int, [_i64] * 5 + [_int, _u32, ctypes.POINTER(_sz)]),
    "mxfp4_moe_linear_ex": (_int, [_vp] * 7 + [_i64] * 5 + [_int, _u32, _vp, _sz, _vp]),
    "mxfp4_moe_linear_noalloc": (_int, [_vp] * 7 + [_i64] * 5 + [_int, _u32, _vp]),
    "mxfp4_moe_select_path": (_int, [_i64] * 5 + [_int, _u32]),
    "mxfp4_moe_bucket_workspace_size": (_int, [_i64] * 3 + [_u32, ctypes.POINTER(_sz)]),
    "mxfp4_moe_bucket": (_int, [_vp] + [_i64] * 3 + [_vp] * 5 + [_u32, _vp, _sz, _vp]),
    "mxfp4_decode_rows": (_int, [_vp] * 2 + [_i64] * 6 + [_int, _vp, _vp]),
    "mxfp4_moe_gemm_stage": (_int, [_vp] * 3 + [_i64] * 5 + [_vp, _sz, _vp]),
    "mxfp4_moe_swiglu_workspace_size": (_int, [_i64] * 6 + [ctypes.POINTER(_sz)]),
    "mxfp4_moe_swiglu_ex": (_int, [_vp] * 9 + [_i64] * 6 + [_u32, _vp, _sz, _vp]),
    "mxfp4_moe_route": (_int, [_vp] * 2 + [_i64] * 3 + [_int, ctypes.c_float, _vp, _vp, _vp]),
    "mxfp4_quantize_mxfp8": (_int, [_vp] + [_i64] * 3 + [_vp, _vp, _vp]),
    "mxfp4_moe_mxfp8_workspace_size": (_int, [_i64] * 5 + [ctypes.POINTER(_sz)]),
    "mxfp4_moe_linear_mxfp8_ex": (_int, [_vp] * 7 + [_i64] * 5 + [_u32, _vp, _sz, _vp]),
    "mxfp4_mx_prepared_size": (_int, [_i64] * 3 + [ctypes.POINTER(_sz)]),
    "mxfp4_prepare_mx": (_int, [_vp] * 2 + [_i64] * 3 + [_vp, _sz, _vp]),
    "mxfp4_moe_linear_mxfp8_prepared_ex": (_int, [_vp] * 6 + [_i64] * 5 + [_u32, _vp, _sz, _vp]),
    "mxfp4_quantize_mxfp4": (_int, [_vp] + [_i64] * 3 + [_vp, _vp, _vp]),
    "mxfp4_moe_mxfp4act_workspace_size": (_int, [_i64] * 5 + [ctypes.POINTER(_sz)]),
    "mxfp4_moe_linear_mxfp4act_ex": (_int, [_vp] * 7 + [_i64] * 5 + [_u32, _vp, _sz, _vp]),
    "mxfp4_moe_linear_mxfp4act_prepared_ex": (_int, [_vp] * 6 + [_i64] * 5 + [_u32, _vp, _sz, _vp]),
    "mxfp4_moe_linear_prepared_ex": (_int, [_vp] * 6 + [_i64] * 5 + [_u32, _vp, _sz, _vp]),
    "mxfp4_moe_gemm_stage_prepared": (_int, [_vp] * 2 + [_i64] * 5 + [_vp, _sz, _vp]),
    "mxfp4_moe_decode_prepared_ex": (_int, [_vp] * 6 + [_i64] * 5 + [_int, _u32, _vp, _sz, _vp]),
    "mxfp4_prepare_bf16": (_int, [_vp] * 2 + [_i64] * 3 + [_vp, _sz, _vp]),
    "mxfp4_prepare_swiglu": (_int, [_vp] * 2 + [_i64] * 3 + [_vp, _sz, _vp]),
    "mxfp4_moe_swiglu_prepared_ex": (_int, [_vp] * 7 + [_i64] * 6 + [_u32, _vp, _sz, _vp]),
    "mxfp4_moe_route_grouped": (_int, [_vp] * 2 + [_i64] * 5 + [_int, ctypes.c_float, _vp, _vp, _vp]),
    "mxfp4_stream_read": (_int, [_vp, _sz, _int, _vp, _vp]),
    "mxfp4_status_string": (ctypes.c_char_p, [_int]),
}

_lib = None


class Mxfp4Error(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} ({status})" if what else f"{status_string(status)} ({status})")


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it is missing or lacks a symbol)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m mxfp4_block_scaled_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def status_string(status: int) -> str:
    return lib().mxfp4_status_string(int(status)).decode()


def check(status: int, what: str = "") -> None:
    if status != OK:
        raise Mxfp4Error(status, what)


def workspace_size(T, E, O, G, K, dtype, flags=0) -> int:
    out = _sz(0)
    check(lib().mxfp4_moe_workspace_size(T, E, O, G, K, dtype, flags, ctypes.byref(out)), "workspace_size")
    return out.value


def swiglu_workspace_size(T, E, F, G, O, K) -> int:
    out = _sz(0)
    check(lib().mxfp4_moe_swiglu_workspace_size(T, E, F, G, O, K, ctypes.byref(out)), "swiglu_workspace_size")
    return out.value


def mxfp8_workspace_size(T, E, O, G, K) -> int:
    out = _sz(0)
    check(lib().mxfp4_moe_mxfp8_workspace_size(T, E, O, G, K, ctypes.byref(out)), "mxfp8_workspace_size")
    return out.value


def mxfp4act_workspace_size(T, E, O, G, K) -> int:
    out = _sz(0)
    check(lib().mxfp4_moe_mxfp4act_workspace_size(T, E, O, G, K, ctypes.byref(out)), "mxfp4act_workspace_size")
    return out.value


def mx_prepared_size(E, O, G) -> int:
    out = _sz(0)
    check(lib().mxfp4_mx_prepared_size(E, O, G, ctypes.byref(out)), "mx_prepared_size")
    return out.value


def bucket_workspace_size(T, K, E, flags=0) -> int:
    out = _sz(0)
    check(lib().mxfp4_moe_bucket_workspace_size(T, K, E, flags, ctypes.byref(out)), "bucket_workspace_size")
    return out.value


def select_path(T, E, O, G, K, dtype, flags=0) -> int:
    r = lib().mxfp4_moe_select_path(T, E, O, G, K, dtype, flags)
    if r < 0:
        raise Mxfp4Error(r, "select_path")
    return r
