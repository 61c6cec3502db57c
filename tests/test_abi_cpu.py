"""The C-ABI library on the CPU: it loads, exports every symbol the header
declares, and its host-side checks return the documented status codes before
anything is enqueued. No call here reaches the GPU: every call either fails
validation or is a host-only query."""

import ctypes
import os
import re

import pytest

from conftest import ROOT
from mxfp4_block_scaled_amd import _abi

HEADER = os.path.join(ROOT, "include", "mxfp4_moe.h")

# fake, 256-byte aligned, never dereferenced: validation fails before any use
A = 0x100000
B = 0x200000
C = 0x300000


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mxfp4_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = _abi.lib()
    names = _declared()
    assert len(names) == 32
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_abi.SIGNATURES)


def test_header_constants_match_binding():
    text = open(HEADER).read()
    consts = dict(re.findall(r"#define (MXFP4_\w+) (0x[0-9a-f]+u?|\(1 << \d+\)|\d+)", text))
    assert int(consts["MXFP4_FLAG_FORCE_GEMV"].rstrip("u"), 16) == _abi.FLAG_FORCE_GEMV
    assert int(consts["MXFP4_FLAG_FORCE_GEMM"].rstrip("u"), 16) == _abi.FLAG_FORCE_GEMM
    assert int(consts["MXFP4_FLAG_CHECK"].rstrip("u"), 16) == _abi.FLAG_CHECK
    assert int(consts["MXFP4_FLAG_GEMV_MFMA"].rstrip("u"), 16) == _abi.FLAG_GEMV_MFMA
    assert int(consts["MXFP4_MAX_EXPERTS"]) == _abi.MAX_EXPERTS
    assert int(consts["MXFP4_ROUTE_SOFTMAX"]) == _abi.ROUTE_SOFTMAX
    assert int(consts["MXFP4_ROUTE_SIGMOID"]) == _abi.ROUTE_SIGMOID
    assert int(consts["MXFP4_ROUTE_MAX_EXPERTS"]) == _abi.ROUTE_MAX_EXPERTS
    assert int(consts["MXFP4_ROUTE_MAX_K"]) == _abi.ROUTE_MAX_K
    for name, val in re.findall(r"(MXFP4_(?:OK|ERR_\w+)) = (-?\d+)", text):
        assert getattr(_abi, name[len("MXFP4_"):]) == int(val)


def test_status_strings():
    assert _abi.status_string(0) == "ok"
    for s in (-1, -2, -3, -4, -5, -6):
        assert _abi.status_string(s) not in ("ok", "unknown status")
    assert _abi.status_string(-99) == "unknown status"


def test_workspace_sizes_host_only():
    assert _abi.workspace_size(0, 4, 32, 2, 2, _abi.DTYPE_F32) == 0
    small = _abi.workspace_size(1, 128, 5760, 90, 4, _abi.DTYPE_F32)
    assert 0 < small <= 4096  # decode-shaped path: a status word only
    big = _abi.workspace_size(4096, 128, 5760, 90, 4, _abi.DTYPE_BF16)
    assert big >= 4096 * 4 * 5760 * 4  # fp32 partial rows [P, O]
    assert _abi.bucket_workspace_size(8192, 8, 384) >= 4 * 384 * 64


def test_path_selection():
    f32, bf16 = _abi.DTYPE_F32, _abi.DTYPE_BF16
    assert _abi.select_path(1, 128, 5760, 90, 4, f32) == _abi.PATH_GEMV
    # the decode-shaped path while one fused launch takes every pair (at most
    # 64 pairs, activations in LDS), the grouped GEMM past that
    assert _abi.select_path(8, 384, 4096, 224, 8, bf16) == _abi.PATH_GEMV
    assert _abi.select_path(9, 384, 4096, 224, 8, bf16) == _abi.PATH_GEMM
    assert _abi.select_path(16, 384, 4096, 224, 8, bf16) == _abi.PATH_GEMM
    assert _abi.select_path(16, 128, 5760, 90, 4, bf16) == _abi.PATH_GEMV
    assert _abi.select_path(17, 128, 5760, 90, 4, bf16) == _abi.PATH_GEMM
    assert _abi.select_path(64, 128, 5760, 2, 1, bf16) == _abi.PATH_GEMV
    assert _abi.select_path(65, 128, 5760, 2, 1, bf16) == _abi.PATH_GEMM
    assert _abi.select_path(4096, 128, 5760, 90, 4, bf16) == _abi.PATH_GEMM
    assert _abi.select_path(4096, 128, 5760, 90, 4, f32) == _abi.PATH_GEMM
    assert _abi.select_path(8, 384, 4096, 224, 8, bf16, _abi.FLAG_FORCE_GEMM) == _abi.PATH_GEMM
    assert _abi.select_path(4096, 128, 5760, 90, 4, bf16, _abi.FLAG_FORCE_GEMV) == _abi.PATH_GEMV
    assert _abi.select_path(4096, 128, 5760, 90, 4, f32, _abi.FLAG_FORCE_GEMV) == _abi.PATH_GEMV
    assert _abi.select_path(4, 4, 32, 2, 2, f32, _abi.FLAG_FORCE_GEMM) == _abi.PATH_GEMM
    # fp32 activations: the grouped GEMM reads three bf16 planes of them
    assert _abi.select_path(5000, 8, 64, 1 << 11, 1, bf16, _abi.FLAG_FORCE_GEMM) == _abi.PATH_GEMM
    with pytest.raises(_abi.Mxfp4Error) as e:
        _abi.select_path(5500, 8, 64, 1 << 11, 1, f32, _abi.FLAG_FORCE_GEMM)
    assert e.value.status == _abi.ERR_UNSUPPORTED
    with pytest.raises(_abi.Mxfp4Error) as e:
        _abi.select_path(4, 4, 32, 2, 2, bf16, _abi.FLAG_FORCE_GEMM | _abi.FLAG_FORCE_GEMV)
    assert e.value.status == _abi.ERR_INVALID_ARG
    # one expert of 2^31 packed bytes or more: beyond every kernel's 32-bit
    # buffer offsets
    O, G = 1 << 16, 1 << 11
    for flags in (0, _abi.FLAG_GEMV_MFMA):
        assert _abi.select_path(1, 2, O, G - 1, 1, bf16, flags) == _abi.PATH_GEMV
        assert _abi.select_path(1, 2, O, G - 1, 1, bf16, flags | _abi.FLAG_FORCE_GEMM) == _abi.PATH_GEMM
        for dt in (f32, bf16):
            with pytest.raises(_abi.Mxfp4Error) as e:
                _abi.select_path(1, 2, O, G, 1, dt, flags)
            assert e.value.status == _abi.ERR_UNSUPPORTED
    # activations of 2^31 bytes or more: beyond the grouped GEMM's offsets;
    # the decode-shaped path takes them in token chunks
    T, G = 1 << 16, 1 << 9
    assert _abi.select_path(T - 1, 8, 64, G, 1, bf16) == _abi.PATH_GEMM
    assert _abi.select_path(T, 8, 64, G, 1, bf16) == _abi.PATH_GEMV
    with pytest.raises(_abi.Mxfp4Error) as e:
        _abi.select_path(T, 8, 64, G, 1, bf16, _abi.FLAG_FORCE_GEMM)
    assert e.value.status == _abi.ERR_UNSUPPORTED


def _ex(x=A, packed=B, scales=C + 0x10000, sel=C + 0x20000, p=C + 0x30000, shared=C + 0x40000, y=C + 0x50000,
        T=1, E=2, O=4, G=1, K=1, dtype=0, flags=0, ws=C + 0x60000, ws_bytes=1 << 20):
    return _abi.lib().mxfp4_moe_linear_ex(x, packed, scales, sel, p, shared, y, T, E, O, G, K, dtype, flags, ws,
                                          ws_bytes, None)


@pytest.mark.parametrize("kw", [
    dict(T=-1), dict(E=0), dict(O=0), dict(G=0), dict(K=0), dict(E=_abi.MAX_EXPERTS + 1),
    dict(T=1 << 24, K=8), dict(dtype=7), dict(x=0), dict(packed=0), dict(scales=0), dict(sel=0), dict(p=0),
    dict(shared=0), dict(y=0), dict(x=A + 4), dict(packed=B + 8), dict(sel=C + 0x20001), dict(p=C + 0x30002),
    dict(y=C + 0x50001), dict(y=A), dict(y=B + 64), dict(y=C + 0x10000), dict(flags=0x100),
    dict(flags=_abi.FLAG_FORCE_GEMV | _abi.FLAG_FORCE_GEMM),
])
def test_invalid_arguments_rejected(kw):
    assert _ex(**kw) == _abi.ERR_INVALID_ARG


def test_workspace_too_small_rejected():
    M = 1 << 28  # far apart: no fake buffer overlaps another at this size
    kw = dict(x=1 * M, packed=2 * M, scales=3 * M, sel=4 * M, p=5 * M, shared=6 * M, y=7 * M, ws=8 * M)
    assert _ex(T=4096, E=128, O=64, G=2, K=4, dtype=1, ws_bytes=1024, **kw) == _abi.ERR_WORKSPACE_TOO_SMALL


def test_fp32_forced_gemm_workspace_holds_the_activation_planes():
    # fp32 activations on the grouped GEMM: the workspace also holds their
    # three bf16 planes (3 * T * I * 2 bytes) beside what the bf16 call needs
    T, E, O, G, K = 300, 8, 64, 4, 2
    f32 = _abi.workspace_size(T, E, O, G, K, _abi.DTYPE_F32, _abi.FLAG_FORCE_GEMM)
    bf16 = _abi.workspace_size(T, E, O, G, K, _abi.DTYPE_BF16, _abi.FLAG_FORCE_GEMM)
    assert f32 >= bf16 + 3 * T * 32 * G * 2
    M = 1 << 28
    kw = dict(x=1 * M, packed=2 * M, scales=3 * M, sel=4 * M, p=5 * M, shared=6 * M, y=7 * M, ws=8 * M)
    assert _ex(T=T, E=E, O=O, G=G, K=K, dtype=0, flags=_abi.FLAG_FORCE_GEMM, ws_bytes=f32 - 1,
               **kw) == _abi.ERR_WORKSPACE_TOO_SMALL


def test_empty_batch_is_a_no_op():
    # T = 0 is valid and enqueues nothing, even with null tensor pointers
    assert _ex(T=0, x=0, packed=0, scales=0, sel=0, p=0, shared=0, y=0, ws=0, ws_bytes=0) == _abi.OK
    lib = _abi.lib()
    assert lib.mxfp4_moe_linear(None, None, None, None, None, None, None, 0, 2, 4, 1, 1, None) == _abi.OK
    assert lib.mxfp4_moe_linear_bf16(None, None, None, None, None, None, None, 0, 2, 4, 1, 1, None) == _abi.OK


def test_plain_entry_points_validate():
    lib = _abi.lib()
    assert lib.mxfp4_moe_linear(A, 0, C, C, C, C, C, 1, 2, 4, 1, 1, None) == _abi.ERR_INVALID_ARG
    assert lib.mxfp4_moe_linear_bf16(A, B, C, C, C, C, C, 1, 0, 4, 1, 1, None) == _abi.ERR_INVALID_ARG


def test_decode_rows_validates():
    lib = _abi.lib()
    f = lib.mxfp4_decode_rows
    assert f(B, C, 2, 4, 1, 2, 0, 1, 0, A, None) == _abi.ERR_INVALID_ARG  # e out of range
    assert f(B, C, 2, 4, 1, 0, 3, 2, 0, A, None) == _abi.ERR_INVALID_ARG  # rows past O
    assert f(B, C, 2, 4, 1, 0, 0, 1, 5, A, None) == _abi.ERR_INVALID_ARG  # dtype
    assert f(B + 1, C, 2, 4, 1, 0, 0, 1, 0, A, None) == _abi.ERR_INVALID_ARG  # misaligned packed
    assert f(B, C, 2, 4, 1, 0, 0, 0, 0, A, None) == _abi.OK  # nothing to do


def test_bucket_validates():
    lib = _abi.lib()
    f = lib.mxfp4_moe_bucket
    assert f(A, 1, 1, 0, B, B, B, B, B, 0, C, 64, None) == _abi.ERR_INVALID_ARG
    assert f(A, 1, 1, 4, 0, B, B, B, B, 0, C, 64, None) == _abi.ERR_INVALID_ARG
    assert f(A, 1, 1, 4, B, B, B, B, B, _abi.FLAG_BUCKET_ONE_BLOCK | _abi.FLAG_BUCKET_MULTI_BLOCK, C, 64,
             None) == _abi.ERR_INVALID_ARG
    assert f(A, 1000, 8, 4, B, B, B, B, B, _abi.FLAG_BUCKET_MULTI_BLOCK, C, 4, None) == _abi.ERR_WORKSPACE_TOO_SMALL


def test_gemm_stage_host_checks():
    # rejected on the host before any device work: sizes, null pointers, workspace size
    lib = _abi.lib()
    a, b = 1 << 40, 1 << 41
    assert lib.mxfp4_moe_gemm_stage(a, a, a, 4, 0, 32, 2, 2, b, 1 << 20, None) == _abi.ERR_INVALID_ARG
    assert lib.mxfp4_moe_gemm_stage(None, a, a, 4, 4, 32, 2, 2, b, 1 << 20, None) == _abi.ERR_INVALID_ARG
    assert lib.mxfp4_moe_gemm_stage(a, a, a, 4, 4, 32, 2, 2, b, 16, None) == _abi.ERR_WORKSPACE_TOO_SMALL
    assert lib.mxfp4_moe_gemm_stage(a, a, a, 0, 4, 32, 2, 2, None, 0, None) == _abi.OK



# ---- the SwiGLU expert block

def _sw(x=A, gu_p=B, gu_s=C + 0x10000, dn_p=B + 0x80000, dn_s=C + 0x18000, sel=C + 0x20000, p=C + 0x30000,
        shared=C + 0x40000, y=C + 0x50000, T=2, E=3, F=32, G=1, O=8, K=2, flags=0, ws=C + 0x60000,
        ws_bytes=1 << 24):
    return _abi.lib().mxfp4_moe_swiglu_ex(x, gu_p, gu_s, dn_p, dn_s, sel, p, shared, y, T, E, F, G, O, K, flags,
                                          ws, ws_bytes, None)


def test_swiglu_workspace_size():
    assert _abi.swiglu_workspace_size(0, 4, 32, 2, 8, 2) == 0
    T, E, F, G, O, K = 4096, 128, 2048, 90, 5760, 4
    ws = _abi.swiglu_workspace_size(T, E, F, G, O, K)
    assert ws >= T * K * O * 4 + T * K * F * 2  # fp32 partial rows and the bf16 intermediate
    with pytest.raises(_abi.Mxfp4Error) as e:  # the intermediate h reaches 2^31 bytes
        _abi.swiglu_workspace_size(1 << 16, 8, 1 << 11, 2, 8, 8)
    assert e.value.status == _abi.ERR_UNSUPPORTED


@pytest.mark.parametrize("kw", [
    dict(T=-1), dict(E=0), dict(F=0), dict(F=48), dict(F=16), dict(G=0), dict(O=0), dict(K=0),
    dict(E=_abi.MAX_EXPERTS + 1), dict(flags=_abi.FLAG_FORCE_GEMM), dict(flags=0x100),
    dict(x=0), dict(gu_p=0), dict(gu_s=0), dict(dn_p=0), dict(dn_s=0), dict(sel=0), dict(p=0), dict(shared=0),
    dict(y=0), dict(x=A + 4), dict(gu_p=B + 8), dict(dn_p=B + 0x80008), dict(sel=C + 0x20001), dict(p=C + 0x30002),
    dict(y=C + 0x50001), dict(y=A), dict(y=B + 64), dict(y=C + 0x18000), dict(y=B + 0x80000),
])
def test_swiglu_host_checks_reject(kw):
    assert _sw(**kw) == _abi.ERR_INVALID_ARG


def test_swiglu_host_checks_workspace_and_empty():
    assert _sw(ws_bytes=16) == _abi.ERR_WORKSPACE_TOO_SMALL
    assert _sw(T=0, x=0, y=0, shared=0, sel=0, p=0) == _abi.OK  # nothing to do, nothing enqueued


# ---- the router

def _route(logits=A, bias=0, T=2, E=8, K=2, mode=0, scale=1.0, sel=B, p=C):
    return _abi.lib().mxfp4_moe_route(logits, bias, T, E, K, mode, scale, sel, p, None)


@pytest.mark.parametrize("kw", [
    dict(T=-1), dict(E=0), dict(K=0), dict(K=9), dict(E=_abi.ROUTE_MAX_EXPERTS + 1, K=2),
    dict(E=128, K=_abi.ROUTE_MAX_K + 1), dict(mode=2), dict(mode=-1), dict(bias=C + 0x1000),
    dict(scale=float("inf")), dict(scale=float("nan")), dict(logits=0), dict(sel=0), dict(p=0),
    dict(logits=A + 2), dict(sel=B + 1), dict(p=C + 3), dict(mode=1, bias=C + 0x1002),
    dict(p=B + 8), dict(sel=A + 32), dict(p=A), dict(mode=1, bias=B + 4), dict(mode=1, bias=C + 12),
])
def test_route_host_checks_reject(kw):
    assert _route(**kw) == _abi.ERR_INVALID_ARG


def test_route_empty_batch_is_a_no_op():
    assert _route(T=0, logits=0, sel=0, p=0) == _abi.OK
    assert _route(T=0, mode=1, bias=C + 0x1000) == _abi.OK


# ---- the block-scaled variant

MX_ENTRY = ["mxfp4_moe_linear_mxfp8_ex", "mxfp4_moe_linear_mxfp4act_ex"]


def _mx(x=A, packed=B, scales=C, sel=C + 0x10000, p=C + 0x20000, shared=C + 0x30000, y=C + 0x40000, T=2, E=3,
        O=8, G=2, K=2, flags=0, ws=C + 0x60000, ws_bytes=1 << 24, fn="mxfp4_moe_linear_mxfp8_ex"):
    return getattr(_abi.lib(), fn)(x, packed, scales, sel, p, shared, y, T, E, O, G, K, flags, ws, ws_bytes, None)


def test_mxfp8_workspace_size():
    assert _abi.mxfp8_workspace_size(0, 4, 8, 2, 2) == 0
    T, E, O, G, K = 4096, 128, 5760, 90, 4
    ws = _abi.mxfp8_workspace_size(T, E, O, G, K)
    assert ws >= T * K * O * 4 + T * 2944 + T * 2944 // 32  # fp32 partial rows, codes and scales of 128-padded rows
    with pytest.raises(_abi.Mxfp4Error) as e:  # O % 4 != 0
        _abi.mxfp8_workspace_size(4, 4, 6, 2, 2)
    assert e.value.status == _abi.ERR_UNSUPPORTED


@pytest.mark.parametrize("kw", [
    dict(T=-1), dict(E=0), dict(O=0), dict(G=0), dict(K=0), dict(flags=_abi.FLAG_FORCE_GEMM), dict(flags=0x100),
    dict(x=0), dict(packed=0), dict(scales=0), dict(sel=0), dict(p=0), dict(shared=0), dict(y=0),
    dict(x=A + 2), dict(sel=C + 0x10001), dict(y=A), dict(y=B + 16),
])
@pytest.mark.parametrize("fn", MX_ENTRY)
def test_mxfp8_host_checks_reject(kw, fn):
    assert _mx(fn=fn, **kw) == _abi.ERR_INVALID_ARG


@pytest.mark.parametrize("fn", MX_ENTRY)
def test_mxfp8_host_checks_workspace_unsupported_and_empty(fn):
    assert _mx(ws_bytes=16, fn=fn) == _abi.ERR_WORKSPACE_TOO_SMALL
    assert _mx(O=6, fn=fn) == _abi.ERR_UNSUPPORTED
    assert _mx(T=0, x=0, y=0, shared=0, sel=0, p=0, fn=fn) == _abi.OK


def test_mxfp4act_workspace_size():
    assert _abi.mxfp4act_workspace_size(0, 4, 8, 2, 2) == 0
    T, E, O, G, K = 4096, 128, 5760, 90, 4
    ws = _abi.mxfp4act_workspace_size(T, E, O, G, K)
    # fp32 partial rows, codes (two per byte) and scales of 128-padded rows
    assert ws >= T * K * O * 4 + T * 2944 // 2 + T * 2944 // 32
    assert ws < _abi.mxfp8_workspace_size(T, E, O, G, K)
    with pytest.raises(_abi.Mxfp4Error) as e:  # O % 4 != 0
        _abi.mxfp4act_workspace_size(4, 4, 6, 2, 2)
    assert e.value.status == _abi.ERR_UNSUPPORTED


@pytest.mark.parametrize("args", [
    (A, -1, 64, 64, B, C), (A, 2, 48, 64, B, C), (A, 2, 64, 48, B, C), (A, 2, 64, 80, B, C), (A, 2, 0, 32, B, C),
    (0, 2, 64, 64, B, C), (A, 2, 64, 64, 0, C), (A, 2, 64, 64, B, 0), (A + 4, 2, 64, 64, B, C),
    (A, 2, 64, 64, B + 2, C), (A, 2, 64, 64, A + 64, C), (A, 2, 64, 64, B, A + 8),
    (A, 1 << 25, 64, 64, B, C),
])
@pytest.mark.parametrize("fn", ["mxfp4_quantize_mxfp8", "mxfp4_quantize_mxfp4"])
def test_quantize_mxfp8_host_checks(args, fn):
    x, T, I, ld, codes, sb = args
    assert getattr(_abi.lib(), fn)(x, T, I, ld, codes, sb, None) == _abi.ERR_INVALID_ARG


@pytest.mark.parametrize("fn", ["mxfp4_quantize_mxfp8", "mxfp4_quantize_mxfp4"])
def test_quantize_mxfp8_empty(fn):
    assert getattr(_abi.lib(), fn)(0, 0, 64, 64, 0, 0, None) == _abi.OK


def test_mx_prepared_size_and_host_checks():
    E, O, G = 128, 5760, 90
    n = _abi.mx_prepared_size(E, O, G)
    assert n == E * 45 * 23 * 512 * 17  # 45 N-tiles, 23 chunks of 4 groups, 512 slots of 17 bytes
    with pytest.raises(_abi.Mxfp4Error) as e:
        _abi.mx_prepared_size(4, 6, 2)  # O % 4 != 0
    assert e.value.status == _abi.ERR_UNSUPPORTED
    lib = _abi.lib()
    small = _abi.mx_prepared_size(2, 8, 2)
    assert lib.mxfp4_prepare_mx(B, C, 2, 8, 2, A, small - 1, None) == _abi.ERR_WORKSPACE_TOO_SMALL
    for args in [(0, C, A), (B, 0, A), (B, C, 0), (B + 4, C, A), (B, C, A + 8), (B, C, B + 64)]:
        assert lib.mxfp4_prepare_mx(args[0], args[1], 2, 8, 2, args[2], small, None) == _abi.ERR_INVALID_ARG
    # the prepared layer: same argument rules as the canonical one
    ws = C + 0x60000
    assert lib.mxfp4_moe_linear_mxfp8_prepared_ex(A, B, C + 0x10000, C + 0x20000, C + 0x30000, C + 0x40000, 2, 2, 8,
                                                  2, 2, 0, ws, 16, None) == _abi.ERR_WORKSPACE_TOO_SMALL
    assert lib.mxfp4_moe_linear_mxfp8_prepared_ex(A, 0, C + 0x10000, C + 0x20000, C + 0x30000, C + 0x40000, 2, 2, 8,
                                                  2, 2, 0, ws, 1 << 24, None) == _abi.ERR_INVALID_ARG
    assert lib.mxfp4_moe_linear_mxfp8_prepared_ex(A, B, C + 0x10000, C + 0x20000, C + 0x30000, B + 32, 2, 2, 8,
                                                  2, 2, 0, ws, 1 << 24, None) == _abi.ERR_INVALID_ARG
    assert lib.mxfp4_moe_linear_mxfp8_prepared_ex(0, 0, 0, 0, 0, 0, 0, 2, 8, 2, 2, 0, 0, 0, None) == _abi.OK
    for fn in (lib.mxfp4_moe_linear_mxfp4act_prepared_ex,):
        assert fn(A, B, C + 0x10000, C + 0x20000, C + 0x30000, C + 0x40000, 2, 2, 8, 2, 2, 0, ws, 16,
                  None) == _abi.ERR_WORKSPACE_TOO_SMALL
        assert fn(A, 0, C + 0x10000, C + 0x20000, C + 0x30000, C + 0x40000, 2, 2, 8, 2, 2, 0, ws, 1 << 24,
                  None) == _abi.ERR_INVALID_ARG
        assert fn(A, B, C + 0x10000, C + 0x20000, C + 0x30000, B + 32, 2, 2, 8, 2, 2, 0, ws, 1 << 24,
                  None) == _abi.ERR_INVALID_ARG
        assert fn(0, 0, 0, 0, 0, 0, 0, 2, 8, 2, 2, 0, 0, 0, None) == _abi.OK


# ------------------------------------------------------------------ prepared-weight entry points (host checks)

M28 = 1 << 28  # far-apart fake device addresses: no buffer overlaps another


def _prep_ex(fn, x=1 * M28, prep=2 * M28, sel=4 * M28, p=5 * M28, shared=6 * M28, y=7 * M28, T=64, E=4, O=64, G=2,
             K=2, flags=0, ws=8 * M28, ws_bytes=1 << 30, dtype=None):
    lib = _abi.lib()
    if fn == "decode":
        return lib.mxfp4_moe_decode_prepared_ex(x, prep, sel, p, shared, y, T, E, O, G, K,
                                                _abi.DTYPE_F32 if dtype is None else dtype, flags, ws, ws_bytes, None)
    return lib.mxfp4_moe_linear_prepared_ex(x, prep, sel, p, shared, y, T, E, O, G, K, flags, ws, ws_bytes, None)


@pytest.mark.parametrize("fn", ["linear", "decode"])
@pytest.mark.parametrize("kw,status", [
    (dict(T=-1), "ERR_INVALID_ARG"), (dict(E=0), "ERR_INVALID_ARG"), (dict(x=0), "ERR_INVALID_ARG"),
    (dict(prep=0), "ERR_INVALID_ARG"), (dict(sel=0), "ERR_INVALID_ARG"), (dict(y=2 * M28), "ERR_INVALID_ARG"),
    (dict(flags=_abi.FLAG_FORCE_GEMM), "ERR_INVALID_ARG"), (dict(O=34), "ERR_UNSUPPORTED"),
    (dict(ws_bytes=16), "ERR_WORKSPACE_TOO_SMALL"), (dict(T=0, x=0, prep=0, sel=0, p=0, shared=0, y=0), "OK"),
])
def test_prepared_entry_points_validate_on_the_host(fn, kw, status):
    assert _prep_ex(fn, **kw) == getattr(_abi, status)


def test_prepare_entry_points_validate_on_the_host():
    lib = _abi.lib()
    n = _abi.mx_prepared_size(4, 64, 2)
    assert n == 4 * 1 * 1 * 512 * 17  # one 128-row tile, one 128-input chunk per expert
    for fn in (lib.mxfp4_prepare_mx, lib.mxfp4_prepare_bf16):
        assert fn(1 * M28, 2 * M28, 4, 64, 2, 3 * M28, n - 1, None) == _abi.ERR_WORKSPACE_TOO_SMALL
        assert fn(1 * M28, 2 * M28, 4, 66, 2, 3 * M28, 1 << 30, None) == _abi.ERR_UNSUPPORTED  # O % 4
        assert fn(1 * M28 + 8, 2 * M28, 4, 64, 2, 3 * M28, n, None) == _abi.ERR_INVALID_ARG    # alignment
        assert fn(1 * M28, 2 * M28, 4, 64, 2, 1 * M28, n, None) == _abi.ERR_INVALID_ARG        # overlap
    # SwiGLU gate/up: F a multiple of 32, the size of a (E, 2F, G) repack
    assert lib.mxfp4_prepare_swiglu(1 * M28, 2 * M28, 4, 48, 2, 3 * M28, 1 << 30, None) == _abi.ERR_INVALID_ARG
    assert lib.mxfp4_prepare_swiglu(1 * M28, 2 * M28, 4, 64, 2, 3 * M28, _abi.mx_prepared_size(4, 128, 2) - 1,
                                    None) == _abi.ERR_WORKSPACE_TOO_SMALL
