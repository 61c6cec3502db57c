"""The allocation-free entry point (mxfp4_moe_linear_noalloc, through the C
ABI) against mxfp4_moe_linear_ex on the same inputs: two calls in a row on
each path, the second with a smaller input, each equal bit for bit to the
workspace entry point's result (same kernels, same order of every sum)."""

import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU-only machines, never run there
    pytest.skip("no GPU", allow_module_level=True)

import mxfp4_block_scaled_amd as mx  # noqa: E402
from mxfp4_block_scaled_amd import _abi  # noqa: E402

DEV = torch.device("cuda:0")


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _inputs(seed, T, E, K, G, O, dtype):
    rng = np.random.default_rng(seed)
    td = torch.float32 if dtype == "fp32" else torch.bfloat16
    x = torch.from_numpy(rng.standard_normal((T, 32 * G)).astype(np.float32)).to(DEV).to(td)
    shared = torch.from_numpy(rng.standard_normal((T, O)).astype(np.float32)).to(DEV).to(td)
    packed = torch.from_numpy(rng.integers(0, 256, (E, O, G, 16), dtype=np.uint8)).to(DEV)
    scales = torch.from_numpy(rng.integers(118, 131, (E, O, G), dtype=np.uint8)).to(DEV)
    sel = torch.from_numpy(np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)).to(DEV)
    p = torch.from_numpy(rng.random((T, K)).astype(np.float32)).to(DEV)
    return x, packed, scales, sel, p, shared


def _noalloc(x, packed, scales, sel, p, shared, flags=0):
    T, I = x.shape
    E, O, G, _ = packed.shape
    K = sel.shape[1]
    dt = _abi.DTYPE_F32 if x.dtype == torch.float32 else _abi.DTYPE_BF16
    y = torch.empty_like(shared)
    st = _abi.lib().mxfp4_moe_linear_noalloc(
        x.data_ptr(), packed.data_ptr(), scales.data_ptr(), sel.data_ptr(), p.data_ptr(), shared.data_ptr(),
        y.data_ptr(), T, E, O, G, K, dt, flags, torch.cuda.current_stream(DEV).cuda_stream)
    return st, y


# (T, E, K, G, O) of a first call, then of a smaller second call
CASES = [
    ((1, 128, 4, 90, 5760), (1, 16, 2, 7, 300)),          # one token: the one-token kernel
    ((8, 64, 8, 224, 512), (3, 20, 4, 9, 130)),           # decode-shaped, several tokens
    ((200, 64, 4, 90, 1024), (70, 8, 2, 5, 260)),         # prefill-shaped: bucketing, grouped GEMM, combine
]


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("first,second", CASES, ids=["one-token", "decode", "prefill"])
def test_noalloc_matches_workspace_entry_point(first, second, dtype):
    for i, shape in enumerate((first, second)):
        T, E, K, G, O = shape
        say(f"no-alloc call {i} {shape} {dtype}")
        args = _inputs(sum(shape) + i, T, E, K, G, O, dtype)
        want = mx.moe_linear(*args)
        st, got = _noalloc(*args)
        torch.cuda.synchronize()
        assert st == _abi.OK, _abi.status_string(st)
        assert torch.equal(got, want), f"call {i} {shape}: differs from mxfp4_moe_linear_ex"


def test_noalloc_forced_paths_and_limit():
    args = _inputs(5, 40, 12, 4, 6, 200, "bf16")
    for flags in (_abi.FLAG_FORCE_GEMV, _abi.FLAG_FORCE_GEMM, _abi.FLAG_FORCE_GEMV | _abi.FLAG_GEMV_MFMA):
        st, got = _noalloc(*args, flags=flags)
        torch.cuda.synchronize()
        assert st == _abi.OK
        assert torch.equal(got, mx.moe_linear(*args, flags=flags))
    # a call whose workspace exceeds the scratch array is refused before anything runs
    T, E, K, G, O = 4096, 128, 4, 90, 5760
    need = _abi.workspace_size(T, E, O, G, K, _abi.DTYPE_BF16)
    assert need > _abi.NOALLOC_SCRATCH_BYTES
    st = _abi.lib().mxfp4_moe_linear_noalloc(1 << 20, 1 << 21, 1 << 22, 1 << 23, 1 << 24, 1 << 25, 1 << 26, T, E, O,
                                             G, K, _abi.DTYPE_BF16, 0, None)
    assert st == _abi.ERR_WORKSPACE_TOO_SMALL
