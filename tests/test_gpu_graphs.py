"""HIP graph capture of the entry points that promise to allocate nothing:
each call is captured once and replayed several times, with eager work on
other buffers between the replays; every replay must equal the eager result
bit for bit (the same kernels on the same inputs)."""

import sys

import numpy as np
import pytest

import workloads

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU-only machines, never run there
    pytest.skip("no GPU", allow_module_level=True)

import mxfp4_block_scaled_amd as mx  # noqa: E402

DEV = torch.device("cuda:0")


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV).to(torch.bfloat16)


def _case(seed, T, E, K, G, O):
    rng = np.random.default_rng(seed)
    x = workloads.round_to_bf16(rng.standard_normal((T, 32 * G)).astype(np.float32))
    shared = workloads.round_to_bf16(rng.standard_normal((T, O)).astype(np.float32))
    packed = torch.from_numpy(rng.integers(0, 256, (E, O, G, 16), dtype=np.uint8)).to(DEV)
    scales = torch.from_numpy(rng.integers(118, 131, (E, O, G), dtype=np.uint8)).to(DEV)
    sel = torch.from_numpy(np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)).to(DEV)
    p = torch.from_numpy(rng.random((T, K)).astype(np.float32)).to(DEV)
    return bf16(x), packed, scales, sel, p, bf16(shared)


def _replays_match(call, out, disturb, n=3):
    """call() writes `out`; compare eager against n graph replays."""
    call()
    torch.cuda.synchronize()
    want = out.clone()
    out.zero_()
    stream = torch.cuda.Stream(device=DEV)
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        call()  # settle the stream outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        call()
    for r in range(n):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want), f"replay {r} differs from the eager call"
        disturb()
        torch.cuda.synchronize()


def test_graph_prefill_shaped_layer():
    say("graph: moe_linear (bf16, prefill-shaped)")
    x, packed, scales, sel, p, shared = _case(1, 300, 8, 4, 6, 264)
    ws = torch.empty(mx.workspace_size(300, 8, 264, 6, 4, mx.DTYPE_BF16), dtype=torch.uint8, device=DEV)
    out = torch.empty_like(shared)
    other = torch.empty_like(shared)
    _replays_match(lambda: mx.moe_linear(x, packed, scales, sel, p, shared, out=out, workspace=ws), out,
                   lambda: mx.moe_linear(x, packed, scales, sel.flip(1).contiguous(), p, shared, out=other))


def test_graph_swiglu_block():
    say("graph: moe_swiglu")
    rng = np.random.default_rng(2)
    T, E, K, G, F, O = 70, 6, 2, 4, 64, 96
    x = bf16(workloads.round_to_bf16(rng.standard_normal((T, 32 * G)).astype(np.float32)))
    shared = bf16(workloads.round_to_bf16(rng.standard_normal((T, O)).astype(np.float32)))
    gu_p = torch.from_numpy(rng.integers(0, 256, (E, 2 * F, G, 16), dtype=np.uint8)).to(DEV)
    gu_s = torch.from_numpy(rng.integers(118, 127, (E, 2 * F, G), dtype=np.uint8)).to(DEV)
    dn_p = torch.from_numpy(rng.integers(0, 256, (E, O, F // 32, 16), dtype=np.uint8)).to(DEV)
    dn_s = torch.from_numpy(rng.integers(118, 127, (E, O, F // 32), dtype=np.uint8)).to(DEV)
    sel = torch.from_numpy(np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)).to(DEV)
    p = torch.from_numpy(rng.random((T, K)).astype(np.float32)).to(DEV)
    ws = torch.empty(mx.swiglu_workspace_size(T, E, F, G, O, K), dtype=torch.uint8, device=DEV)
    out = torch.empty_like(shared)
    other = torch.empty_like(shared)
    _replays_match(lambda: mx.moe_swiglu(x, gu_p, gu_s, dn_p, dn_s, sel, p, shared, out=out, workspace=ws), out,
                   lambda: mx.moe_swiglu(x, gu_p, gu_s, dn_p, dn_s, sel, p * 2, shared, out=other))


@pytest.mark.parametrize("prepared", [False, True])
def test_graph_block_scaled_variant(prepared):
    say(f"graph: moe_linear_mxfp8 prepared={prepared}")
    x, packed, scales, sel, p, shared = _case(3, 200, 8, 4, 9, 520)
    ws = torch.empty(mx.mxfp8_workspace_size(200, 8, 520, 9, 4), dtype=torch.uint8, device=DEV)
    out = torch.empty_like(shared)
    other = torch.empty_like(shared)
    if prepared:
        prep = mx.prepare_mx(packed, scales)
        call = lambda: mx.moe_linear_mxfp8_prepared(x, prep, sel, p, shared, out=out, workspace=ws)  # noqa: E731
        disturb = lambda: mx.moe_linear_mxfp8_prepared(x, prep, sel, p, shared, out=other)  # noqa: E731
    else:
        call = lambda: mx.moe_linear_mxfp8(x, packed, scales, sel, p, shared, out=out, workspace=ws)  # noqa: E731
        disturb = lambda: mx.moe_linear_mxfp8(x, packed, scales, sel, p, shared, out=other)  # noqa: E731
    _replays_match(call, out, disturb)


def test_graph_prepared_bf16():
    say("graph: moe_linear_prepared")
    x, packed, scales, sel, p, shared = _case(4, 300, 8, 4, 9, 1040)
    prep = mx.prepare_bf16(packed, scales)
    ws = torch.empty(mx.workspace_size(300, 8, 1040, 9, 4, mx.DTYPE_BF16, mx.FLAG_FORCE_GEMM), dtype=torch.uint8,
                     device=DEV)
    out = torch.empty_like(shared)
    other = torch.empty_like(shared)
    _replays_match(lambda: mx.moe_linear_prepared(x, prep, sel, p, shared, out=out, workspace=ws), out,
                   lambda: mx.moe_linear_prepared(x, prep, sel.flip(1).contiguous(), p, shared, out=other))


def test_graph_decode_prepared():
    say("graph: moe_decode_prepared (fp32)")
    rng = np.random.default_rng(6)
    T, E, K, G, O = 3, 16, 4, 9, 264
    x = torch.from_numpy(rng.standard_normal((T, 32 * G)).astype(np.float32)).to(DEV)
    shared = torch.from_numpy(rng.standard_normal((T, O)).astype(np.float32)).to(DEV)
    packed = torch.from_numpy(rng.integers(0, 256, (E, O, G, 16), dtype=np.uint8)).to(DEV)
    scales = torch.from_numpy(rng.integers(118, 131, (E, O, G), dtype=np.uint8)).to(DEV)
    sel = torch.from_numpy(np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)).to(DEV)
    p = torch.from_numpy(rng.random((T, K)).astype(np.float32)).to(DEV)
    prep = mx.prepare_mx(packed, scales)
    ws = torch.empty(mx.workspace_size(T, E, O, G, K, mx.DTYPE_F32, mx.FLAG_FORCE_GEMV), dtype=torch.uint8,
                     device=DEV)
    out = torch.empty_like(shared)
    other = torch.empty_like(shared)
    _replays_match(lambda: mx.moe_decode_prepared(x, prep, sel, p, shared, out=out, workspace=ws), out,
                   lambda: mx.moe_decode_prepared(x, prep, sel.flip(1).contiguous(), p, shared, out=other))


def test_graph_swiglu_prepared():
    say("graph: moe_swiglu_prepared")
    rng = np.random.default_rng(7)
    T, E, K, G, F, O = 70, 6, 2, 4, 64, 96
    x = bf16(workloads.round_to_bf16(rng.standard_normal((T, 32 * G)).astype(np.float32)))
    shared = bf16(workloads.round_to_bf16(rng.standard_normal((T, O)).astype(np.float32)))
    dv = lambda a: torch.from_numpy(a).to(DEV)  # noqa: E731
    prep = mx.prepare_swiglu(dv(rng.integers(0, 256, (E, 2 * F, G, 16), dtype=np.uint8)),
                             dv(rng.integers(118, 127, (E, 2 * F, G), dtype=np.uint8)),
                             dv(rng.integers(0, 256, (E, O, F // 32, 16), dtype=np.uint8)),
                             dv(rng.integers(118, 127, (E, O, F // 32), dtype=np.uint8)))
    sel = dv(np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32))
    p = dv(rng.random((T, K)).astype(np.float32))
    ws = torch.empty(mx.swiglu_workspace_size(T, E, F, G, O, K), dtype=torch.uint8, device=DEV)
    out = torch.empty_like(shared)
    other = torch.empty_like(shared)
    _replays_match(lambda: mx.moe_swiglu_prepared(x, prep, sel, p, shared, out=out, workspace=ws), out,
                   lambda: mx.moe_swiglu_prepared(x, prep, sel, p * 2, shared, out=other))


def test_graph_router():
    say("graph: route")
    logits, bias = workloads.router_logits(700, 96, seed=5, bias_std=0.1)
    lg = torch.from_numpy(logits).to(DEV)
    b = torch.from_numpy(bias).to(DEV)
    sel = torch.empty((700, 6), dtype=torch.int32, device=DEV)
    p = torch.empty((700, 6), dtype=torch.float32, device=DEV)
    sel2, p2 = torch.empty_like(sel), torch.empty_like(p)
    _replays_match(lambda: mx.route(lg, 6, "sigmoid", b, 1.0, sel=sel, p=p), p,
                   lambda: mx.route(lg * 2, 6, "softmax", None, 1.0, sel=sel2, p=p2))
