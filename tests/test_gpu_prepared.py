"""GPU parity of the bf16 routed linear on prepared weights
(mxfp4_moe_linear_prepared_ex and mxfp4_moe_gemm_stage_prepared, through
their C ABI) against the float64 oracle.

Bar (written in each check): relative L2 <= 1e-2 against oracle.expert_linear
on the same bf16 inputs - the bf16 bar - and every output within
1e-2 * (|y_ref| + rms(y_ref)); what remains is the bf16 output rounding (the
decoded weights are exact in bf16, the products exact in fp32, the sums
fp32).
"""

import sys

import numpy as np
import pytest

import oracle
import workloads

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU-only machines, never run there
    pytest.skip("no GPU", allow_module_level=True)

import mxfp4_block_scaled_amd as mx  # noqa: E402
from mxfp4_block_scaled_amd import _abi  # noqa: E402

DEV = torch.device("cuda:0")
BF16_REL_L2 = 1e-2


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def rel_l2(y, ref):
    return float(np.linalg.norm(y - ref) / max(np.linalg.norm(ref), 1e-300))


def bf16_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV).to(torch.bfloat16)


def host64(y):
    return y.float().cpu().numpy().astype(np.float64)


def case(seed, T, E, K, G, O, scale_lo=118, scale_hi=130, distinct=True, empty_experts=()):
    rng = np.random.default_rng(seed)
    x = workloads.round_to_bf16(rng.standard_normal((T, 32 * G)).astype(np.float32))
    shared = workloads.round_to_bf16(rng.standard_normal((T, O)).astype(np.float32))
    packed = rng.integers(0, 256, (E, O, G, 16), dtype=np.uint8)
    scales = rng.integers(scale_lo, scale_hi + 1, (E, O, G), dtype=np.uint8)
    pool = [e for e in range(E) if e not in empty_experts]
    if distinct:
        sel = np.stack([rng.permutation(pool)[:K] for _ in range(T)]).astype(np.int32)
    else:
        sel = rng.choice(pool, (T, K)).astype(np.int32)
    p = rng.random((T, K)).astype(np.float32)
    return x, packed, scales, sel, p, shared


def run_case(x, packed, scales, sel, p, shared, out=None):
    prep = mx.prepare_bf16(torch.from_numpy(packed).to(DEV), torch.from_numpy(scales).to(DEV))
    y = mx.moe_linear_prepared(bf16_dev(x), prep, torch.from_numpy(sel).to(DEV), torch.from_numpy(p).to(DEV),
                               bf16_dev(shared), out=out)
    torch.cuda.synchronize()
    return y


BF16_ELEM = 1e-2


def check(y, ref, what):
    yh = host64(y) if isinstance(y, torch.Tensor) else y
    r = rel_l2(yh, ref)
    err = np.abs(yh - ref)
    bound = BF16_ELEM * (np.abs(ref) + float(np.sqrt(np.mean(ref * ref))))
    worst = float(np.max(err / np.maximum(bound, 1e-300)))
    say(f"  {what}: rel L2 {r:.3e}, max err/elementwise bound {worst:.3f}")
    assert np.all(np.isfinite(yh))
    assert r <= BF16_REL_L2, f"{what}: relative L2 {r:.3e}"
    assert np.all(err <= bound), f"{what}: an output misses the elementwise bound by {worst:.3g}x"


def tile_rows(O, n, seed, extra=()):
    """n random rows, the given ones, and one random row in every 128-row
    tile (so every prepared tile and every 512-row N-tile is read)."""
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(O, min(n, O), replace=False).tolist()) | {r for r in extra if 0 <= r < O}
    rows.update(int(rng.integers(t, min(t + 128, O))) for t in range(0, O, 128))
    return np.array(sorted(rows))


CASES = [  # seed, T, E, K, G, O
    (1, 1, 4, 2, 4, 128),       # one chunk of 128 inputs, one 128-row tile
    (2, 5, 3, 2, 1, 40),        # G = 1, O not a multiple of 16 or 128
    (3, 37, 8, 3, 6, 256),      # a 2-group last chunk
    (4, 130, 4, 2, 9, 132),     # M-tiles past 128 rows, a 4-row last tile
    (5, 300, 16, 4, 90, 200),   # the prefill input width (a half chunk at the end)
    (6, 150, 2, 2, 7, 1028),    # three 512-row N-tiles, the last with 4 rows; tiles of 128 and 22 pairs
    (7, 70, 1, 1, 5, 520),      # 70 pairs: the second half of the waves holds 6
]


@pytest.mark.parametrize("c", CASES, ids=[f"T{c[1]}E{c[2]}K{c[3]}G{c[4]}O{c[5]}" for c in CASES])
def test_prepared_against_oracle(c):
    args = case(*c)
    say(f"prepared bf16 case {c}")
    check(run_case(*args), oracle.expert_linear(*args), f"case {c}")


def test_prepared_edges():
    # duplicate experts in a token, experts nobody picks, K = 1
    args = case(8, 50, 6, 3, 3, 64, distinct=False, empty_experts=(1, 4))
    check(run_case(*args), oracle.expert_linear(*args), "duplicates and empty experts")
    args = case(9, 9, 5, 1, 5, 36)
    check(run_case(*args), oracle.expert_linear(*args), "K = 1")
    # every token on one expert: 5 full M-tiles and a ragged one
    x, packed, scales, sel, p, shared = case(10, 700, 3, 1, 4, 64)
    sel[:] = 2
    args = (x, packed, scales, sel, p, shared)
    check(run_case(*args), oracle.expert_linear(*args), "one hot expert")
    # in place: out = shared
    x, packed, scales, sel, p, shared = case(11, 12, 4, 2, 2, 48)
    prep = mx.prepare_bf16(torch.from_numpy(packed).to(DEV), torch.from_numpy(scales).to(DEV))
    sh = bf16_dev(shared)
    y = mx.moe_linear_prepared(bf16_dev(x), prep, torch.from_numpy(sel).to(DEV), torch.from_numpy(p).to(DEV), sh,
                               out=sh)
    torch.cuda.synchronize()
    assert y.data_ptr() == sh.data_ptr()
    check(y, oracle.expert_linear(x, packed, scales, sel, p, shared), "in place")


def test_prepared_largest_scales_with_finite_weights():
    """Scale bytes 253..255 with codes small enough that every decoded weight
    is a finite bf16 value (|E2M1| <= 1.5 at 253/254, <= 0.5 at 255): the
    shifted decode of such tiles is checked against the float64 oracle."""
    T, E, K, G, O = 20, 3, 2, 37, 72
    x, packed, scales, sel, p, shared = case(12, T, E, K, G, O)
    x = workloads.round_to_bf16((x * np.float32(2.0 ** -110)).astype(np.float32))
    rng = np.random.default_rng(13)
    scales = rng.integers(253, 256, scales.shape).astype(np.uint8)
    small = np.array([0, 1, 8, 9], np.uint8)              # 0, 0.5, -0, -0.5
    mid = np.array([0, 1, 2, 3, 8, 9, 10, 11], np.uint8)  # |E2M1| <= 1.5
    lo255, hi255 = rng.choice(small, packed.shape), rng.choice(small, packed.shape)
    lo, hi = rng.choice(mid, packed.shape), rng.choice(mid, packed.shape)
    is255 = (scales == 255)[..., None]
    packed = np.where(is255, lo255 | (hi255 << 4), lo | (hi << 4)).astype(np.uint8)
    ref = oracle.expert_linear(x, packed, scales, sel, p, shared)
    assert np.all(np.isfinite(ref))
    check(run_case(x, packed, scales, sel, p, shared), ref, "scales 253..255, finite weights")


def test_prepared_largest_scales_against_oracle():
    """Scale bytes 250..255 with every code: decoded weights from 2^126 up
    leave the bf16 range, the layer's value does not (tiny activations). The
    prepared GEMM and the canonical GEMM both match the exact result."""
    T, E, K, G, O = 24, 3, 2, 37, 132
    x, packed, scales, sel, p, shared = case(14, T, E, K, G, O)
    x = workloads.round_to_bf16((x * np.float32(2.0 ** -100)).astype(np.float32))
    scales = np.random.default_rng(15).integers(250, 256, scales.shape).astype(np.uint8)
    scales[:, 3, :] = 255   # a whole row at 2^128
    args = (x, packed, scales, sel, p, shared)
    ref = oracle.expert_linear(*args)
    assert np.all(np.isfinite(ref)) and np.abs(ref).max() > 1e6
    check(run_case(*args), ref, "prepared, scales 250..255")
    d = [torch.from_numpy(a).to(DEV) for a in (packed, scales, sel, p)]
    y_can = mx.moe_linear(bf16_dev(x), d[0], d[1], d[2], d[3], bf16_dev(shared), flags=_abi.FLAG_FORCE_GEMM)
    torch.cuda.synchronize()
    check(y_can, ref, "canonical GEMM, scales 250..255")


def test_prepared_deterministic_and_gemm_stage():
    args = case(15, 64, 8, 4, 8, 96)
    x, packed, scales, sel, p, shared = args
    prep = mx.prepare_bf16(torch.from_numpy(packed).to(DEV), torch.from_numpy(scales).to(DEV))
    xd, seld, pd, shd = bf16_dev(x), torch.from_numpy(sel).to(DEV), torch.from_numpy(p).to(DEV), bf16_dev(shared)
    ws = torch.empty(mx.workspace_size(64, 8, 96, 8, 4, mx.DTYPE_BF16, mx.FLAG_FORCE_GEMM), dtype=torch.uint8,
                     device=DEV)
    y1 = mx.moe_linear_prepared(xd, prep, seld, pd, shd, workspace=ws)
    torch.cuda.synchronize()
    part = ws.clone()
    mx.gemm_stage_prepared(xd, prep, 4, ws)  # the GEMM alone, again, on the same bucketing
    torch.cuda.synchronize()
    assert torch.equal(ws, part)
    y2 = mx.moe_linear_prepared(xd, prep, seld, pd, shd)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    check(y1, oracle.expert_linear(*args), "deterministic")


@pytest.mark.parametrize("name,nrows", [("prefill", 48), ("skewed", 40)])
def test_prepared_full_workloads_sampled_rows(name, nrows):
    inp = workloads.make_inputs(name, n_routing_sets=1)
    w = inp.workload
    say(f"prepared bf16 at {name}: T={w.T} E={w.E} K={w.K} G={w.G} O={w.O}")
    pk = torch.empty(inp.packed.shape, dtype=torch.uint8, device=DEV)
    sc = torch.empty(inp.scales.shape, dtype=torch.uint8, device=DEV)
    for e in range(w.E):  # the expert tensors are drawn expert by expert
        pk[e].copy_(torch.from_numpy(np.ascontiguousarray(inp.packed[e])))
        sc[e].copy_(torch.from_numpy(np.ascontiguousarray(inp.scales[e])))
    prep = mx.prepare_bf16(pk, sc)
    del pk, sc
    y = mx.moe_linear_prepared(bf16_dev(inp.x), prep, torch.from_numpy(inp.sel).to(DEV),
                               torch.from_numpy(inp.p).to(DEV), bf16_dev(inp.shared))
    torch.cuda.synchronize()
    rows = tile_rows(w.O, nrows, 7, (0, 127, 128, 511, 512, w.O - 1))
    ref = oracle.expert_linear_rows(inp.x, inp.packed, inp.scales, inp.sel, inp.p, inp.shared, rows)
    check(y[:, torch.from_numpy(rows).to(DEV)], ref, name)
    assert torch.isfinite(y.float()).all()


def test_prepared_rejects_unsupported_and_empty():
    x, packed, scales, sel, p, shared = case(16, 3, 2, 1, 2, 34)  # O % 4 != 0: no prepared layout
    with pytest.raises(mx.Mxfp4Error):
        mx.prepare_bf16(torch.from_numpy(packed).to(DEV), torch.from_numpy(scales).to(DEV))
    x, packed, scales, sel, p, shared = case(17, 3, 2, 1, 2, 32)
    prep = mx.prepare_bf16(torch.from_numpy(packed).to(DEV), torch.from_numpy(scales).to(DEV))
    y = mx.moe_linear_prepared(bf16_dev(x[:0]), prep, torch.from_numpy(sel[:0]).to(DEV),
                               torch.from_numpy(p[:0]).to(DEV), bf16_dev(shared[:0]))
    assert tuple(y.shape) == (0, 32)


# ------------------------------------------------------------------ SwiGLU block on prepared weights

def swiglu_case(seed, T, E, K, G, F, O, scale_lo=118, scale_hi=126, distinct=True):
    rng = np.random.default_rng(seed)
    x = workloads.round_to_bf16(rng.standard_normal((T, 32 * G)).astype(np.float32))
    shared = workloads.round_to_bf16(rng.standard_normal((T, O)).astype(np.float32))
    gu_p = rng.integers(0, 256, (E, 2 * F, G, 16), dtype=np.uint8)
    gu_s = rng.integers(scale_lo, scale_hi + 1, (E, 2 * F, G), dtype=np.uint8)
    dn_p = rng.integers(0, 256, (E, O, F // 32, 16), dtype=np.uint8)
    dn_s = rng.integers(scale_lo, scale_hi + 1, (E, O, F // 32), dtype=np.uint8)
    if distinct:
        sel = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    else:
        sel = rng.integers(0, E, (T, K)).astype(np.int32)
    p = rng.random((T, K)).astype(np.float32)
    return x, gu_p, gu_s, dn_p, dn_s, sel, p, shared


def run_swiglu_prepared(x, gu_p, gu_s, dn_p, dn_s, sel, p, shared):
    dv = lambda a: torch.from_numpy(a).to(DEV)  # noqa: E731
    prep = mx.prepare_swiglu(dv(gu_p), dv(gu_s), dv(dn_p), dv(dn_s))
    y = mx.moe_swiglu_prepared(bf16_dev(x), prep, dv(sel), dv(p), bf16_dev(shared))
    torch.cuda.synchronize()
    return y


SWIGLU_CASES = [  # T, E, K, G, F, O, distinct
    (1, 3, 1, 1, 32, 8, True),         # F = 32: half of one prepared gate/up tile
    (5, 4, 2, 2, 64, 40, True),
    (33, 6, 3, 3, 96, 132, True),      # F = 1.5 prepared tiles, a 4-row last down tile
    (70, 16, 4, 5, 160, 72, True),     # several M-tiles, odd G
    (40, 3, 2, 17, 64, 36, False),     # duplicates within a token
    (300, 8, 4, 4, 544, 520, True),    # three 512-row gate/up N-tiles (2F = 1088), two down N-tiles
]


@pytest.mark.parametrize("c", SWIGLU_CASES, ids=lambda c: "T{}E{}K{}G{}F{}O{}{}".format(*c[:6], "" if c[6] else "dup"))
def test_swiglu_prepared_against_oracle(c):
    T, E, K, G, F, O, distinct = c
    say(f"swiglu prepared {c}")
    host = swiglu_case(sum(c[:6]), T, E, K, G, F, O, distinct=distinct)
    check(run_swiglu_prepared(*host), oracle.expert_swiglu(*host), f"swiglu prepared {c}")


def test_swiglu_prepared_matches_canonical_and_ignores_unselected():
    host = list(swiglu_case(21, 48, 10, 3, 3, 96, 64))
    x, gu_p, gu_s, dn_p, dn_s, sel, p, shared = host
    y = run_swiglu_prepared(*host)
    assert torch.equal(y, run_swiglu_prepared(*host)), "not deterministic"
    dv = lambda a: torch.from_numpy(a).to(DEV)  # noqa: E731
    y_can = mx.moe_swiglu(bf16_dev(x), dv(gu_p), dv(gu_s), dv(dn_p), dv(dn_s), dv(sel), dv(p), bf16_dev(shared))
    torch.cuda.synchronize()
    assert rel_l2(host64(y), host64(y_can)) <= BF16_REL_L2
    rng = np.random.default_rng(22)
    gu2, dn2, gs2, ds2 = gu_p.copy(), dn_p.copy(), gu_s.copy(), dn_s.copy()
    for e in set(range(10)) - set(np.unique(sel).tolist()):
        gu2[e] = rng.integers(0, 256, gu2[e].shape)
        dn2[e] = rng.integers(0, 256, dn2[e].shape)
        gs2[e] = 255
        ds2[e] = 255
    assert torch.equal(run_swiglu_prepared(x, gu2, gs2, dn2, ds2, sel, p, shared), y)


@pytest.mark.parametrize("which", ["gate_up", "down"])
def test_swiglu_largest_scales_against_oracle(which):
    """Scale bytes 250..255 on one of the two projections (tiny activations,
    resp. a tiny hidden vector, keep the block's value finite): the canonical
    and the prepared block both match the exact result."""
    T, E, K, G, F, O = 40, 4, 2, 3, 96, 64
    x, gu_p, gu_s, dn_p, dn_s, sel, p, shared = swiglu_case(23, T, E, K, G, F, O)
    rng = np.random.default_rng(24)
    if which == "gate_up":
        x = workloads.round_to_bf16((x * np.float32(2.0 ** -110)).astype(np.float32))
        gu_s = rng.integers(250, 256, gu_s.shape).astype(np.uint8)
    else:
        x = workloads.round_to_bf16((x * np.float32(2.0 ** -60)).astype(np.float32))
        dn_s = rng.integers(250, 256, dn_s.shape).astype(np.uint8)
    host = (x, gu_p, gu_s, dn_p, dn_s, sel, p, shared)
    ref = oracle.expert_swiglu(*host)
    assert np.all(np.isfinite(ref))
    check(run_swiglu_prepared(*host), ref, f"swiglu prepared, large {which} scales")
    dv = lambda a: torch.from_numpy(a).to(DEV)  # noqa: E731
    y_can = mx.moe_swiglu(bf16_dev(x), dv(gu_p), dv(gu_s), dv(dn_p), dv(dn_s), dv(sel), dv(p), bf16_dev(shared))
    torch.cuda.synchronize()
    check(y_can, ref, f"swiglu canonical, large {which} scales")


def test_swiglu_prepared_large_shape_sampled():
    """The gate/up shape of the SwiGLU workload (I = 7168, 2F = 4096, O = 7168)
    with 16 experts and 512 tokens (128 pairs per expert, several M-tiles);
    the oracle checks two tokens on a sample of output rows."""
    T, E, K, G, F, O = 512, 16, 4, 224, 2048, 7168
    host = swiglu_case(2027, T, E, K, G, F, O)
    x, gu_p, gu_s, dn_p, dn_s, sel, p, shared = host
    y = host64(run_swiglu_prepared(*host))
    toks = np.array([0, 311])
    rows = np.sort(np.random.default_rng(3).choice(O, 64, replace=False))
    ref = oracle.expert_swiglu_rows(x[toks], gu_p, gu_s, dn_p, dn_s, sel[toks], p[toks], shared[toks], rows)
    r = rel_l2(y[np.ix_(toks, rows)], ref)
    say(f"  swiglu prepared large: rel L2 {r:.3e}")
    assert r <= BF16_REL_L2
    assert np.all(np.isfinite(y))


def _interleaved_layout_numpy(packed, scales):
    """prepare_bf16's documented layout, built with numpy: slot (e, n, q, f, l)
    holds group 4q + l // 16 of row 128n + 16f + l % 16 (zeros past O / G);
    its dword s sits at byte ((((e, n, q) * 2 + f // 4) * 4 + s) * 64 + l) * 16
    + 4 (f % 4) of the codes, its scale byte at (((e, n, q) * 2 + f // 4) * 64
    + l) * 4 + f % 4 of the scale array that follows."""
    E, O, G, _ = packed.shape
    NT, NQ = -(-O // 128), -(-(32 * G) // 128)
    e, n, q, f, l = np.meshgrid(np.arange(E), np.arange(NT), np.arange(NQ), np.arange(8), np.arange(64), indexing="ij")
    row = 128 * n + 16 * f + l % 16
    g = 4 * q + l // 16
    ok = (row < O) & (g < G)
    codes = np.zeros(e.shape + (16,), np.uint8)
    sc = np.zeros(e.shape, np.uint8)
    codes[ok] = packed[e[ok], row[ok], g[ok]]
    sc[ok] = scales[e[ok], row[ok], g[ok]]
    # (e, n, q, half, f % 4, l, s, byte) -> (e, n, q, half, s, l, f % 4, byte)
    codes = codes.reshape(E, NT, NQ, 2, 4, 64, 4, 4).transpose(0, 1, 2, 3, 6, 5, 4, 7)
    sc = sc.reshape(E, NT, NQ, 2, 4, 64).transpose(0, 1, 2, 3, 5, 4)
    return np.concatenate([codes.reshape(-1), sc.reshape(-1)])


@pytest.mark.parametrize("E,O,G", [(2, 40, 1), (3, 132, 9), (2, 256, 6)])
def test_prepare_bf16_layout_bytes(E, O, G):
    rng = np.random.default_rng(E * O + G + 1)
    packed = rng.integers(0, 256, (E, O, G, 16), dtype=np.uint8)
    scales = rng.integers(0, 255, (E, O, G), dtype=np.uint8)
    prep = mx.prepare_bf16(torch.from_numpy(packed).to(DEV), torch.from_numpy(scales).to(DEV))
    torch.cuda.synchronize()
    assert np.array_equal(prep.buf.cpu().numpy(), _interleaved_layout_numpy(packed, scales))
    # the two orders are different permutations of the same slots
    other = mx.prepare_mx(torch.from_numpy(packed).to(DEV), torch.from_numpy(scales).to(DEV))
    torch.cuda.synchronize()
    a, b = prep.buf.cpu().numpy(), other.buf.cpu().numpy()
    assert np.array_equal(np.sort(a), np.sort(b)) and (G * O < 16 or not np.array_equal(a, b))
    with pytest.raises(ValueError):  # the fragment-major order is refused by the bf16 path
        mx.moe_linear_prepared(bf16_dev(np.zeros((1, 32 * G))), other, torch.zeros((1, 1), dtype=torch.int32, device=DEV),
                               torch.ones((1, 1), dtype=torch.float32, device=DEV), bf16_dev(np.zeros((1, O))))


# ------------------------------------------------------------------ decode-shaped path on prepared weights

F32_TOL = 1e-4


def _decode_both(x, packed, scales, sel, p, shared, dtype):
    """(prepared, canonical MFMA decode kernel) results on the same inputs."""
    td = torch.float32 if dtype == "fp32" else torch.bfloat16
    dv = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)  # noqa: E731
    xd = dv(x.astype(np.float32)).to(td)
    shd = dv(shared.astype(np.float32)).to(td)
    pk, sc = dv(packed), dv(scales)
    prep = mx.prepare_mx(pk, sc)
    y_p = mx.moe_decode_prepared(xd, prep, dv(sel), dv(p), shd)
    y_c = mx.moe_linear(xd, pk, sc, dv(sel), dv(p), shd, flags=_abi.FLAG_FORCE_GEMV | _abi.FLAG_GEMV_MFMA)
    torch.cuda.synchronize()
    return y_p, y_c


def _check_decode(y, ref, dtype, what):
    yh = host64(y)
    if dtype == "fp32":
        err = np.abs(yh - ref)
        bound = F32_TOL * (1.0 + np.abs(ref))
        say(f"  {what}: max err/bound {np.max(err / bound):.3g}")
        assert np.all(err <= bound), what
    else:
        check(y, ref, what)


DECODE_CASES = [  # seed, T, E, K, G, O, dtype, distinct
    (1, 4, 4, 2, 2, 32, "fp32", True),      # the tiny workload's shape
    (2, 1, 128, 4, 90, 5760, "fp32", True),  # the decode workload's shape (fewer experts drawn)
    (3, 8, 24, 8, 37, 264, "bf16", True),   # odd G, a partial last 128-row tile
    (4, 5, 6, 4, 2, 16, "bf16", False),     # duplicates within a token
    (5, 40, 9, 3, 5, 132, "fp32", True),    # 120 pairs: several token chunks
    (6, 3, 3, 3, 9, 1028, "bf16", True),    # every expert in every token, 65 row blocks (a remapped group of 32 and a tail)
]


@pytest.mark.parametrize("c", DECODE_CASES, ids=lambda c: "T{}E{}K{}G{}O{}{}{}".format(*c[1:7], "" if c[7] else "dup"))
def test_decode_prepared_against_oracle_and_canonical(c):
    seed, T, E, K, G, O, dtype, distinct = c
    say(f"decode prepared {c}")
    x, packed, scales, sel, p, shared = case(seed, T, E, K, G, O, distinct=distinct)
    if dtype == "fp32":
        rng = np.random.default_rng(seed + 100)
        x = rng.standard_normal(x.shape).astype(np.float32)
        shared = rng.standard_normal(shared.shape).astype(np.float32)
    y_p, y_c = _decode_both(x, packed, scales, sel, p, shared, dtype)
    # the same MFMA sequence on the same operands: bit for bit the canonical kernel's result
    assert torch.equal(y_p, y_c), "differs from the canonical MFMA decode kernel"
    _check_decode(y_p, oracle.expert_linear(x, packed, scales, sel, p, shared), dtype, f"decode prepared {c}")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_decode_prepared_largest_scales(dtype):
    """Scale bytes 253..255 (the kernels' 2^-8 second accumulator) with
    tiny activations: finite results equal to the float64 oracle's."""
    T, E, K, G, O = 3, 4, 2, 9, 72
    x, packed, scales, sel, p, shared = case(31, T, E, K, G, O)
    # small but well inside the normal range, so that the three-piece bf16 split of fp32 x stays exact
    x = (np.random.default_rng(32).standard_normal(x.shape) * 2.0 ** -100).astype(np.float32)
    if dtype == "bf16":
        x = workloads.round_to_bf16(x)
    scales = np.random.default_rng(33).integers(253, 256, scales.shape).astype(np.uint8)
    y_p, y_c = _decode_both(x, packed, scales, sel, p, shared, dtype)
    assert torch.equal(y_p, y_c)
    ref = oracle.expert_linear(x, packed, scales, sel, p, shared)
    assert np.all(np.isfinite(ref)) and np.all(np.isfinite(host64(y_p)))
    _check_decode(y_p, ref, dtype, f"decode prepared scales 253..255 {dtype}")


def test_decode_prepared_decode8_workload_sampled():
    inp = workloads.make_inputs("decode8", n_routing_sets=1)
    w = inp.workload
    say(f"decode prepared at decode8: T={w.T} E={w.E} K={w.K} G={w.G} O={w.O}")
    pk = torch.empty(inp.packed.shape, dtype=torch.uint8, device=DEV)
    sc = torch.empty(inp.scales.shape, dtype=torch.uint8, device=DEV)
    for e in range(w.E):
        pk[e].copy_(torch.from_numpy(np.ascontiguousarray(inp.packed[e])))
        sc[e].copy_(torch.from_numpy(np.ascontiguousarray(inp.scales[e])))
    prep = mx.prepare_mx(pk, sc)
    y = mx.moe_decode_prepared(bf16_dev(inp.x), prep, torch.from_numpy(inp.sel).to(DEV),
                               torch.from_numpy(inp.p).to(DEV), bf16_dev(inp.shared))
    torch.cuda.synchronize()
    rows = np.array(sorted(set(np.random.default_rng(8).choice(w.O, 96, replace=False).tolist()) | {0, w.O - 1}))
    ref = oracle.expert_linear_rows(inp.x, inp.packed, inp.scales, inp.sel, inp.p, inp.shared, rows)
    check(y[:, torch.from_numpy(rows).to(DEV)], ref, "decode8 prepared")
