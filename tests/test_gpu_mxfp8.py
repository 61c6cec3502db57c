"""GPU parity of the block-scaled variant (MXFP8 activations on the scaled
MFMA) through its C ABI, against the float64 oracle.

Bars (written in each check):
* quantised activations (codes and scale bytes): bit-exact against
  oracle.quantize_mxfp8;
* the layer: relative L2 <= 1e-2 against the variant's own definition,
  oracle.expert_linear_mxfp8 (the routed linear of the dequantised MXFP8
  activations, exact in float64) - the bf16 bar; what remains is the bf16
  output rounding and the MFMA's internal alignment of products;
* the error of the variant against the exact layer (oracle.expert_linear,
  unquantised activations) is the activation rounding: printed, and checked
  only to stay below 5e-2 relative L2.
"""

import functools
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
VS_EXACT_REL_L2 = 5e-2


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def rel_l2(y, ref):
    return float(np.linalg.norm(y - ref) / max(np.linalg.norm(ref), 1e-300))


def bf16_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV).to(torch.bfloat16)


def host64(y):
    return y.float().cpu().numpy().astype(np.float64)


# ------------------------------------------------------------------ quantisation

def _special_activations(T, I, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, I)) * np.ldexp(1.0, rng.integers(-30, 30, (T, 1)))
    x[0, :32] = 0.0                                   # an all-zero block
    x[1 % T, :32] = np.linspace(-448.0, 448.0, 32)    # fits at scale byte 127 exactly
    if I >= 64:
        x[0, 32:64] = -0.0                            # negative zeros
        x[1 % T, 32:64] = 3.0e38 * np.sign(rng.standard_normal(32))  # the largest bf16 magnitudes
    if T > 2 and I >= 64:
        x[2, :32] = np.ldexp(1.0, -133) * rng.integers(-3, 4, 32)  # bf16 subnormals
        x[2, 32:64] = rng.standard_normal(32) * 1e-3
        x[2, 40] = 1e3                                # one large value: the rest rounds to few bits
    return workloads.round_to_bf16(x.astype(np.float32))


@pytest.mark.parametrize("T,I,ld", [(1, 32, 32), (3, 64, 128), (17, 2880, 2944), (64, 7168, 7168), (5, 96, 96)])
def test_quantize_bit_exact(T, I, ld):
    say(f"quantize T={T} I={I} ld={ld}")
    x = _special_activations(T, I, seed=T + I)
    codes, sb = mx.quantize_mxfp8(bf16_dev(x), ld)
    torch.cuda.synchronize()
    codes, sb = codes.cpu().numpy(), sb.cpu().numpy()
    want_c, want_s = oracle.quantize_mxfp8(x.astype(np.float64))
    assert np.array_equal(codes[:, :I], want_c)
    assert np.array_equal(sb[:, :I // 32], want_s)
    assert np.all(codes[:, I:] == 0) and np.all(sb[:, I // 32:] == 0)


def test_quantize_every_bf16_value():
    """Every finite bf16 value once (both signs), in blocks of neighbours
    (similar magnitudes) and again shuffled (mixed magnitudes: many values
    far below their block's maximum)."""
    pats = np.arange(0, 0x7F80, dtype=np.uint32)  # +0 .. largest finite positive
    vals = (pats << 16).view(np.float32)
    vals = np.concatenate([vals, -vals])           # 65280 values = 1020 rows of 64
    rng = np.random.default_rng(12)
    for name, arr in (("neighbours", vals), ("shuffled", rng.permutation(vals))):
        x = np.ascontiguousarray(arr.reshape(-1, 64))
        say(f"quantize every bf16 value, {name}: {x.shape[0]} rows")
        codes, sb = mx.quantize_mxfp8(bf16_dev(x))
        torch.cuda.synchronize()
        want_c, want_s = oracle.quantize_mxfp8(x.astype(np.float64))
        assert np.array_equal(codes.cpu().numpy(), want_c), name
        assert np.array_equal(sb.cpu().numpy(), want_s), name


# ------------------------------------------------------------------ the layer

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
    y = mx.moe_linear_mxfp8(bf16_dev(x), torch.from_numpy(packed).to(DEV), torch.from_numpy(scales).to(DEV),
                            torch.from_numpy(sel).to(DEV), torch.from_numpy(p).to(DEV), bf16_dev(shared), out=out)
    torch.cuda.synchronize()
    return y


def check_layer(y, args, what):
    ref = oracle.expert_linear_mxfp8(*args)
    exact = oracle.expert_linear(*args)
    yh = host64(y)
    r = rel_l2(yh, ref)
    # compare the routed parts: the shared rows are common to all three
    sh = args[5]
    rq = rel_l2(ref - sh, exact - sh)
    say(f"  {what}: rel L2 vs variant oracle {r:.3e}; variant vs exact layer (routed part) {rq:.3e}")
    assert r <= BF16_REL_L2, f"{what}: {r:.3e}"
    assert rq <= VS_EXACT_REL_L2, f"{what}: variant error {rq:.3e}"
    assert np.all(np.isfinite(yh))


CASES = [  # seed, T, E, K, G, O
    (1, 1, 4, 2, 4, 128),      # one chunk of 128 inputs
    (2, 5, 3, 2, 1, 40),       # G = 1: a single group, O not a multiple of 16
    (3, 37, 8, 3, 6, 256),     # a partial chunk (6 groups), two N-tiles
    (4, 130, 4, 2, 9, 132),    # M-tiles past 128 rows, a ragged N-tile
    (5, 300, 16, 4, 90, 200),  # the prefill input width (90 groups: a half chunk at the end)
]


@pytest.mark.parametrize("c", CASES, ids=[f"T{c[1]}E{c[2]}K{c[3]}G{c[4]}O{c[5]}" for c in CASES])
def test_variant_against_oracle(c):
    args = case(*c)
    say(f"mxfp8 variant case {c}")
    check_layer(run_case(*args), args, f"case {c}")


def test_variant_edges():
    # duplicate experts in a token, experts nobody picks, K = 1
    args = case(6, 50, 6, 3, 3, 64, distinct=False, empty_experts=(1, 4))
    check_layer(run_case(*args), args, "duplicates and empty experts")
    args = case(7, 9, 5, 1, 5, 36)
    check_layer(run_case(*args), args, "K = 1")
    # every token on one expert: 5 full M-tiles and a ragged one
    x, packed, scales, sel, p, shared = case(8, 700, 3, 1, 4, 64)
    sel[:] = 2
    check_layer(run_case(x, packed, scales, sel, p, shared), (x, packed, scales, sel, p, shared), "one hot expert")
    # in place: out = shared
    args = case(9, 12, 4, 2, 2, 48)
    sh = bf16_dev(args[5])
    y = mx.moe_linear_mxfp8(bf16_dev(args[0]), torch.from_numpy(args[1]).to(DEV), torch.from_numpy(args[2]).to(DEV),
                            torch.from_numpy(args[3]).to(DEV), torch.from_numpy(args[4]).to(DEV), sh, out=sh)
    torch.cuda.synchronize()
    assert y.data_ptr() == sh.data_ptr()
    check_layer(y, args, "in place")


def test_variant_deterministic_and_linear_in_p():
    args = case(10, 64, 8, 4, 8, 96)
    y1 = host64(run_case(*args))
    y2 = host64(run_case(*args))
    assert np.array_equal(y1, y2)
    x, packed, scales, sel, p, shared = args
    z = np.zeros_like(shared)
    ya = host64(run_case(x, packed, scales, sel, p, z))
    yb = host64(run_case(x, packed, scales, sel, 2 * p, z))
    assert rel_l2(yb, 2 * ya) <= 1e-2


def test_empty_batch_and_unsupported():
    x = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    packed = torch.zeros((2, 8, 2, 16), dtype=torch.uint8, device=DEV)
    scales = torch.zeros((2, 8, 2), dtype=torch.uint8, device=DEV)
    y = mx.moe_linear_mxfp8(x, packed, scales, torch.empty((0, 1), dtype=torch.int32, device=DEV),
                            torch.empty((0, 1), device=DEV), torch.empty((0, 8), dtype=torch.bfloat16, device=DEV))
    assert y.shape == (0, 8)
    with pytest.raises(mx.Mxfp4Error) as e:  # O % 4 != 0
        mx.moe_linear_mxfp8(torch.zeros((1, 64), dtype=torch.bfloat16, device=DEV),
                            torch.zeros((2, 6, 2, 16), dtype=torch.uint8, device=DEV),
                            torch.zeros((2, 6, 2), dtype=torch.uint8, device=DEV),
                            torch.zeros((1, 1), dtype=torch.int32, device=DEV), torch.ones((1, 1), device=DEV),
                            torch.zeros((1, 6), dtype=torch.bfloat16, device=DEV))
    assert e.value.status == _abi.ERR_UNSUPPORTED


def _sample_rows(O, n, seed):
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(O, size=min(n, O), replace=False).tolist())
    rows.update({0, O - 1, min(O - 1, 127), min(O - 1, 128)})
    return np.array(sorted(rows))


@functools.lru_cache(maxsize=1)
def _workload(name):
    inp = workloads.make_inputs(name)
    w = inp.workload
    say(f"uploading {name}")
    packed = torch.empty((w.E, w.O, w.G, 16), dtype=torch.uint8, device=DEV)
    scales = torch.empty((w.E, w.O, w.G), dtype=torch.uint8, device=DEV)
    for e in range(w.E):
        packed[e].copy_(torch.from_numpy(inp.packed[e]))
        scales[e].copy_(torch.from_numpy(inp.scales[e]))
    return inp, packed, scales


@pytest.mark.parametrize("name,nrows", [("prefill", 40), ("skewed", 32)])
def test_variant_full_workloads_sampled_rows(name, nrows):
    inp, packed, scales = _workload(name)
    w = inp.workload
    rows = _sample_rows(w.O, nrows, 11)
    say(f"mxfp8 variant on {name}: oracle on {rows.size} rows x {w.T} tokens")
    y = mx.moe_linear_mxfp8(bf16_dev(inp.x), packed, scales, torch.from_numpy(inp.sel).to(DEV),
                            torch.from_numpy(inp.p).to(DEV), bf16_dev(inp.shared))
    torch.cuda.synchronize()
    yh = host64(y)
    assert np.all(np.isfinite(yh))
    ref = oracle.expert_linear_mxfp8_rows(inp.x, inp.packed, inp.scales, inp.sel, inp.p, inp.shared, rows)
    exact = oracle.expert_linear_rows(inp.x, inp.packed, inp.scales, inp.sel, inp.p, inp.shared, rows)
    sh = inp.shared.astype(np.float64)[:, rows]
    r = rel_l2(yh[:, rows], ref)
    rq = rel_l2(ref - sh, exact - sh)
    say(f"  {name}: rel L2 vs variant oracle {r:.3e}; variant vs exact layer (routed part) {rq:.3e}")
    assert r <= BF16_REL_L2
    assert rq <= VS_EXACT_REL_L2


# ------------------------------------------------------------------ prepared weights

def _prepared_layout_numpy(packed, scales):
    """The documented prepared layout, built with numpy: slot (e, n, q, f, l)
    holds group 4q + l // 16 of row 128n + 16f + l % 16, zeros past O / G;
    its scale byte sits at (((e, n, q) * 2 + f // 4) * 64 + l) * 4 + f % 4."""
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
    # scales: (e, n, q, half, l, f % 4)
    sc = sc.reshape(E, NT, NQ, 2, 4, 64).transpose(0, 1, 2, 3, 5, 4)
    return np.concatenate([codes.reshape(-1), sc.reshape(-1)])


@pytest.mark.parametrize("E,O,G", [(2, 40, 1), (3, 132, 9), (2, 256, 6)])
def test_prepared_layout_bytes(E, O, G):
    rng = np.random.default_rng(E * O + G)
    packed = rng.integers(0, 256, (E, O, G, 16), dtype=np.uint8)
    scales = rng.integers(0, 255, (E, O, G), dtype=np.uint8)
    prep = mx.prepare_mx(torch.from_numpy(packed).to(DEV), torch.from_numpy(scales).to(DEV))
    torch.cuda.synchronize()
    assert np.array_equal(prep.buf.cpu().numpy(), _prepared_layout_numpy(packed, scales))


def run_prepared(x, packed, scales, sel, p, shared):
    prep = mx.prepare_mx(torch.from_numpy(packed).to(DEV), torch.from_numpy(scales).to(DEV))
    y = mx.moe_linear_mxfp8_prepared(bf16_dev(x), prep, torch.from_numpy(sel).to(DEV), torch.from_numpy(p).to(DEV),
                                     bf16_dev(shared))
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("c", CASES, ids=[f"T{c[1]}E{c[2]}K{c[3]}G{c[4]}O{c[5]}" for c in CASES])
def test_prepared_matches_canonical_bit_for_bit(c):
    args = case(*c)
    say(f"prepared weights, case {c}")
    y0 = run_case(*args)
    y1 = run_prepared(*args)
    assert torch.equal(y0, y1)


@pytest.mark.parametrize("name", ["prefill", "skewed"])
def test_prepared_full_workloads_match_canonical(name):
    inp, packed, scales = _workload(name)
    say(f"prepared weights on {name}")
    x, sel, p, sh = bf16_dev(inp.x), torch.from_numpy(inp.sel).to(DEV), torch.from_numpy(inp.p).to(DEV), bf16_dev(inp.shared)
    y0 = mx.moe_linear_mxfp8(x, packed, scales, sel, p, sh)
    prep = mx.prepare_mx(packed, scales)
    y1 = mx.moe_linear_mxfp8_prepared(x, prep, sel, p, sh)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)
