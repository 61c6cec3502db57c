"""GPU parity of the block-scaled variant with MXFP4 activations (both
operands of the scaled MFMA in E2M1) through its C ABI, against the float64
oracle.

Bars (written in each check):
* quantised activations (packed codes and scale bytes): bit-exact against
  oracle.quantize_mxfp4 and oracle.pack_codes;
* the layer: relative L2 <= 1e-2 against the variant's own definition,
  oracle.expert_linear_mxfp4act (the routed linear of the dequantised MXFP4
  activations, exact in float64) - the bf16 bar;
* the error of the variant against the exact layer (unquantised
  activations) is the E2M1 rounding of the activations: printed, and checked
  only to stay below 0.3 relative L2.
"""

import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU-only machines, never run there
    pytest.skip("no GPU", allow_module_level=True)

import mxfp4_block_scaled_amd as mx  # noqa: E402
from mxfp4_block_scaled_amd import _abi  # noqa: E402
from test_gpu_mxfp8 import (  # noqa: E402
    CASES, DEV, BF16_REL_L2, _sample_rows, _special_activations, _workload, bf16_dev, case, host64, rel_l2, say,
)

VS_EXACT_REL_L2 = 0.3


# ------------------------------------------------------------------ quantisation

def _check_quantized(x, ld):
    codes, sb = mx.quantize_mxfp4(bf16_dev(x), ld)
    torch.cuda.synchronize()
    codes, sb = codes.cpu().numpy(), sb.cpu().numpy()
    T, I = x.shape
    want_c, want_s = oracle.quantize_mxfp4(x.astype(np.float64))
    assert np.array_equal(codes[:, :I // 2], oracle.pack_codes(want_c))
    assert np.array_equal(sb[:, :I // 32], want_s)
    assert np.all(codes[:, I // 2:] == 0) and np.all(sb[:, I // 32:] == 0)


@pytest.mark.parametrize("T,I,ld", [(1, 32, 32), (3, 64, 128), (17, 2880, 2944), (64, 7168, 7168), (5, 96, 96)])
def test_quantize_bit_exact(T, I, ld):
    say(f"quantize mxfp4 T={T} I={I} ld={ld}")
    x = _special_activations(T, I, seed=T + I + 5)
    if I >= 96:
        x[0, 64:96] = np.linspace(-6.0, 6.0, 32)       # fits at scale byte 127 exactly
        x[0, 70] = 5.0                                 # a tie between 4 and 6: to 4
        x[0, 71] = 0.25                                # a tie between 0 and 0.5: to 0
    _check_quantized(x, ld)


def test_quantize_every_bf16_value():
    """Every finite bf16 value once (both signs), in blocks of neighbours and
    again shuffled (most values far below their block's maximum)."""
    pats = np.arange(0, 0x7F80, dtype=np.uint32)
    vals = (pats << 16).view(np.float32)
    vals = np.concatenate([vals, -vals])
    rng = np.random.default_rng(13)
    for name, arr in (("neighbours", vals), ("shuffled", rng.permutation(vals))):
        x = np.ascontiguousarray(arr.reshape(-1, 64))
        say(f"quantize mxfp4 every bf16 value, {name}: {x.shape[0]} rows")
        _check_quantized(x, 64)


# ------------------------------------------------------------------ the layer

def run_case(x, packed, scales, sel, p, shared, out=None):
    y = mx.moe_linear_mxfp4act(bf16_dev(x), torch.from_numpy(packed).to(DEV), torch.from_numpy(scales).to(DEV),
                               torch.from_numpy(sel).to(DEV), torch.from_numpy(p).to(DEV), bf16_dev(shared), out=out)
    torch.cuda.synchronize()
    return y


def check_layer(y, args, what):
    ref = oracle.expert_linear_mxfp4act(*args)
    exact = oracle.expert_linear(*args)
    yh = host64(y)
    r = rel_l2(yh, ref)
    sh = args[5]
    rq = rel_l2(ref - sh, exact - sh)
    say(f"  {what}: rel L2 vs variant oracle {r:.3e}; variant vs exact layer (routed part) {rq:.3e}")
    assert r <= BF16_REL_L2, f"{what}: {r:.3e}"
    assert rq <= VS_EXACT_REL_L2, f"{what}: variant error {rq:.3e}"
    assert np.all(np.isfinite(yh))


@pytest.mark.parametrize("c", CASES, ids=[f"T{c[1]}E{c[2]}K{c[3]}G{c[4]}O{c[5]}" for c in CASES])
def test_variant_against_oracle(c):
    args = case(*c)
    say(f"mxfp4-activation variant case {c}")
    check_layer(run_case(*args), args, f"case {c}")


def test_variant_edges():
    args = case(6, 50, 6, 3, 3, 64, distinct=False, empty_experts=(1, 4))
    check_layer(run_case(*args), args, "duplicates and empty experts")
    args = case(7, 9, 5, 1, 5, 36)
    check_layer(run_case(*args), args, "K = 1")
    x, packed, scales, sel, p, shared = case(8, 700, 3, 1, 4, 64)
    sel[:] = 2
    check_layer(run_case(x, packed, scales, sel, p, shared), (x, packed, scales, sel, p, shared), "one hot expert")
    args = case(9, 12, 4, 2, 2, 48)
    sh = bf16_dev(args[5])
    y = mx.moe_linear_mxfp4act(bf16_dev(args[0]), torch.from_numpy(args[1]).to(DEV),
                               torch.from_numpy(args[2]).to(DEV), torch.from_numpy(args[3]).to(DEV),
                               torch.from_numpy(args[4]).to(DEV), sh, out=sh)
    torch.cuda.synchronize()
    assert y.data_ptr() == sh.data_ptr()
    check_layer(y, args, "in place")


def test_variant_on_grid_activations_is_the_exact_layer():
    """Activations that are E2M1 values times a block scale quantise to
    themselves: the variant is then the exact layer (up to the output
    rounding)."""
    x, packed, scales, sel, p, shared = case(14, 40, 6, 2, 5, 64)
    rng = np.random.default_rng(14)
    r = np.ldexp(1.0, rng.integers(-3, 3, (40, 1)))
    xg = oracle.E2M1_TABLE[rng.integers(0, 16, (40, 160))] * r
    xg[:, ::32] = 6.0 * r
    args = (xg.astype(np.float32), packed, scales, sel, p, shared)
    y = host64(run_case(*args))
    assert rel_l2(y, oracle.expert_linear(*args)) <= BF16_REL_L2


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
    y = mx.moe_linear_mxfp4act(x, packed, scales, torch.empty((0, 1), dtype=torch.int32, device=DEV),
                               torch.empty((0, 1), device=DEV), torch.empty((0, 8), dtype=torch.bfloat16, device=DEV))
    assert y.shape == (0, 8)
    with pytest.raises(mx.Mxfp4Error) as e:  # O % 4 != 0
        mx.moe_linear_mxfp4act(torch.zeros((1, 64), dtype=torch.bfloat16, device=DEV),
                               torch.zeros((2, 6, 2, 16), dtype=torch.uint8, device=DEV),
                               torch.zeros((2, 6, 2), dtype=torch.uint8, device=DEV),
                               torch.zeros((1, 1), dtype=torch.int32, device=DEV), torch.ones((1, 1), device=DEV),
                               torch.zeros((1, 6), dtype=torch.bfloat16, device=DEV))
    assert e.value.status == _abi.ERR_UNSUPPORTED


@pytest.mark.parametrize("name,nrows", [("prefill", 40), ("skewed", 32)])
def test_variant_full_workloads_sampled_rows(name, nrows):
    inp, packed, scales = _workload(name)
    w = inp.workload
    rows = _sample_rows(w.O, nrows, 12)
    say(f"mxfp4-activation variant on {name}: oracle on {rows.size} rows x {w.T} tokens")
    y = mx.moe_linear_mxfp4act(bf16_dev(inp.x), packed, scales, torch.from_numpy(inp.sel).to(DEV),
                               torch.from_numpy(inp.p).to(DEV), bf16_dev(inp.shared))
    torch.cuda.synchronize()
    yh = host64(y)
    assert np.all(np.isfinite(yh))
    ref = oracle.expert_linear_mxfp4act_rows(inp.x, inp.packed, inp.scales, inp.sel, inp.p, inp.shared, rows)
    exact = oracle.expert_linear_rows(inp.x, inp.packed, inp.scales, inp.sel, inp.p, inp.shared, rows)
    sh = inp.shared.astype(np.float64)[:, rows]
    r = rel_l2(yh[:, rows], ref)
    rq = rel_l2(ref - sh, exact - sh)
    say(f"  {name}: rel L2 vs variant oracle {r:.3e}; variant vs exact layer (routed part) {rq:.3e}")
    assert r <= BF16_REL_L2
    assert rq <= VS_EXACT_REL_L2


# ------------------------------------------------------------------ prepared weights

@pytest.mark.parametrize("c", CASES, ids=[f"T{c[1]}E{c[2]}K{c[3]}G{c[4]}O{c[5]}" for c in CASES])
def test_prepared_matches_canonical_bit_for_bit(c):
    x, packed, scales, sel, p, shared = case(*c)
    say(f"mxfp4-activation variant on prepared weights, case {c}")
    y0 = run_case(x, packed, scales, sel, p, shared)
    prep = mx.prepare_mx(torch.from_numpy(packed).to(DEV), torch.from_numpy(scales).to(DEV))
    y1 = mx.moe_linear_mxfp4act_prepared(bf16_dev(x), prep, torch.from_numpy(sel).to(DEV),
                                         torch.from_numpy(p).to(DEV), bf16_dev(shared))
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)


@pytest.mark.parametrize("name", ["prefill", "skewed"])
def test_prepared_full_workloads_match_canonical(name):
    inp, packed, scales = _workload(name)
    say(f"mxfp4-activation variant, prepared weights on {name}")
    x, sel, p, sh = bf16_dev(inp.x), torch.from_numpy(inp.sel).to(DEV), torch.from_numpy(inp.p).to(DEV), bf16_dev(inp.shared)
    y0 = mx.moe_linear_mxfp4act(x, packed, scales, sel, p, sh)
    prep = mx.prepare_mx(packed, scales)
    y1 = mx.moe_linear_mxfp4act_prepared(x, prep, sel, p, sh)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)
