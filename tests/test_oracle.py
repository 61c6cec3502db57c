"""Pins of the float64 oracle to facts other than itself (CPU only).

Each test ties the oracle to something the pages print (fixtures under
tests/golden, each with its citation), to a closed form, to an invariant of
the definition, to a library routine in a special case, or to the brute-force
scalar version. ``test_planted_mistakes_are_caught`` plants plausible
mistakes in the oracle and checks that the pins fail on each of them.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import mxfp4_oracle as om
import workloads
from conftest import GOLDEN


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rng(seed):
    return np.random.default_rng(seed)


def _random_case(seed, T, E, K, G, O, scale_lo=120, scale_hi=134, distinct=True):
    rng = _rng(seed)
    x = rng.standard_normal((T, 32 * G)).astype(np.float32)
    shared = rng.standard_normal((T, O)).astype(np.float32)
    packed = rng.integers(0, 256, (E, O, G, 16), dtype=np.uint8)
    scales = rng.integers(scale_lo, scale_hi + 1, (E, O, G), dtype=np.uint8)
    if distinct:
        sel = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    else:
        sel = rng.integers(0, E, (T, K)).astype(np.int32)
    p = rng.random((T, K)).astype(np.float32)
    return x, packed, scales, sel, p, shared


# ----------------------------------------------------------- printed values

def test_table_matches_printed_list_bit_for_bit():
    g = _golden("e2m1_table.json")
    assert len(oracle.E2M1_TABLE) == 16
    for i, v in enumerate(g["values"]):
        assert oracle.E2M1_TABLE[i] == v
        assert np.signbit(oracle.E2M1_TABLE[i]) == (math.copysign(1.0, v) < 0)
    assert np.signbit(oracle.E2M1_TABLE[g["negative_zero_index"]])
    # what decoding actually produces: codes 0..15 at unit scale (byte j of the
    # group holds codes 2j (low nibble) and 2j+1 (high nibble), j < 8)
    packed = np.zeros((1, 1, 16), np.uint8)
    packed[0, 0, :8] = [2 * j + 16 * (2 * j + 1) for j in range(8)]
    row = oracle.decode_rows(packed, np.array([[127]], np.uint8))[0, :16]
    for i, v in enumerate(g["values"]):
        assert row[i] == v and np.signbit(row[i]) == (math.copysign(1.0, v) < 0)


def _decode_single_group(byte_values, scale):
    packed = np.zeros((1, 1, 16), dtype=np.uint8)
    packed[0, 0, : len(byte_values)] = byte_values
    return oracle.decode_rows(packed, np.array([[scale]], dtype=np.uint8))[0]


def test_byte_0x21_decodes_low_nibble_first():
    g = _golden("byte_0x21_example.json")
    row = _decode_single_group([g["byte"]], g["scale_byte"])
    assert list(row[:2]) == g["decoded_in_order"]
    assert list(row[:2]) != g["decoded_if_high_first"]
    # through the whole layer: x = e_0 picks the first value, x = e_1 the second
    packed = np.zeros((1, 1, 1, 16), dtype=np.uint8)
    packed[0, 0, 0, 0] = g["byte"]
    scales = np.full((1, 1, 1), g["scale_byte"], dtype=np.uint8)
    for pos, want in enumerate(g["decoded_in_order"]):
        x = np.zeros((1, 32), dtype=np.float32)
        x[0, pos] = 1.0
        y = oracle.expert_linear(x, packed, scales, np.array([[0]]), np.array([[1.0]], np.float32),
                                 np.zeros((1, 1), np.float32))
        assert y[0, 0] == want


def test_scale_bias_examples():
    g = _golden("scale_bias_examples.json")
    one = 2 | (2 << 4)  # both nibbles code 2, the table's 1.0
    for s, factor in g["factors"].items():
        row = _decode_single_group([one] * 16, int(s))
        assert np.all(row == factor)
        assert np.all(oracle.scale_factor(np.array([int(s)], np.uint8)) == factor)


def test_numeric_example_gives_32():
    g = _golden("numeric_example.json")
    args = [np.array(g[k]) for k in ("latent_tokens", "packed_weights", "scale_bytes",
                                     "selected_experts", "mixture_weights", "shared_output")]
    args[0] = args[0].astype(np.float32)
    args[1] = args[1].astype(np.uint8)
    args[2] = args[2].astype(np.uint8)
    args[4] = args[4].astype(np.float32)
    args[5] = args[5].astype(np.float32)
    y = oracle.expert_linear(*args)
    assert y.tolist() == g["output"]
    assert oracle.expert_linear_scalar(*[a.tolist() for a in args]) == g["output"]


def test_shape_examples():
    g = _golden("shape_examples.json")
    rng = _rng(5)
    for case in g["cases"]:
        T, I = case["latent_tokens"]
        E, O, G, _ = case["packed_weights"]
        K = case["selected_experts"][1]
        x = rng.standard_normal((T, I)).astype(np.float32)
        packed = rng.integers(0, 256, case["packed_weights"], dtype=np.uint8)
        scales = rng.integers(120, 130, (E, O, G), dtype=np.uint8)
        sel = np.stack([rng.permutation(E)[:K] for _ in range(T)])
        p = np.full((T, K), 1.0 / K, np.float32)
        shared = rng.standard_normal(case["shared_output"]).astype(np.float32)
        assert list(oracle.expert_linear(x, packed, scales, sel, p, shared).shape) == case["output"]


# ----------------------------------------------------------- exhaustive grid

def test_every_code_and_scale():
    table = _golden("e2m1_table.json")["values"]
    for s in range(256):
        for code in range(16):
            row = _decode_single_group([code | (code << 4)] * 16, s)
            want = math.ldexp(table[code], s - 127)
            assert np.all(row == want)
            assert np.all(np.signbit(row) == (math.copysign(1.0, want) < 0))


def test_nibble_split_exhaustive():
    b = np.arange(256, dtype=np.uint8)
    lo, hi = oracle.split_nibbles(b)
    for v in range(256):
        assert (int(lo[v]), int(hi[v])) == (v % 16, v // 16)
    codes = oracle.group_codes(b.reshape(16, 16))
    for j in range(16):
        for v in range(16):
            byte = 16 * j + v
            assert codes[j, 2 * v] == byte % 16 and codes[j, 2 * v + 1] == byte // 16


# ----------------------------------------------------------- closed forms

@pytest.mark.parametrize("byte,scale", [(0x21, 128), (0x22, 127), (0x9F, 125), (0x7E, 130), (0x08, 127)])
def test_closed_form_constant_matrix(byte, scale):
    """One byte value and one scale everywhere, x = ones: every output is
    shared + sum_k p_k * 16 G (LUT[lo] + LUT[hi]) 2^(s-127)."""
    table = _golden("e2m1_table.json")["values"]
    T, E, K, G, O = 3, 5, 2, 3, 4
    rng = _rng(byte)
    packed = np.full((E, O, G, 16), byte, np.uint8)
    scales = np.full((E, O, G), scale, np.uint8)
    sel = np.stack([rng.permutation(E)[:K] for _ in range(T)])
    p = rng.random((T, K)).astype(np.float32)
    shared = rng.standard_normal((T, O)).astype(np.float32)
    y = oracle.expert_linear(np.ones((T, 32 * G), np.float32), packed, scales, sel, p, shared)
    lo, hi = divmod(byte, 16)[1], divmod(byte, 16)[0]
    per_expert = 16 * G * (table[lo] + table[hi]) * 2.0 ** (scale - 127)
    for t in range(T):
        for o in range(O):
            want = float(shared[t, o]) + sum(float(p[t, k]) for k in range(K)) * per_expert
            assert math.isclose(y[t, o], want, rel_tol=1e-14, abs_tol=1e-14)


def test_encoded_matrix_is_a_plain_matvec():
    """Draw a matrix of table values with per-group powers of two, encode it
    into bytes by the stated layout, and compare with numpy's matmul."""
    table = np.array(_golden("e2m1_table.json")["values"])
    rng = _rng(11)
    T, E, G, O = 5, 3, 4, 7
    I = 32 * G
    codes = rng.integers(0, 16, (E, O, I))
    scales = rng.integers(118, 137, (E, O, G), dtype=np.uint8)
    W = table[codes] * np.repeat(2.0 ** (scales.astype(np.int64) - 127), 32, axis=2)
    packed = (codes[..., 0::2] + 16 * codes[..., 1::2]).reshape(E, O, G, 16).astype(np.uint8)
    x = rng.standard_normal((T, I)).astype(np.float32)
    sel = rng.integers(0, E, (T, 1)).astype(np.int32)
    p = np.ones((T, 1), np.float32)
    y = oracle.expert_linear(x, packed, scales, sel, p, np.zeros((T, O), np.float32))
    want = np.stack([W[sel[t, 0]] @ x[t].astype(np.float64) for t in range(T)])
    np.testing.assert_allclose(y, want, rtol=1e-13, atol=1e-13)
    # and the rows decoded directly
    for e in range(E):
        np.testing.assert_array_equal(oracle.decode_expert(packed[e], scales[e]), W[e])


# ----------------------------------------------------------- brute force

@pytest.mark.parametrize("seed", range(6))
def test_brute_force_matches(seed):
    rng = _rng(100 + seed)
    T, E, K, G, O = (int(v) for v in rng.integers(1, 5, 5))
    K = min(K, E)
    x, packed, scales, sel, p, shared = _random_case(seed, T, E, K, G, O, distinct=seed % 2 == 0)
    y = oracle.expert_linear(x, packed, scales, sel, p, shared)
    ys = np.array(oracle.expert_linear_scalar(x.tolist(), packed.tolist(), scales.tolist(),
                                              sel.tolist(), p.tolist(), shared.tolist()))
    np.testing.assert_allclose(y, ys, rtol=1e-12, atol=1e-12)


def test_brute_force_matches_tiny_workload():
    inp = workloads.make_inputs("tiny")
    y = oracle.expert_linear(inp.x, inp.packed, inp.scales, inp.sel, inp.p, inp.shared)
    ys = np.array(oracle.expert_linear_scalar(inp.x.tolist(), inp.packed.materialize().tolist(),
                                              inp.scales.materialize().tolist(), inp.sel.tolist(),
                                              inp.p.tolist(), inp.shared.tolist()))
    np.testing.assert_allclose(y, ys, rtol=1e-12, atol=1e-12)


def test_rows_variant_matches_full():
    x, packed, scales, sel, p, shared = _random_case(3, 6, 5, 3, 3, 40)
    y = oracle.expert_linear(x, packed, scales, sel, p, shared)
    rows = [0, 7, 39, 12]
    yr = oracle.expert_linear_rows(x, packed, scales, sel, p, shared, rows)
    np.testing.assert_allclose(yr, y[:, rows], rtol=1e-13, atol=1e-13)


# ----------------------------------------------------------- invariants

def test_unselected_experts_do_not_matter():
    x, packed, scales, sel, p, shared = _random_case(4, 4, 9, 2, 2, 8)
    y = oracle.expert_linear(x, packed, scales, sel, p, shared)
    rng = _rng(44)
    packed2, scales2 = packed.copy(), scales.copy()
    for e in set(range(9)) - set(np.unique(sel).tolist()):
        packed2[e] = rng.integers(0, 256, packed2[e].shape)
        scales2[e] = 255
    assert np.array_equal(oracle.expert_linear(x, packed2, scales2, sel, p, shared), y)


def test_linear_in_x_and_p():
    x1, packed, scales, sel, p1, shared = _random_case(6, 3, 4, 2, 3, 6)
    x2, _, _, _, p2, _ = _random_case(7, 3, 4, 2, 3, 6)
    a, b = 0.75, -1.25
    f = lambda x, p: oracle.expert_linear(x, packed, scales, sel, p, shared) - shared
    lhs = f(a * x1.astype(np.float64) + b * x2.astype(np.float64), p1)
    np.testing.assert_allclose(lhs, a * f(x1, p1) + b * f(x2, p1), rtol=1e-11, atol=1e-11)
    lhs = f(x1, a * p1.astype(np.float64) + b * p2.astype(np.float64))
    np.testing.assert_allclose(lhs, a * f(x1, p1) + b * f(x1, p2), rtol=1e-11, atol=1e-11)


def test_sign_flip_negates_routed_part():
    x, packed, scales, sel, p, shared = _random_case(8, 4, 5, 2, 3, 6)
    zero = np.zeros_like(shared)
    y = oracle.expert_linear(x, packed, scales, sel, p, zero)
    yn = oracle.expert_linear(x, packed ^ np.uint8(0x88), scales, sel, p, zero)
    assert np.array_equal(yn, -y)


def test_scale_shift_doubles_routed_part():
    x, packed, scales, sel, p, shared = _random_case(9, 4, 5, 2, 3, 6)
    zero = np.zeros_like(shared)
    y = oracle.expert_linear(x, packed, scales, sel, p, zero)
    y2 = oracle.expert_linear(x, packed, scales + np.uint8(1), sel, p, zero)
    assert np.array_equal(y2, 2 * y)


def test_nibble_swap_equals_input_pair_swap():
    x, packed, scales, sel, p, shared = _random_case(10, 3, 4, 2, 2, 5)
    swapped = ((packed & 0x0F) << 4) | (packed >> 4)
    xs = x.copy()
    xs[:, 0::2], xs[:, 1::2] = x[:, 1::2], x[:, 0::2]
    np.testing.assert_allclose(oracle.expert_linear(xs, swapped, scales, sel, p, shared),
                               oracle.expert_linear(x, packed, scales, sel, p, shared),
                               rtol=1e-13, atol=1e-13)


def test_duplicate_selection_counts_twice():
    x, packed, scales, sel, p, shared = _random_case(12, 2, 3, 1, 2, 4)
    zero = np.zeros_like(shared)
    single = oracle.expert_linear(x, packed, scales, sel, p, zero)
    twice = oracle.expert_linear(x, packed, scales, np.concatenate([sel, sel], 1),
                                 np.concatenate([p, p], 1), zero)
    np.testing.assert_allclose(twice, 2 * single, rtol=1e-14)


def test_inputs_not_mutated_and_fresh_output():
    x, packed, scales, sel, p, shared = _random_case(13, 3, 4, 2, 2, 5)
    copies = [a.copy() for a in (x, packed, scales, sel, p, shared)]
    y = oracle.expert_linear(x, packed, scales, sel, p, shared)
    for a, c in zip((x, packed, scales, sel, p, shared), copies):
        assert np.array_equal(a, c)
    assert not np.shares_memory(y, shared)


def test_invalid_index_raises():
    x, packed, scales, sel, p, shared = _random_case(14, 2, 3, 1, 1, 2)
    sel[0, 0] = 3
    with pytest.raises(ValueError):
        oracle.expert_linear(x, packed, scales, sel, p, shared)


# ----------------------------------------------------------- bucketing

@pytest.mark.parametrize("seed,T,K,E", [(0, 1, 4, 128), (1, 8, 8, 384), (2, 37, 3, 5), (3, 200, 8, 64)])
def test_bucketing_is_a_stable_sort(seed, T, K, E):
    rng = _rng(seed)
    sel = rng.integers(0, E, (T, K)).astype(np.int32)
    b = oracle.bucket_pairs(sel, E)
    flat = sel.ravel()
    assert np.array_equal(b["count"], np.bincount(flat, minlength=E))
    assert np.array_equal(b["offsets"], np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))]))
    assert np.array_equal(b["perm"], np.argsort(flat, kind="stable"))
    assert np.array_equal(b["perm"][b["slot_of_pair"]], np.arange(flat.size))
    assert b["n_invalid"] == 0


def test_bucketing_drops_invalid():
    sel = np.array([[0, 5], [-1, 2], [2, 0]], np.int32)
    b = oracle.bucket_pairs(sel, 3)
    assert b["n_invalid"] == 2
    assert b["count"].tolist() == [2, 0, 2]
    assert b["perm"].tolist() == [0, 5, 3, 4]
    assert b["slot_of_pair"].tolist() == [0, -1, -1, 2, 3, 1]


# ----------------------------------------------------------- workloads

def test_workload_shapes_and_routing():
    for name, w in workloads.WORKLOADS.items():
        if w.T * w.E > 4_000_000:
            continue
        inp = workloads.make_inputs(w, n_routing_sets=2)
        assert inp.x.shape == (w.T, 32 * w.G) and inp.shared.shape == (w.T, w.O)
        assert inp.sel.shape == (w.T, w.K) and inp.p.shape == (w.T, w.K)
        assert inp.sel.dtype == np.int32 and inp.p.dtype == np.float32
        for row in inp.sel:
            assert len(set(row.tolist())) == w.K  # distinct experts per token
        np.testing.assert_allclose(inp.p.sum(1), 1.0, rtol=1e-6)
        if w.F:  # SwiGLU block: stacked gate/up, then the down projection
            assert inp.packed[0].shape == (2 * w.F, w.G, 16)
            assert inp.dn_packed[1].shape == (w.O, w.F // 32, 16)
            assert inp.dn_scales[2].shape == (w.O, w.F // 32)
        else:
            assert inp.packed[0].shape == (w.O, w.G, 16) and inp.dn_packed is None
        s = inp.scales[w.E - 1]
        assert s.min() >= w.scale_lo and s.max() <= w.scale_hi
        assert not np.array_equal(inp.routing_sets[0][0], inp.routing_sets[1][0])
        if w.dtype == "bf16":
            assert np.all((inp.x.view(np.uint32) & 0xFFFF) == 0)


# ----------------------------------------------------------- planted mistakes

def _pins_pass():
    """Run the value pins; return False as soon as one fails."""
    checks = [test_byte_0x21_decodes_low_nibble_first, test_scale_bias_examples,
              test_numeric_example_gives_32, test_encoded_matrix_is_a_plain_matvec,
              test_table_matches_printed_list_bit_for_bit, test_brute_force_matches_tiny_workload]
    checks += [lambda b=b, s=s: test_closed_form_constant_matrix(b, s) for b, s in [(0x21, 128), (0x9F, 125)]]
    for c in checks:
        try:
            c()
        except AssertionError:
            return False
    return True


def test_planted_mistakes_are_caught(monkeypatch):
    assert _pins_pass()
    orig_split = om.split_nibbles
    orig_table = om.E2M1_TABLE.copy()
    orig_factor = om.scale_factor
    orig_decode_rows = om.decode_rows
    mistakes = {
        "high nibble first": lambda mp: mp.setattr(om, "split_nibbles", lambda b: orig_split(b)[::-1]),
        "positive zero at index 8": lambda mp: mp.setattr(om, "E2M1_TABLE", np.where(np.arange(16) == 8, 0.0, orig_table)),
        "wrong LUT entry": lambda mp: mp.setattr(om, "E2M1_TABLE", np.where(np.arange(16) == 6, 5.0, orig_table)),
        "bias sign flipped": lambda mp: mp.setattr(om, "scale_factor", lambda s: 1.0 / orig_factor(s)),
        "off-by-one bias": lambda mp: mp.setattr(om, "scale_factor", lambda s: 2.0 * orig_factor(s)),
        "groups reversed": lambda mp: mp.setattr(
            om, "decode_rows", lambda pk, sc: orig_decode_rows(np.asarray(pk)[:, ::-1], np.asarray(sc)[:, ::-1])),
    }
    for name, plant in mistakes.items():
        with monkeypatch.context() as mp:
            plant(mp)
            assert not _pins_pass(), f"planted mistake not caught: {name}"
    assert _pins_pass()


def test_planted_combine_mistakes_are_caught(monkeypatch):
    """Mistakes in the layer itself: dropping shared, ignoring p, or using
    the transpose of W all change the brute-force comparison."""
    x, packed, scales, sel, p, shared = _random_case(21, 3, 4, 2, 1, 32)
    ys = np.array(oracle.expert_linear_scalar(x.tolist(), packed.tolist(), scales.tolist(),
                                              sel.tolist(), p.tolist(), shared.tolist()))
    good = oracle.expert_linear(x, packed, scales, sel, p, shared)
    np.testing.assert_allclose(good, ys, rtol=1e-12, atol=1e-12)
    assert not np.allclose(good - shared, ys, rtol=1e-6)  # dropped shared term
    assert not np.allclose(oracle.expert_linear(x, packed, scales, sel, np.ones_like(p), shared), ys)
    orig = om.decode_expert
    with monkeypatch.context() as mp:  # square case: I = O = 32, transposed operand
        mp.setattr(om, "decode_expert", lambda pk, sc: orig(pk, sc).T)
        assert not np.allclose(oracle.expert_linear(x, packed, scales, sel, p, shared), ys)


# ------------------------------------------------------- the SwiGLU expert

def _swiglu_case(seed, T, E, K, G, F, O, scale_lo=118, scale_hi=126, distinct=True):
    """Random gate/up (E, 2F, G, 16) and down (E, O, F/32, 16) experts."""
    rng = _rng(seed)
    x, _, _, sel, p, shared = _random_case(seed, T, E, K, G, O, distinct=distinct)
    gu_p = rng.integers(0, 256, (E, 2 * F, G, 16), dtype=np.uint8)
    gu_s = rng.integers(scale_lo, scale_hi + 1, (E, 2 * F, G), dtype=np.uint8)
    dn_p = rng.integers(0, 256, (E, O, F // 32, 16), dtype=np.uint8)
    dn_s = rng.integers(scale_lo, scale_hi + 1, (E, O, F // 32), dtype=np.uint8)
    return x, gu_p, gu_s, dn_p, dn_s, sel, p, shared


def test_silu_closed_forms():
    assert oracle.silu(0.0) == 0.0
    assert oracle.silu(1.0) == pytest.approx(1.0 / (1.0 + math.exp(-1.0)), rel=1e-15)
    v = np.linspace(-30, 30, 121)
    # silu(-v) = silu(v) - v, and silu(v) -> v, -> 0 at the ends
    np.testing.assert_allclose(oracle.silu(-v), oracle.silu(v) - v, rtol=0, atol=1e-12)
    assert oracle.silu(60.0) == pytest.approx(60.0, rel=1e-15)
    assert abs(oracle.silu(-60.0)) < 1e-20
    assert oracle.silu(-1e6) == 0.0


@pytest.mark.parametrize("seed", [0, 1])
def test_swiglu_brute_force_matches(seed):
    T, E, K, G, F, O = 3, 3, 2, 1, 32, 5
    args = _swiglu_case(seed, T, E, K, G, F, O, distinct=seed == 0)
    ys = np.array(oracle.expert_swiglu_scalar(*[a.tolist() for a in args]))
    y = oracle.expert_swiglu(*args)
    np.testing.assert_allclose(y, ys, rtol=1e-11, atol=1e-9)


def test_swiglu_closed_form_pins_gate_then_up():
    # x = ones (I = 32); gate rows all 0.5 -> g = 16; up rows all -1 -> u = -32;
    # down rows all 1 -> every output is F * silu(16) * (-32). With gate and
    # up swapped it would be F * silu(-32) * 16, which is tiny.
    F, O = 32, 3
    x = np.ones((1, 32), np.float32)
    gu_p = np.zeros((1, 2 * F, 1, 16), np.uint8)
    gu_p[0, :F] = 0x11       # code 1 = 0.5 in both nibbles
    gu_p[0, F:] = 0xAA       # code 10 = -1
    gu_s = np.full((1, 2 * F, 1), 127, np.uint8)
    dn_p = np.full((1, O, 1, 16), 0x22, np.uint8)  # code 2 = 1
    dn_s = np.full((1, O, 1), 127, np.uint8)
    sel = np.zeros((1, 1), np.int32)
    p = np.ones((1, 1), np.float32)
    shared = np.zeros((1, O), np.float32)
    y = oracle.expert_swiglu(x, gu_p, gu_s, dn_p, dn_s, sel, p, shared)
    want = F * (16.0 / (1.0 + math.exp(-16.0))) * -32.0
    np.testing.assert_allclose(y, np.full((1, O), want), rtol=1e-14)


def test_swiglu_zero_gate_or_up_gives_shared():
    args = list(_swiglu_case(3, 4, 5, 2, 2, 64, 7))
    x, gu_p, gu_s, dn_p, dn_s, sel, p, shared = args
    for half in (slice(0, 64), slice(64, 128)):
        z = gu_p.copy()
        z[:, half] = 0
        y = oracle.expert_swiglu(x, z, gu_s, dn_p, dn_s, sel, p, shared)
        assert np.array_equal(y, shared.astype(np.float64))


def test_swiglu_scale_shifts_double_the_routed_part():
    x, gu_p, gu_s, dn_p, dn_s, sel, p, shared = _swiglu_case(4, 4, 5, 2, 2, 64, 7)
    base = oracle.expert_swiglu(x, gu_p, gu_s, dn_p, dn_s, sel, p, shared) - shared
    up_s = gu_s.copy()
    up_s[:, 64:] += 1  # up doubles: h doubles (h is linear in up)
    y_up = oracle.expert_swiglu(x, gu_p, up_s, dn_p, dn_s, sel, p, shared) - shared
    np.testing.assert_allclose(y_up, 2 * base, rtol=1e-12, atol=1e-12)
    y_dn = oracle.expert_swiglu(x, gu_p, gu_s, dn_p, dn_s + np.uint8(1), sel, p, shared) - shared
    np.testing.assert_allclose(y_dn, 2 * base, rtol=1e-12, atol=1e-12)
    # doubling the gate does not double the result (silu is not linear)
    g_s = gu_s.copy()
    g_s[:, :64] += 1
    y_g = oracle.expert_swiglu(x, gu_p, g_s, dn_p, dn_s, sel, p, shared) - shared
    assert not np.allclose(y_g, 2 * base, rtol=1e-3)


def test_swiglu_is_the_composition_of_two_expert_linears():
    # gate, up and down each computed by the (pinned) routed linear with one
    # slot per pair and unit weights, then combined by hand
    x, gu_p, gu_s, dn_p, dn_s, sel, p, shared = _swiglu_case(5, 3, 4, 2, 2, 32, 6)
    T, K = sel.shape
    y = shared.astype(np.float64).copy()
    for k in range(K):
        one = np.ones((T, 1), np.float32)
        s1 = sel[:, k:k + 1]
        g = oracle.expert_linear(x, gu_p[:, :32], gu_s[:, :32], s1, one, np.zeros((T, 32), np.float32))
        u = oracle.expert_linear(x, gu_p[:, 32:], gu_s[:, 32:], s1, one, np.zeros((T, 32), np.float32))
        h = g / (1.0 + np.exp(-g)) * u
        d = oracle.expert_linear(h, dn_p, dn_s, s1, one, np.zeros((T, 6), np.float32))
        y += p[:, k:k + 1].astype(np.float64) * d
    np.testing.assert_allclose(oracle.expert_swiglu(x, gu_p, gu_s, dn_p, dn_s, sel, p, shared), y,
                               rtol=1e-12, atol=1e-9)


def test_swiglu_rows_variant_matches_full():
    args = _swiglu_case(6, 5, 6, 3, 2, 64, 40)
    full = oracle.expert_swiglu(*args)
    rows = np.array([0, 7, 8, 39])
    np.testing.assert_allclose(oracle.expert_swiglu_rows(*args, rows), full[:, rows], rtol=1e-13, atol=1e-12)


def test_swiglu_planted_mistakes_are_caught(monkeypatch):
    args = _swiglu_case(7, 3, 3, 2, 1, 32, 4)
    ys = np.array(oracle.expert_swiglu_scalar(*[a.tolist() for a in args]))
    np.testing.assert_allclose(oracle.expert_swiglu(*args), ys, rtol=1e-11, atol=1e-9)
    orig_silu, orig_hidden = om.silu, om.swiglu_hidden
    mistakes = {
        "sigmoid instead of silu": lambda mp: mp.setattr(om, "silu", lambda v: 1.0 / (1.0 + np.exp(-np.asarray(v)))),
        "gate and up swapped": lambda mp: mp.setattr(
            om, "swiglu_hidden", lambda xr, pk, sc: orig_hidden(xr, np.roll(np.asarray(pk), 32, axis=0),
                                                                np.roll(np.asarray(sc), 32, axis=0))),
        "silu dropped (identity)": lambda mp: mp.setattr(
            om, "silu", lambda v: orig_silu(v) * 0 + np.asarray(v, dtype=np.float64)),
    }
    for name, plant in mistakes.items():
        with monkeypatch.context() as mp:
            plant(mp)
            assert not np.allclose(oracle.expert_swiglu(*args), ys, rtol=1e-6), f"planted mistake not caught: {name}"


# ----------------------------------------------------------------- routers

@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("mode", ["softmax", "sigmoid"])
def test_router_brute_force_matches(seed, mode):
    rng = _rng(seed)
    logits = rng.standard_normal((6, 12)) * 2
    bias = rng.standard_normal(12) * 0.3 if mode == "sigmoid" else None
    K = 4
    sel, p = (oracle.route_softmax(logits, K, 2.5) if mode == "softmax" else oracle.route_sigmoid(logits, bias, K, 2.5))
    s2, p2 = oracle.route_scalar(logits.tolist(), None if bias is None else bias.tolist(), K, mode, 2.5)
    assert sel.tolist() == s2
    np.testing.assert_allclose(p, np.array(p2), rtol=1e-14)


def test_router_ties_go_to_the_lower_index_in_order():
    logits = np.array([[0.0, 3.0, 1.0, 3.0, 1.0, 3.0]])
    sel, p = oracle.route_softmax(logits, 4)
    assert sel.tolist() == [[1, 3, 5, 2]]
    sel, _ = oracle.route_sigmoid(logits, None, 4)
    assert sel.tolist() == [[1, 3, 5, 2]]
    # the three tied experts share the selected mass equally
    np.testing.assert_allclose(p[0, :3], p[0, 0], rtol=1e-15)


def test_softmax_router_closed_forms():
    rng = _rng(4)
    logits = rng.standard_normal((5, 9))
    sel, p = oracle.route_softmax(logits, 9)  # every expert: the weights are the softmax itself
    z = np.exp(logits - logits.max(1, keepdims=True))
    np.testing.assert_allclose(p, np.take_along_axis(z / z.sum(1, keepdims=True), sel, 1), rtol=1e-14)
    np.testing.assert_allclose(p.sum(1), 1.0, rtol=1e-14)
    sel, p = oracle.route_softmax(logits, 3, scale=2.0)  # renormalised over the chosen three, times 2
    np.testing.assert_allclose(p.sum(1), 2.0, rtol=1e-14)
    e = np.exp(np.take_along_axis(logits, sel, 1))
    np.testing.assert_allclose(p, 2.0 * e / e.sum(1, keepdims=True), rtol=1e-13)
    # K = 1: weight = scale, whatever the logits
    _, p1 = oracle.route_softmax(logits, 1, scale=1.5)
    np.testing.assert_allclose(p1, 1.5, rtol=1e-15)


def test_sigmoid_router_bias_steers_selection_only():
    logits = np.array([[2.0, 1.0, 0.0]])
    bias = np.array([0.0, 0.0, 0.9])  # sigmoid(0) + 0.9 = 1.4 > sigmoid(2) = 0.88
    sel, p = oracle.route_sigmoid(logits, bias, 2)
    assert sel.tolist() == [[2, 0]]
    s = 1.0 / (1.0 + np.exp(-np.array([0.0, 2.0])))
    np.testing.assert_allclose(p[0], s / (s.sum() + oracle.SIGMOID_EPS), rtol=1e-15)  # unbiased scores
    sel0, _ = oracle.route_sigmoid(logits, None, 2)
    assert sel0.tolist() == [[0, 1]]


def test_router_planted_mistakes_are_caught(monkeypatch):
    rng = _rng(5)
    logits = np.round(rng.standard_normal((8, 10)), 1)  # rounded: ties among the largest
    bias = np.round(rng.standard_normal(10) * 0.2, 1) * 0  # a zero bias keeps the ties
    want_s, want_p = oracle.route_scalar(logits.tolist(), bias.tolist(), 3, "sigmoid", 1.0)
    got_s, got_p = oracle.route_sigmoid(logits, bias, 3)
    assert got_s.tolist() == want_s
    assert any(len(set(np.round(np.sort(r)[-4:], 6))) < 4 for r in logits)  # the case has a tie near the top
    orig = om._topk_desc
    mistakes = {
        "ties to the higher index": lambda mp: mp.setattr(
            om, "_topk_desc", lambda k, K: (k.shape[1] - 1 - np.argsort(-k[:, ::-1], axis=1, kind="stable"))[:, :K]),
        "ascending order": lambda mp: mp.setattr(om, "_topk_desc", lambda k, K: orig(k, K)[:, ::-1]),
    }
    for name, plant in mistakes.items():
        with monkeypatch.context() as mp:
            plant(mp)
            s, _ = oracle.route_sigmoid(logits, bias, 3)
            assert s.tolist() != want_s, f"planted mistake not caught: {name}"
    # weights from the biased scores would differ from the brute force
    bias2 = rng.standard_normal(10) * 0.2
    want_s2, want_p2 = oracle.route_scalar(logits.tolist(), bias2.tolist(), 3, "sigmoid", 1.0)
    s = 1.0 / (1.0 + np.exp(-logits))
    biased = np.take_along_axis(s + bias2, np.array(want_s2), 1)
    assert not np.allclose(biased / biased.sum(1, keepdims=True), np.array(want_p2), rtol=1e-6)


def test_grouped_router_worked_example():
    """Eight experts in four pairs, all logits 0 (every unbiased score 1/2),
    the bias alone ranks: choice scores 0.9 0.1 | 0.8 0.8 | 0.5 0.5 | 0 0.95.
    Group scores (sum of the two best) 1.0, 1.6, 1.0, 0.95: the two kept
    groups are 1 and then 0 (tied with 2, the lower index wins), so the best
    expert overall (7, 0.95) is out; inside the kept groups the best two are
    0 (0.9) and 2 (0.8, tied with 3). The weights are the unbiased scores
    (1/2 each) over their sum: 1/2 each, times the scale."""
    logits = np.zeros((1, 8))
    bias = np.array([0.4, -0.4, 0.3, 0.3, 0.0, 0.0, -0.5, 0.45])
    sel, p = oracle.route_sigmoid_grouped(logits, bias, 2, n_group=4, topk_group=2, scale=3.0)
    assert sel.tolist() == [[0, 2]]
    np.testing.assert_allclose(p, [[1.5, 1.5]], rtol=1e-15)
    sel_raw, p_raw = oracle.route_sigmoid_grouped(logits, bias, 2, 4, 2, scale=3.0, renormalize=False)
    assert sel_raw.tolist() == [[0, 2]]
    np.testing.assert_allclose(p_raw, [[1.5, 1.5]], rtol=1e-15)  # the gathered scores 1/2, times 3
    # scoring a group by its single best expert instead would keep groups 3 and 0
    assert oracle.route_sigmoid(logits, bias, 2)[0].tolist() == [[7, 0]]


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_grouped_router_brute_force_matches(seed):
    rng = _rng(40 + seed)
    E, n_group = [(16, 4), (24, 6), (12, 2), (32, 8)][seed]
    logits = rng.standard_normal((7, E)) * 2
    bias = rng.standard_normal(E) * 0.2
    for topk_group, K, renorm in ((1, 2, True), (2, 3, False), (n_group, 4, True)):
        sel, p = oracle.route_sigmoid_grouped(logits, bias, K, n_group, topk_group, 1.25, renorm)
        s2, p2 = oracle.route_grouped_scalar(logits.tolist(), bias.tolist(), K, n_group, topk_group, 1.25, renorm)
        assert sel.tolist() == s2
        np.testing.assert_allclose(p, np.array(p2), rtol=1e-14)


def test_grouped_router_special_cases():
    rng = _rng(45)
    logits = rng.standard_normal((9, 20)) * 1.5
    bias = rng.standard_normal(20) * 0.1
    # every group kept: the ungrouped sigmoid router
    s_all, p_all = oracle.route_sigmoid_grouped(logits, bias, 5, n_group=5, topk_group=5, scale=2.0)
    s_ref, p_ref = oracle.route_sigmoid(logits, bias, 5, scale=2.0)
    assert np.array_equal(s_all, s_ref)
    np.testing.assert_allclose(p_all, p_ref, rtol=1e-15)
    # one group kept: every chosen expert lies in the group with the best two-score sum
    sel, _ = oracle.route_sigmoid_grouped(logits, bias, 3, n_group=5, topk_group=1)
    keys = 1.0 / (1.0 + np.exp(-logits)) + bias
    two = -np.sort(-keys.reshape(9, 5, 4), axis=2)[:, :, :2].sum(2)
    assert np.array_equal(sel // 4, np.repeat(two.argmax(1)[:, None], 3, axis=1))
    # NaN logits read as -inf: never chosen while finite experts remain
    bad = logits.copy()
    bad[:, 0] = np.nan
    sel, _ = oracle.route_sigmoid_grouped(bad, bias, 3, n_group=5, topk_group=2)
    assert not np.any(sel == 0)


def test_grouped_router_planted_mistakes_are_caught(monkeypatch):
    rng = _rng(46)
    logits = rng.standard_normal((12, 32)) * 2
    bias = rng.standard_normal(32) * 0.3
    want_s, want_p = oracle.route_grouped_scalar(logits.tolist(), bias.tolist(), 4, 8, 3, 1.0, True)
    orig_keys = om.route_keys
    mistakes = {
        "group score = best expert only": lambda mp: mp.setattr(
            om, "_group_scores", lambda k, n: k.reshape(k.shape[0], n, -1).max(axis=2)),
        "unbiased ranking": lambda mp: mp.setattr(om, "route_keys", lambda l, b, m: orig_keys(l, None, m)),
    }
    for name, plant in mistakes.items():
        with monkeypatch.context() as mp:
            plant(mp)
            s, _ = oracle.route_sigmoid_grouped(logits, bias, 4, 8, 3)
            assert s.tolist() != want_s, f"planted mistake not caught: {name}"
    # weights from the biased scores would differ from the brute force
    keys = 1.0 / (1.0 + np.exp(-logits)) + bias
    biased = np.take_along_axis(keys, np.array(want_s), 1)
    assert not np.allclose(biased / biased.sum(1, keepdims=True), np.array(want_p), rtol=1e-6)


@pytest.mark.parametrize("mode", ["softmax", "sigmoid"])
def test_router_weights_of_any_selection_brute_force(mode):
    """route_weights on a selection that is not the top k (the GPU may pick
    another member of a near tie): plain-Python weights of that selection."""
    rng = _rng(6)
    logits = rng.standard_normal((5, 11)) * 1.5
    sel = np.stack([rng.permutation(11)[:4] for _ in range(5)])
    p = oracle.route_weights(logits, sel, mode, 0.75)
    for t in range(5):
        row = [float(v) for v in logits[t]]
        if mode == "softmax":
            m = max(row)
            z = [math.exp(v - m) for v in row]
            score = [v / sum(z) for v in z]
        else:
            score = [1.0 / (1.0 + math.exp(-v)) for v in row]
        mass = 0.0
        for e in sel[t]:
            mass += score[int(e)]
        den = max(mass, oracle.SOFTMAX_MASS_FLOOR) if mode == "softmax" else mass + oracle.SIGMOID_EPS
        np.testing.assert_allclose(p[t], [score[int(e)] / den * 0.75 for e in sel[t]], rtol=1e-14)
    keys = oracle.route_keys(logits, np.arange(11) * 0.1, mode)
    want = logits if mode == "softmax" else 1.0 / (1.0 + np.exp(-logits)) + np.arange(11) * 0.1
    np.testing.assert_allclose(keys, want, rtol=1e-15)


# ------------------------------------------- MXFP8 activations (variant)

def test_e4m3_table_facts():
    t = oracle.E4M3_TABLE
    assert t[0x38] == 1.0 and t[0x7E] == 448.0 and t[0x08] == 2.0 ** -6 and t[0x01] == 2.0 ** -9
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert t[0x80] == 0.0 and math.copysign(1.0, t[0x80]) == -1.0
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0)  # 0x00 .. 0x7e strictly increasing
    np.testing.assert_array_equal(t[0x80:0xFF], -pos)
    # eight steps per binade from 2^-6 up; the subnormals are multiples of 2^-9
    for e in range(-6, 9):
        codes = [c for c in range(0x7F) if 2.0 ** e <= t[c] < 2.0 ** (e + 1)]
        assert len(codes) == (8 if e < 8 else 7), e
        np.testing.assert_allclose(np.diff(t[codes]), 2.0 ** (e - 3))
    np.testing.assert_array_equal(t[:8], np.arange(8) * 2.0 ** -9)


def test_e4m3_round_trip_every_finite_code():
    t = oracle.E4M3_TABLE
    fin = [c for c in range(256) if not np.isnan(t[c])]
    assert oracle.quantize_e4m3(t[fin]).tolist() == fin


def _nearest_e4m3_brute(v):
    """Nearest finite E4M3 value by search; ties to the even code; beyond
    448 the clamp; the sign kept."""
    t = oracle.E4M3_TABLE
    a = min(abs(v), 448.0)
    best = None
    for c in range(0x7F):
        d = abs(t[c] - a)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return best[1] | (0x80 if math.copysign(1.0, v) < 0 else 0)


def test_e4m3_quantize_brute_force():
    rng = _rng(7)
    mags = np.ldexp(rng.uniform(0.5, 1.0, 400), rng.integers(-12, 11, 400))
    vals = mags * rng.choice([-1.0, 1.0], 400)
    # exact ties between neighbours, and the top of the range
    t = oracle.E4M3_TABLE
    ties = [(t[c] + t[c + 1]) / 2 for c in range(0, 0x7E, 3)]
    vals = np.concatenate([vals, ties, [-x for x in ties], [447.0, 448.0, 455.9, 456.0, 463.9, 464.0, 500.0, 1e9]])
    got = oracle.quantize_e4m3(vals)
    want = [_nearest_e4m3_brute(float(v)) for v in vals]
    assert got.tolist() == want


def test_mxfp8_block_exponent_brute_force():
    rng = _rng(8)
    amax = np.concatenate([np.ldexp(rng.uniform(0.5, 1.0, 300), rng.integers(-140, 130, 300)),
                           [448.0, np.nextafter(448.0, 1e9), 1.0, 0.875 * 2.0 ** 9, 2.0 ** -140, 0.0]])
    got = oracle.mxfp8_block_exponent(amax)
    for a, X in zip(amax, got):
        if a == 0:
            assert X == -127
            continue
        want = next(x for x in range(-127, 128) if a <= 448.0 * 2.0 ** x) if a <= 448.0 * 2.0 ** 127 else 127
        assert X == want, (a, X, want)
    assert got[-6:-1].tolist() == [0, 1, -8, 0, -127]


def test_mxfp8_quantize_blocks():
    rng = _rng(9)
    x = rng.standard_normal((5, 96)) * np.ldexp(1.0, rng.integers(-20, 20, (5, 1)))
    x[2, 32:64] = 0.0  # an all-zero block
    x[3, 0:32] = np.linspace(-448.0, 448.0, 32)  # a block that fits at X = 0 exactly
    codes, sb = oracle.quantize_mxfp8(x)
    assert codes.shape == (5, 96) and sb.shape == (5, 3)
    assert sb[2, 1] == 0 and np.all(codes[2, 32:64] == 0)
    assert sb[3, 0] == 127
    xh = oracle.dequantize_mxfp8(codes, sb)
    blocks = np.abs(x).reshape(5, 3, 32)
    X = sb.astype(np.int64) - 127
    # the block max fits without clamping: within 448 * 2^X and above half of it
    nz = blocks.max(2) > 0
    assert np.all(blocks.max(2)[nz] <= 448.0 * np.ldexp(1.0, X[nz]))
    assert np.all(blocks.max(2)[nz] > 224.0 * np.ldexp(1.0, X[nz]))
    # error: half a quantum of the element's binade (2^-4 relative for normals,
    # 2^(X-10) absolute below 2^(X-6))
    err = np.abs(xh - x).reshape(5, 3, 32)
    scale = np.ldexp(1.0, X)[:, :, None]
    bound = np.maximum(blocks * 2.0 ** -4, scale * 2.0 ** -10)
    assert np.all(err <= bound)
    # values already on the grid come back unchanged
    r = np.ldexp(1.0, rng.integers(-5, 5, (4, 1)))
    ong = oracle.E4M3_TABLE[rng.integers(0, 0x7F, (4, 64))] * r
    ong[:, 0] = ong[:, 32] = 448.0 * r[:, 0]  # each block's maximum fixes its scale at r
    np.testing.assert_array_equal(oracle.dequantize_mxfp8(*oracle.quantize_mxfp8(ong)), ong)


def test_mxfp8_linear_composition_and_error():
    """On grid activations the variant equals the exact layer; on normal
    activations it differs by the activation rounding only (relative L2 a few
    percent, far above the exact layer's rounding)."""
    rng = _rng(10)
    T, E, K, G, O = 6, 5, 2, 3, 24
    packed = rng.integers(0, 256, (E, O, G, 16), dtype=np.uint8)
    scales = rng.integers(120, 131, (E, O, G), dtype=np.uint8)
    sel = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    p = rng.uniform(0.1, 1.0, (T, K))
    shared = rng.standard_normal((T, O))
    r = np.ldexp(1.0, rng.integers(-3, 3, (T, 1)))
    xg = oracle.E4M3_TABLE[rng.integers(0, 0x7F, (T, 32 * G))] * r
    xg[:, ::32] = 448.0 * r  # each block's maximum fixes its scale at r
    np.testing.assert_array_equal(oracle.expert_linear_mxfp8(xg, packed, scales, sel, p, shared),
                                  oracle.expert_linear(xg, packed, scales, sel, p, shared))
    x = rng.standard_normal((T, 32 * G))
    ya = oracle.expert_linear_mxfp8(x, packed, scales, sel, p, shared * 0)
    ye = oracle.expert_linear(x, packed, scales, sel, p, shared * 0)
    rel = np.linalg.norm(ya - ye) / np.linalg.norm(ye)
    assert 1e-3 < rel < 5e-2, rel
    rows = np.array([0, 7, 23])
    np.testing.assert_array_equal(oracle.expert_linear_mxfp8_rows(x, packed, scales, sel, p, shared, rows),
                                  oracle.expert_linear_mxfp8(x, packed, scales, sel, p, shared)[:, rows])


def test_mxfp8_planted_mistakes_are_caught(monkeypatch):
    rng = _rng(11)
    vals = np.concatenate([(oracle.E4M3_TABLE[1:0x7E] + oracle.E4M3_TABLE[2:0x7F]) / 2, rng.uniform(-500, 500, 50)])
    want = [_nearest_e4m3_brute(float(v)) for v in vals]
    mistakes = {
        "ties away from zero": lambda mp: mp.setattr(om.np, "rint", lambda a: np.floor(np.asarray(a) + 0.5)),
        "bias 8": lambda mp: mp.setattr(om, "E4M3_BIAS", 8),
        "no subnormal floor": lambda mp: mp.setattr(om, "E4M3_MIN_NORMAL_EXP", -60),
    }
    for name, plant in mistakes.items():
        with monkeypatch.context() as mp:
            plant(mp)
            assert om.quantize_e4m3(vals).tolist() != want, f"planted mistake not caught: {name}"
    # the standard's floor(log2 amax) - 8 scale rule instead of the fitting one
    amax = np.array([300.0, 448.0, 500.0, 1.0])
    floor_rule = np.floor(np.log2(amax)).astype(np.int64) - 8
    assert not np.array_equal(floor_rule, oracle.mxfp8_block_exponent(amax))


# ------------------------------------------- MXFP4 activations (variant)

def _nearest_e2m1_brute(v):
    """Nearest E2M1 value by search over the 8 magnitudes; ties to the even
    code; beyond 6 the clamp; the sign kept."""
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    a = min(abs(v), 6.0)
    best = None
    for c, m in enumerate(mags):
        d = abs(m - a)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return best[1] | (8 if math.copysign(1.0, v) < 0 else 0)


def test_e2m1_quantize_grid_ties_and_clamp():
    t = oracle.E2M1_TABLE
    # every code's own value comes back as that code (both zeros included)
    assert oracle.quantize_e2m1(t).tolist() == list(range(16))
    # midpoints go to the even code
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    assert oracle.quantize_e2m1(mids).tolist() == [0, 2, 2, 4, 4, 6, 6]
    assert oracle.quantize_e2m1([-m for m in mids]).tolist() == [8, 10, 10, 12, 12, 14, 14]
    # just off the midpoints, the nearer one
    assert oracle.quantize_e2m1([0.2501, 0.7499, 4.999, 5.001, 6.9, 100.0]).tolist() == [1, 1, 6, 7, 7, 7]
    assert oracle.quantize_e2m1([-0.1, -0.0]).tolist() == [8, 8]


def test_e2m1_quantize_brute_force():
    rng = _rng(17)
    vals = np.concatenate([rng.uniform(-7.0, 7.0, 600), np.ldexp(rng.uniform(0.5, 1.0, 100), rng.integers(-8, 3, 100))])
    mags = oracle.E2M1_TABLE[:8]
    ties = (mags[:-1] + mags[1:]) / 2
    vals = np.concatenate([vals, ties, -ties])
    got = oracle.quantize_e2m1(vals)
    assert got.tolist() == [_nearest_e2m1_brute(float(v)) for v in vals]


def test_mxfp4_block_exponent_brute_force():
    rng = _rng(18)
    amax = np.concatenate([np.ldexp(rng.uniform(0.5, 1.0, 300), rng.integers(-140, 130, 300)),
                           [6.0, np.nextafter(6.0, 1e9), 3.0, np.nextafter(3.0, 1e9), 1.0, 2.0 ** -140, 0.0]])
    got = oracle.mxfp4_block_exponent(amax)
    for a, X in zip(amax, got):
        if a == 0:
            assert X == -127
            continue
        want = next(x for x in range(-127, 128) if a <= 6.0 * 2.0 ** x) if a <= 6.0 * 2.0 ** 127 else 127
        assert X == want, (a, X, want)
    assert got[-7:-1].tolist() == [0, 1, -1, 0, -2, -127]


def test_mxfp4_quantize_blocks():
    rng = _rng(19)
    x = rng.standard_normal((5, 96)) * np.ldexp(1.0, rng.integers(-20, 20, (5, 1)))
    x[2, 32:64] = 0.0                          # an all-zero block
    x[3, 0:32] = np.linspace(-6.0, 6.0, 32)    # a block that fits at X = 0 exactly
    codes, sb = oracle.quantize_mxfp4(x)
    assert codes.shape == (5, 96) and sb.shape == (5, 3) and codes.max() < 16
    assert sb[2, 1] == 0 and np.all(codes[2, 32:64] == 0)
    assert sb[3, 0] == 127
    xh = oracle.dequantize_mxfp4(codes, sb)
    blocks = np.abs(x).reshape(5, 3, 32)
    X = sb.astype(np.int64) - 127
    nz = blocks.max(2) > 0
    # the block max fits without clamping: within 6 * 2^X and above half of it
    assert np.all(blocks.max(2)[nz] <= 6.0 * np.ldexp(1.0, X[nz]))
    assert np.all(blocks.max(2)[nz] > 3.0 * np.ldexp(1.0, X[nz]))
    # each element against the brute-force nearest value at its block's scale
    for t in range(5):
        for b in range(3):
            s = 2.0 ** X[t, b]
            for k in range(32):
                v = x[t, 32 * b + k]
                assert codes[t, 32 * b + k] == _nearest_e2m1_brute(v / s), (t, b, k)
    # error: half the step of the element's range (0.25, 0.5 or 1 times 2^X)
    err = np.abs(xh - x).reshape(5, 3, 32)
    assert np.all(err <= np.ldexp(1.0, X)[:, :, None] * 1.0)
    # values already on the grid come back unchanged
    r = np.ldexp(1.0, rng.integers(-5, 5, (4, 1)))
    ong = oracle.E2M1_TABLE[rng.integers(0, 16, (4, 64))] * r
    ong[:, 0] = ong[:, 32] = 6.0 * r[:, 0]  # each block's maximum fixes its scale at r
    np.testing.assert_array_equal(oracle.dequantize_mxfp4(*oracle.quantize_mxfp4(ong)), ong)


def test_mxfp4_pack_is_the_weight_nibble_order():
    rng = _rng(20)
    codes = rng.integers(0, 16, (3, 64)).astype(np.uint8)
    packed = oracle.pack_codes(codes)
    assert packed.shape == (3, 32)
    lo, hi = oracle.split_nibbles(packed)
    np.testing.assert_array_equal(lo, codes[:, 0::2])
    np.testing.assert_array_equal(hi, codes[:, 1::2])
    # the printed example: 0x21 holds code 1 (first) and code 2 (second)
    assert oracle.pack_codes(np.array([[1, 2]], dtype=np.uint8)).tolist() == [[0x21]]


def test_mxfp4act_linear_composition_and_error():
    """On grid activations the variant equals the exact layer; on normal
    activations it differs by the E2M1 rounding of the activations (a
    relative L2 of roughly a tenth)."""
    rng = _rng(21)
    T, E, K, G, O = 6, 5, 2, 3, 24
    packed = rng.integers(0, 256, (E, O, G, 16), dtype=np.uint8)
    scales = rng.integers(120, 131, (E, O, G), dtype=np.uint8)
    sel = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    p = rng.uniform(0.1, 1.0, (T, K))
    shared = rng.standard_normal((T, O))
    r = np.ldexp(1.0, rng.integers(-3, 3, (T, 1)))
    xg = oracle.E2M1_TABLE[rng.integers(0, 16, (T, 32 * G))] * r
    xg[:, ::32] = 6.0 * r
    np.testing.assert_array_equal(oracle.expert_linear_mxfp4act(xg, packed, scales, sel, p, shared),
                                  oracle.expert_linear(xg, packed, scales, sel, p, shared))
    x = rng.standard_normal((T, 32 * G))
    ya = oracle.expert_linear_mxfp4act(x, packed, scales, sel, p, shared * 0)
    ye = oracle.expert_linear(x, packed, scales, sel, p, shared * 0)
    rel = np.linalg.norm(ya - ye) / np.linalg.norm(ye)
    assert 3e-2 < rel < 0.3, rel
    y8 = oracle.expert_linear_mxfp8(x, packed, scales, sel, p, shared * 0)
    assert np.linalg.norm(y8 - ye) < np.linalg.norm(ya - ye)  # MXFP8 activations round far less
    rows = np.array([0, 7, 23])
    np.testing.assert_array_equal(oracle.expert_linear_mxfp4act_rows(x, packed, scales, sel, p, shared, rows),
                                  oracle.expert_linear_mxfp4act(x, packed, scales, sel, p, shared)[:, rows])


def test_mxfp4_planted_mistakes_are_caught(monkeypatch):
    rng = _rng(22)
    mags = oracle.E2M1_TABLE[:8]
    vals = np.concatenate([(mags[:-1] + mags[1:]) / 2, rng.uniform(-7, 7, 60), [7.0, 7.5, -9.0, 100.0]])
    want = [_nearest_e2m1_brute(float(v)) for v in vals]
    mistakes = {
        "ties away from zero": lambda mp: mp.setattr(om.np, "rint", lambda a: np.floor(np.asarray(a) + 0.5)),
        "largest magnitude 8": lambda mp: mp.setattr(om, "E2M1_MAX", 8.0),
    }
    for name, plant in mistakes.items():
        with monkeypatch.context() as mp:
            plant(mp)
            assert om.quantize_e2m1(vals).tolist() != want, f"planted mistake not caught: {name}"
    # the standard's floor(log2 amax) - 2 scale rule instead of the fitting one
    amax = np.array([7.0, 6.0, 3.5, 1.0])
    floor_rule = np.floor(np.log2(amax)).astype(np.int64) - 2
    assert not np.array_equal(floor_rule, oracle.mxfp4_block_exponent(amax))
