"""GPU parity: the HIP library (through its C ABI) against the float64 oracle.

Bars (written in each check):
* decoded weights and all bucketing outputs: bit-exact;
* fp32 activations: max |y - y_ref| <= 1e-4 * (1 + |y_ref|), elementwise;
* bf16 activations: relative L2 error <= 1e-2 over the compared outputs,
  and every output within 1e-2 * (|y_ref| + rms(y_ref)) (so that a wrong
  tile cannot hide under the norm).
Full-size workloads run the whole layer on the GPU in the launch
configuration the benchmark times and compare a sample of output rows
(all tokens) that the oracle computes row by row.
"""

import functools
import sys
import zlib

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
F32_TOL = 1e-4
BF16_REL_L2 = 1e-2


def say(*a):
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------------------ helpers

class DevInputs:
    def __init__(self, x, packed, scales, sel, p, shared, dtype):
        self.x, self.packed, self.scales, self.sel, self.p, self.shared = x, packed, scales, sel, p, shared
        self.dtype = dtype


def _tdtype(name):
    return torch.float32 if name == "fp32" else torch.bfloat16


def upload(x, packed, scales, sel, p, shared, dtype):
    """Host arrays (packed/scales may be lazy per-expert tensors) -> device."""
    td = _tdtype(dtype)
    E = len(packed)
    pk0 = np.asarray(packed[0])
    dpk = torch.empty((E,) + pk0.shape, dtype=torch.uint8, device=DEV)
    dsc = torch.empty((E,) + np.asarray(scales[0]).shape, dtype=torch.uint8, device=DEV)
    for e in range(E):
        dpk[e].copy_(torch.from_numpy(np.ascontiguousarray(packed[e])))
        dsc[e].copy_(torch.from_numpy(np.ascontiguousarray(scales[e])))
    return DevInputs(torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV).to(td), dpk, dsc,
                     torch.from_numpy(np.ascontiguousarray(sel, dtype=np.int32)).to(DEV),
                     torch.from_numpy(np.ascontiguousarray(p, dtype=np.float32)).to(DEV),
                     torch.from_numpy(np.ascontiguousarray(shared, dtype=np.float32)).to(DEV).to(td), dtype)


def run(d: DevInputs, flags=0, sel=None, p=None, out=None):
    y = mx.moe_linear(d.x, d.packed, d.scales, d.sel if sel is None else sel, d.p if p is None else p, d.shared,
                      flags=flags, out=out)
    torch.cuda.synchronize()
    return y


def host64(y):
    return y.float().cpu().numpy().astype(np.float64)


def assert_fp32_close(y, ref, what=""):
    err = np.abs(y - ref)
    bound = F32_TOL * (1.0 + np.abs(ref))
    worst = np.max(err / bound) if err.size else 0.0
    assert np.all(err <= bound), f"{what}: max err/bound {worst:.3g} (max abs err {err.max():.3g})"


def rel_l2(y, ref):
    return float(np.linalg.norm(y - ref) / max(np.linalg.norm(ref), 1e-300))


BF16_ELEM = 1e-2


def assert_bf16_close(y, ref, what=""):
    r = rel_l2(y, ref)
    err = np.abs(y - ref)
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    bound = BF16_ELEM * (np.abs(ref) + rms)
    worst = float(np.max(err / np.maximum(bound, 1e-300))) if err.size else 0.0
    say(f"  {what}: rel L2 {r:.3e}, max abs {err.max() if err.size else 0:.3e}, max err/elementwise bound {worst:.3f}")
    assert r <= BF16_REL_L2, f"{what}: relative L2 {r:.3e} > {BF16_REL_L2}"
    assert np.all(err <= bound), f"{what}: an output misses |y - ref| <= {BF16_ELEM} (|ref| + rms) by {worst:.3g}x"


def assert_close_at_scale(y, ref, dtype, unit, what=""):
    """The bars for data that is ordinary data times the power of two `unit`
    (a result is then exactly `unit` times the unit-scale result, so the fp32
    bar's absolute term scales with it): fp32 |y - ref| <= 1e-4 (unit +
    |ref|); the bf16 bars are scale-free already."""
    if dtype == "fp32":
        err = np.abs(y - ref)
        bound = F32_TOL * (unit + np.abs(ref))
        worst = np.max(err / bound) if err.size else 0.0
        assert np.all(err <= bound), f"{what}: max err/bound {worst:.3g} (max abs err {err.max():.3g})"
    else:
        assert_bf16_close(y, ref, what)


def assert_close(y, ref, dtype, what=""):
    if dtype == "fp32":
        assert_fp32_close(y, ref, what)
    else:
        assert_bf16_close(y, ref, what)


def random_case(seed, T, E, K, G, O, dtype, scale_lo=118, scale_hi=130, distinct=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, 32 * G)).astype(np.float32)
    shared = rng.standard_normal((T, O)).astype(np.float32)
    if dtype == "bf16":
        x, shared = workloads.round_to_bf16(x), workloads.round_to_bf16(shared)
    packed = rng.integers(0, 256, (E, O, G, 16), dtype=np.uint8)
    scales = rng.integers(scale_lo, scale_hi + 1, (E, O, G), dtype=np.uint8)
    if distinct:
        sel = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    else:
        sel = rng.integers(0, E, (T, K)).astype(np.int32)
    p = rng.random((T, K)).astype(np.float32)
    return x, packed, scales, sel, p, shared


# ------------------------------------------------------------------ exact decode

@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_decode_rows_every_byte_and_scale_bit_exact(dtype):
    say(f"decode_rows exhaustive {dtype}")
    # row s holds every byte value (group g, byte j = 16 g + j) at scale s
    packed = np.broadcast_to(np.arange(256, dtype=np.uint8).reshape(1, 1, 16, 16), (1, 256, 16, 16)).copy()
    scales = np.broadcast_to(np.arange(256, dtype=np.uint8).reshape(1, 256, 1), (1, 256, 16)).copy()
    want64 = oracle.decode_rows(packed[0], scales[0])
    with np.errstate(over="ignore"):
        want32 = want64.astype(np.float32)
    got = mx.decode_rows(torch.from_numpy(packed).to(DEV), torch.from_numpy(scales).to(DEV), 0, 0, 256,
                         _tdtype(dtype))
    torch.cuda.synchronize()
    if dtype == "fp32":
        g = got.cpu().numpy().view(np.uint32)
        assert np.array_equal(g, want32.view(np.uint32))
    else:
        g = got.view(torch.int16).cpu().numpy().view(np.uint16)
        wb = want32.view(np.uint32)
        assert np.all((wb & 0xFFFF) == 0)  # every decoded value is a bf16 value (or +-inf)
        assert np.array_equal(g, (wb >> 16).astype(np.uint16))
    # negative zero survives
    neg0 = (want32 == 0) & np.signbit(want32)
    assert neg0.any()


def test_decode_rows_window_of_a_larger_expert():
    x, packed, scales, sel, p, shared = random_case(3, 1, 3, 1, 5, 37, "fp32", 100, 160)
    got = mx.decode_rows(torch.from_numpy(packed).to(DEV), torch.from_numpy(scales).to(DEV), 2, 11, 20)
    want = oracle.decode_rows(packed[2, 11:31], scales[2, 11:31]).astype(np.float32)
    assert np.array_equal(got.cpu().numpy().view(np.uint32), want.view(np.uint32))


# ------------------------------------------------------------------ printed examples

@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_printed_examples_on_gpu(dtype):
    td = _tdtype(dtype)
    # byte 0x21 at scale 128 decodes to (1.0, 2.0) in this order
    packed = torch.zeros((1, 1, 1, 16), dtype=torch.uint8, device=DEV)
    packed[0, 0, 0, 0] = 0x21
    scales = torch.full((1, 1, 1), 128, dtype=torch.uint8, device=DEV)
    for pos, want in ((0, 1.0), (1, 2.0)):
        x = torch.zeros((1, 32), dtype=td, device=DEV)
        x[0, pos] = 1
        y = mx.mxfp4_expert_linear(x, packed, scales, torch.tensor([[0]], device=DEV),
                                   torch.tensor([[1.0]], device=DEV), torch.zeros((1, 1), dtype=td, device=DEV))
        assert y.dtype == td and y.shape == (1, 1)
        assert float(y[0, 0]) == want
    # every byte 0x22, scale 127, ones input: 32.0
    y = mx.mxfp4_expert_linear(torch.ones((1, 32), dtype=td, device=DEV),
                               torch.full((1, 1, 1, 16), 34, dtype=torch.uint8, device=DEV),
                               torch.full((1, 1, 1), 127, dtype=torch.uint8, device=DEV),
                               torch.tensor([[0]], device=DEV), torch.tensor([[1.0]], device=DEV),
                               torch.zeros((1, 1), dtype=td, device=DEV))
    assert float(y[0, 0]) == 32.0


# ------------------------------------------------------------------ bucketing

def _bucket_case(name):
    if name in workloads.WORKLOADS:
        return workloads.make_inputs(name).sel, workloads.WORKLOADS[name].E
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    if name == "invalid":
        sel = rng.integers(-3, 9, (37, 3)).astype(np.int32)
        return sel, 6
    if name == "one_expert":
        return np.zeros((2000, 2), np.int32), 1
    if name == "duplicates":
        return rng.integers(0, 7, (300, 5)).astype(np.int32), 7
    if name == "many_experts":
        return rng.integers(0, 8192, (3000, 8)).astype(np.int32), 8192
    raise KeyError(name)


@pytest.mark.parametrize("algo", [_abi.FLAG_BUCKET_ONE_BLOCK, _abi.FLAG_BUCKET_MULTI_BLOCK])
@pytest.mark.parametrize("case", ["tiny", "decode", "decode8", "prefill", "skewed", "invalid", "one_expert",
                                  "duplicates", "many_experts"])
def test_bucketing_bit_exact(case, algo):
    sel, E = _bucket_case(case)
    say(f"bucket {case} algo={algo:#x} P={sel.size} E={E}")
    want = oracle.bucket_pairs(sel, E)
    got = mx.bucket(torch.from_numpy(sel).to(DEV), E, algo)
    torch.cuda.synchronize()
    g = {k: v.cpu().numpy() for k, v in got.items()}
    nv = int(want["offsets"][-1])
    assert np.array_equal(g["count"], want["count"])
    assert np.array_equal(g["offsets"], want["offsets"])
    assert np.array_equal(g["perm"][:nv], want["perm"])
    assert np.all(g["perm"][nv:] == -7)  # untouched past the valid pairs
    assert np.array_equal(g["slot_of_pair"], want["slot_of_pair"])
    assert int(g["n_invalid"][0]) == want["n_invalid"]


# ------------------------------------------------------------------ workloads

@functools.lru_cache(maxsize=1)
def _workload_dev(name):
    inp = workloads.make_inputs(name, n_routing_sets=2)
    say(f"uploading {name}")
    return inp, upload(inp.x, inp.packed, inp.scales, inp.sel, inp.p, inp.shared, inp.workload.dtype)


def _sample_rows(O, n, seed):
    """n random output rows, the tile edges 0, 127, 128, O - 1, and one
    random row in every 128-row tile, so that every N-tile of every kernel is
    checked."""
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(O, size=min(n, O), replace=False).tolist())
    rows.update({0, O - 1, min(O - 1, 127), min(O - 1, 128)})
    rows.update(int(rng.integers(t, min(t + 128, O))) for t in range(0, O, 128))
    return np.array(sorted(rows))


def _tokens_of_every_kind(sel, E, n_random, seed):
    """Tokens whose pairs reach the most-used and the least-used (non-empty)
    experts, plus n_random others."""
    counts = np.bincount(sel.ravel(), minlength=E)
    used = np.nonzero(counts)[0]
    hot, cold = int(used[np.argmax(counts[used])]), int(used[np.argmin(counts[used])])
    toks = {int(np.nonzero((sel == hot).any(axis=1))[0][0]), int(np.nonzero((sel == cold).any(axis=1))[0][0])}
    rng = np.random.default_rng(seed)
    toks.update(rng.choice(sel.shape[0], size=n_random, replace=False).tolist())
    return np.array(sorted(toks)), hot, cold


# decode-shaped kernels: row-contiguous (default) and 16-row MFMA tiles
GEMV_KERNELS = [0, _abi.FLAG_GEMV_MFMA]


@pytest.mark.parametrize("kernel", GEMV_KERNELS)
@pytest.mark.parametrize("name", ["tiny", "decode"])
def test_small_workloads_full_oracle(name, kernel):
    inp, d = _workload_dev(name)
    say(f"workload {name} full oracle kernel={kernel}")
    ref = oracle.expert_linear(inp.x, inp.packed, inp.scales, inp.sel, inp.p, inp.shared)
    y = run(d, flags=kernel)
    assert y.dtype == torch.float32 and tuple(y.shape) == ref.shape
    assert_fp32_close(host64(y), ref, name)
    # second routing draw on the same weights
    sel2, p2 = inp.routing_sets[1]
    ref2 = oracle.expert_linear(inp.x, inp.packed, inp.scales, sel2, p2, inp.shared)
    y2 = run(d, sel=torch.from_numpy(sel2).to(DEV), p=torch.from_numpy(p2).to(DEV), flags=kernel)
    assert_fp32_close(host64(y2), ref2, name + " routing set 1")


@pytest.mark.parametrize("name,nrows", [("decode8", 160), ("prefill", 48), ("skewed", 40)])
def test_large_workloads_sampled_rows(name, nrows):
    inp, d = _workload_dev(name)
    w = inp.workload
    rows = _sample_rows(w.O, nrows, 7)
    say(f"workload {name}: GPU run, oracle on {rows.size} rows x {w.T} tokens")
    y = run(d)
    assert y.dtype == torch.bfloat16 and tuple(y.shape) == (w.T, w.O)
    ref = oracle.expert_linear_rows(inp.x, inp.packed, inp.scales, inp.sel, inp.p, inp.shared, rows)
    assert_bf16_close(host64(y)[:, rows], ref, name)
    assert np.all(np.isfinite(host64(y)))


@pytest.mark.parametrize("name", ["prefill", "skewed"])
def test_large_workloads_full_rows_of_some_tokens(name):
    # every output feature of tokens that reach the hottest and the coldest
    # expert (and a few others), so that every M-tile kind and N-tile is read
    inp, d = _workload_dev(name)
    toks, hot, cold = _tokens_of_every_kind(inp.sel, inp.workload.E, 3, 11)
    say(f"workload {name}: all rows of tokens {toks.tolist()} (hot expert {hot}, cold expert {cold})")
    y = host64(run(d))[toks]
    ref = oracle.expert_linear(inp.x[toks], inp.packed, inp.scales, inp.sel[toks], inp.p[toks], inp.shared[toks])
    assert_bf16_close(y, ref, f"{name}, tokens {toks.tolist()}")


def test_prefill_fp32_activations_sampled():
    # the prefill shape with genuine fp32 activations: the grouped GEMM on the
    # three-piece bf16 split, at the fp32 bar
    w = workloads.WORKLOADS["prefill_fp32"]
    inp = workloads.make_inputs(w)
    assert mx.select_path(w.T, w.E, w.O, w.G, w.K, _abi.DTYPE_F32) == _abi.PATH_GEMM
    d = upload(inp.x, inp.packed, inp.scales, inp.sel, inp.p, inp.shared, "fp32")
    rows = _sample_rows(w.O, 16, 12)
    say(f"prefill fp32: GPU run, oracle on {rows.size} rows x {w.T} tokens")
    y = run(d)
    assert y.dtype == torch.float32
    ref = oracle.expert_linear_rows(inp.x, inp.packed, inp.scales, inp.sel, inp.p, inp.shared, rows)
    assert_fp32_close(host64(y)[:, rows], ref, "prefill fp32")
    toks, _, _ = _tokens_of_every_kind(inp.sel, w.E, 1, 13)
    ref_t = oracle.expert_linear(inp.x[toks], inp.packed, inp.scales, inp.sel[toks], inp.p[toks], inp.shared[toks])
    assert_fp32_close(host64(y)[toks], ref_t, f"prefill fp32 tokens {toks.tolist()}")


def test_decode8_both_paths():
    inp, d = _workload_dev("decode8")
    rows = _sample_rows(inp.workload.O, 96, 8)
    ref = oracle.expert_linear_rows(inp.x, inp.packed, inp.scales, inp.sel, inp.p, inp.shared, rows)
    for flags in (_abi.FLAG_FORCE_GEMV, _abi.FLAG_FORCE_GEMV | _abi.FLAG_GEMV_MFMA, _abi.FLAG_FORCE_GEMM):
        say(f"decode8 flags={flags}")
        y = host64(run(d, flags=flags))
        assert_bf16_close(y[:, rows], ref, f"decode8 flags={flags}")


# ------------------------------------------------------------------ paths, thresholds, edges

def _gemv_switch(E, O, G, K, dtype):
    """The smallest T that the default path sends to the grouped GEMM."""
    for T in range(1, 200):
        if mx.select_path(T, E, O, G, K, dtype) == _abi.PATH_GEMM:
            return T
    raise AssertionError("no switch below 200 tokens")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("K", [1, 2, 4, 8])
def test_threshold_sweep(K, dtype):
    # one token below, at and above the switch between the decode-shaped path
    # and the grouped GEMM (the switch is where one fused launch no longer
    # takes every pair): every path on the same inputs, and the default call
    # equal bit for bit to the forced path it chose
    E, O, G = 40, 136, 8
    dt = _abi.DTYPE_BF16 if dtype == "bf16" else _abi.DTYPE_F32
    Ts = _gemv_switch(E, O, G, K, dt)
    assert (Ts - 1) * K <= 64  # never more than 64 pairs in one fused launch
    for T in (Ts - 1, Ts, Ts + 1):
        case = random_case(100 * K + T, T, E, K, G, O, dtype)
        d = upload(*case, dtype)
        want_path = _abi.PATH_GEMV if T < Ts else _abi.PATH_GEMM
        assert mx.select_path(T, E, O, G, K, dt) == want_path
        ref = oracle.expert_linear(*case)
        results = {}
        for flags in (0, _abi.FLAG_FORCE_GEMV, _abi.FLAG_FORCE_GEMV | _abi.FLAG_GEMV_MFMA, _abi.FLAG_FORCE_GEMM):
            y = host64(run(d, flags=flags))
            assert_close(y, ref, dtype, f"K={K} T={T} flags={flags}")
            results[flags] = y
        assert np.array_equal(results[0], results[_abi.FLAG_FORCE_GEMV if T < Ts else _abi.FLAG_FORCE_GEMM])


EDGE_CASES = [
    # T, E, K, G, O, distinct
    (1, 1, 1, 1, 1, True),
    (1, 3, 1, 1, 17, True),
    (2, 5, 5, 3, 33, True),      # every expert chosen by every token, odd G
    (3, 8, 2, 7, 130, True),     # ragged 128-row N-tile
    (5, 6, 4, 2, 16, False),     # duplicates within a token
    (9, 64, 2, 5, 257, True),    # most experts empty
    (40, 3, 2, 4, 64, False),    # many rows per expert, duplicates
    (33, 200, 8, 3, 96, True),   # P spans a ragged 128-row M-tile
    (20, 4, 2, 33, 40, True),    # odd G over three 16-group scale chunks
    (17, 3, 3, 47, 129, True),   # odd G, ragged N-tile, scale rows at every byte offset
    (6, 5, 2, 32, 36, True),     # G an exact multiple of the scale chunk
    (150, 2, 2, 6, 516, True),   # M-tiles of 128 and 22 pairs, a 4-row last N-tile
    (70, 1, 1, 90, 260, True),   # one expert, 70 pairs, the prefill input width
]


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("case", EDGE_CASES, ids=lambda c: "T{}E{}K{}G{}O{}{}".format(*c[:5], "" if c[5] else "dup"))
def test_edge_shapes(case, dtype):
    T, E, K, G, O, distinct = case
    say(f"edge {case} {dtype}")
    host = random_case(sum(case[:5]), T, E, K, G, O, dtype, distinct=distinct)
    d = upload(*host, dtype)
    ref = oracle.expert_linear(*host)
    mf = _abi.FLAG_GEMV_MFMA
    flag_sets = [0, _abi.FLAG_FORCE_GEMV, _abi.FLAG_FORCE_GEMV | mf, _abi.FLAG_FORCE_GEMM]
    for flags in flag_sets:
        y = run(d, flags=flags)
        assert y.dtype == _tdtype(dtype)
        assert_close(host64(y), ref, dtype, f"{case} flags={flags}")


# Prefill-shaped GEMM on canonical weights with O % 4 == 0 (the register-decode
# kernel): input widths around its 4-group chunks and 8-group scale windows
# (partial chunks, partial windows, groups past G), rows across 128-row
# fragments and 512-row N-tiles, scale rows at every byte offset.
GEMM_WINDOW_CASES = [
    # T, E, K, G, O
    (40, 3, 2, 1, 20),
    (40, 3, 2, 3, 132),
    (40, 3, 2, 4, 20),
    (40, 3, 2, 5, 132),
    (40, 3, 2, 7, 20),
    (40, 3, 2, 8, 132),
    (40, 3, 2, 9, 516),
    (40, 3, 2, 12, 20),
    (40, 3, 2, 15, 132),
    (40, 3, 2, 16, 20),
    (40, 3, 2, 17, 132),
    (40, 3, 2, 23, 20),
    (130, 2, 2, 33, 268),
]


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("case", GEMM_WINDOW_CASES, ids=lambda c: "T{}E{}K{}G{}O{}".format(*c))
def test_gemm_chunk_and_scale_window_edges(case, dtype):
    T, E, K, G, O = case
    say(f"gemm window edges {case} {dtype}")
    host = random_case(1000 + 7 * G + O, T, E, K, G, O, dtype)
    d = upload(*host, dtype)
    ref = oracle.expert_linear(*host)
    y = run(d, flags=_abi.FLAG_FORCE_GEMM)
    assert_close(host64(y), ref, dtype, f"{case} forced GEMM")


ONE_TOKEN_CASES = [
    # E, K, G, O, distinct: the one-token kernel's lane layouts (lanes per row
    # 64 / 32 / 16 / 2 / 1), ragged row sets, G up to its limit, many slots
    (4, 2, 90, 5760, True),      # 32 lanes per row, 3 groups each (the decode workload's G)
    (6, 3, 64, 130, True),       # 64 lanes per row, one group each; O not a multiple of anything
    (5, 1, 2, 33, True),         # 2 lanes per row, 32 rows per wave-wide load
    (3, 2, 1, 7, True),          # 1 lane per row, 64 rows per load
    (9, 8, 7, 100, True),        # 8 lanes per row
    (80, 64, 13, 40, True),      # 64 slots
    (7, 5, 256, 64, True),       # the largest G on this kernel (4 groups per lane)
    (7, 5, 257, 64, True),       # one group more: the row-contiguous kernel's layout
    (3, 6, 11, 50, False),       # duplicates
    (128, 4, 224, 96, True),     # the decode8 input width
]


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("case", ONE_TOKEN_CASES, ids=lambda c: "E{}K{}G{}O{}{}".format(*c[:4], "" if c[4] else "dup"))
def test_one_token(case, dtype):
    # T = 1 on the default path (the one-token kernel, activations in
    # registers) against the oracle and against the 16-row MFMA kernel
    E, K, G, O, distinct = case
    say(f"one token {case} {dtype}")
    host = random_case(sum(case[:4]) + 7, 1, E, K, G, O, dtype, distinct=distinct)
    d = upload(*host, dtype)
    ref = oracle.expert_linear(*host)
    y = host64(run(d))
    assert_close(y, ref, dtype, f"one token {case}")
    y_mfma = host64(run(d, flags=_abi.FLAG_FORCE_GEMV | _abi.FLAG_GEMV_MFMA))
    assert_close(y_mfma, ref, dtype, f"one token {case}, MFMA kernel")
    assert np.array_equal(y, host64(run(d))), "not deterministic"


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_one_token_invalid_index_and_large_scales(dtype):
    E, K, G, O = 5, 4, 37, 70
    x, packed, scales, sel, p, shared = random_case(61, 1, E, K, G, O, dtype)
    x = (x * np.float32(2.0 ** -100)).astype(np.float32)
    if dtype == "bf16":
        x = workloads.round_to_bf16(x)
    scales = np.random.default_rng(62).integers(250, 256, scales.shape).astype(np.uint8)
    ref = oracle.expert_linear(x, packed, scales, sel, p, shared)
    y = host64(run(upload(x, packed, scales, sel, p, shared, dtype)))
    assert_close_at_scale(y, ref, dtype, 2.0 ** 28, "one token, scales 250..255")
    # an index outside [0, E) contributes nothing and is reported under CHECK
    bad = sel.copy()
    bad[0, 1] = E + 3
    keep = np.ones_like(p)
    keep[0, 1] = 0
    d = upload(x, packed, scales, bad, p, shared, dtype)
    ref_bad = oracle.expert_linear(x, packed, scales, np.where(keep > 0, bad, 0), p * keep, shared)
    y_bad = host64(run(d))
    assert_close_at_scale(y_bad, ref_bad, dtype, 2.0 ** 28, "one token, invalid index dropped")
    with pytest.raises(_abi.Mxfp4Error) as e:
        mx.moe_linear(d.x, d.packed, d.scales, d.sel, d.p, d.shared, flags=_abi.FLAG_CHECK)
    assert e.value.status == _abi.ERR_INVALID_INDEX


@pytest.mark.parametrize("kernel", GEMV_KERNELS)
def test_fp32_many_tokens_uses_chunked_fused_launches(kernel):
    # more pairs than one fused launch takes: the fp32 path splits tokens into chunks
    host = random_case(5, 300, 16, 3, 2, 40, "fp32")
    d = upload(*host, "fp32")
    assert_fp32_close(host64(run(d, flags=kernel)), oracle.expert_linear(*host), "fp32 T=300")


LARGE_SCALE_FLAGS = [("fp32", 0), ("fp32", _abi.FLAG_GEMV_MFMA), ("fp32", _abi.FLAG_FORCE_GEMM),
                     ("bf16", _abi.FLAG_FORCE_GEMV), ("bf16", _abi.FLAG_FORCE_GEMV | _abi.FLAG_GEMV_MFMA),
                     ("bf16", _abi.FLAG_FORCE_GEMM)]


@pytest.mark.parametrize("dtype,flags", LARGE_SCALE_FLAGS)
def test_largest_scales_against_oracle(dtype, flags):
    # scale bytes 253..255 (2^126..2^128): E2M1 * 2^(s-127) overflows fp32
    # and bf16 for the larger codes, the layer's result does not; tiny
    # activations keep every output finite, so the exact (float64) result is
    # the reference, on every path
    T, E, K, G, O = 3, 4, 2, 5, 40
    x, packed, scales, sel, p, shared = random_case(55, T, E, K, G, O, dtype)
    x = (x * np.float32(2.0 ** -100)).astype(np.float32)
    if dtype == "bf16":
        x = workloads.round_to_bf16(x)
    scales = np.broadcast_to((255 - np.arange(G) % 3).astype(np.uint8), scales.shape).copy()
    d = upload(x, packed, scales, sel, p, shared, dtype)
    ref = oracle.expert_linear(x, packed, scales, sel, p, shared)
    assert np.all(np.isfinite(ref)) and np.abs(ref).max() > 1e6
    # the data is unit-scale data times 2^(128 - 100)
    assert_close_at_scale(host64(run(d, flags=flags)), ref, dtype, 2.0 ** 28, f"scales 253..255 {dtype} flags={flags}")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_largest_scales_same_result_on_both_sides_of_the_switch(dtype):
    # the same large-scale weights with one token fewer and one token more
    # than the decode-shaped path takes: both calls (decode-shaped, grouped
    # GEMM) finite and at the bar against the exact result; the shared
    # tokens agree within the bar
    E, K, G, O = 6, 4, 37, 130
    dt = _abi.DTYPE_BF16 if dtype == "bf16" else _abi.DTYPE_F32
    Ts = _gemv_switch(E, O, G, K, dt)
    x, packed, scales, sel, p, shared = random_case(57, Ts, E, K, G, O, dtype)
    x = (x * np.float32(2.0 ** -100)).astype(np.float32)
    if dtype == "bf16":
        x = workloads.round_to_bf16(x)
    scales = np.random.default_rng(58).integers(250, 256, scales.shape).astype(np.uint8)
    ys = {}
    for T in (Ts - 1, Ts):
        args = (x[:T], packed, scales, sel[:T], p[:T], shared[:T])
        assert mx.select_path(T, E, O, G, K, dt) == (_abi.PATH_GEMV if T < Ts else _abi.PATH_GEMM)
        ref = oracle.expert_linear(*args)
        assert np.all(np.isfinite(ref)) and np.abs(ref).max() > 1e6
        y = host64(run(upload(*args, dtype)))
        assert np.all(np.isfinite(y)), f"T={T}: non-finite output"
        # unit-scale data times 2^(128 - 100)
        assert_close_at_scale(y, ref, dtype, 2.0 ** 28, f"scales 250..255 T={T}")
        ys[T] = y
    assert_close_at_scale(ys[Ts][:Ts - 1], ys[Ts - 1], dtype, 2.0 ** 28, "the tokens both calls share")


def test_empty_batch():
    d = upload(*random_case(1, 2, 4, 2, 2, 8, "fp32"), "fp32")
    y = mx.moe_linear(d.x[:0], d.packed, d.scales, d.sel[:0], d.p[:0], d.shared[:0])
    assert y.shape == (0, 8)


# ------------------------------------------------------------------ invariants

@pytest.mark.parametrize("flags", [_abi.FLAG_FORCE_GEMM, _abi.FLAG_FORCE_GEMV, _abi.FLAG_FORCE_GEMV | _abi.FLAG_GEMV_MFMA])
def test_largest_scales_with_bf16_weights_in_range(flags):
    # scale bytes 253..255 with codes small enough that every decoded weight
    # is a finite bf16 value (|E2M1| <= 1.5 at 253/254, <= 0.5 at 255): the
    # grouped GEMM's shifted decode of such tiles
    # is checked against the float64 oracle
    T, E, K, G, O = 20, 3, 2, 37, 70
    x, packed, scales, sel, p, shared = random_case(91, T, E, K, G, O, "bf16")
    x = workloads.round_to_bf16((x * np.float32(2.0 ** -110)).astype(np.float32))
    scales = np.random.default_rng(92).integers(253, 256, scales.shape).astype(np.uint8)
    small = np.array([0, 1, 8, 9], np.uint8)        # 0, 0.5, -0, -0.5
    mid = np.array([0, 1, 2, 3, 8, 9, 10, 11], np.uint8)  # |E2M1| <= 1.5
    rng = np.random.default_rng(93)
    lo255, hi255 = rng.choice(small, packed.shape), rng.choice(small, packed.shape)
    lo, hi = rng.choice(mid, packed.shape), rng.choice(mid, packed.shape)
    is255 = (scales == 255)[..., None]
    packed = np.where(is255, lo255 | (hi255 << 4), lo | (hi << 4)).astype(np.uint8)
    d = upload(x, packed, scales, sel, p, shared, "bf16")
    ref = oracle.expert_linear(x, packed, scales, sel, p, shared)
    assert np.all(np.isfinite(ref))
    assert_close(host64(run(d, flags=flags)), ref, "bf16", f"scales 253..255, finite weights, flags={flags}")


@pytest.mark.parametrize("dtype,flags", [("fp32", 0), ("fp32", _abi.FLAG_GEMV_MFMA), ("bf16", _abi.FLAG_FORCE_GEMV),
                                         ("bf16", _abi.FLAG_FORCE_GEMV | _abi.FLAG_GEMV_MFMA),
                                         ("bf16", _abi.FLAG_FORCE_GEMM)])
def test_invariants(dtype, flags):
    T, E, K, G, O = 6, 12, 3, 6, 200
    x, packed, scales, sel, p, shared = random_case(77, T, E, K, G, O, dtype)
    zero = np.zeros_like(shared)
    d = upload(x, packed, scales, sel, p, zero, dtype)
    y = run(d, flags=flags)
    y_again = run(d, flags=flags)
    assert torch.equal(y, y_again), "not deterministic"
    # unselected experts do not matter, bit for bit
    pk2, sc2 = packed.copy(), scales.copy()
    rng = np.random.default_rng(1)
    for e in set(range(E)) - set(np.unique(sel).tolist()):
        pk2[e] = rng.integers(0, 256, pk2[e].shape)
        sc2[e] = 255
    assert torch.equal(run(upload(x, pk2, sc2, sel, p, zero, dtype), flags=flags), y)
    # b ^ 0x88 flips every sign: the routed part is negated. Within the
    # tolerance bar, not bit for bit: the MFMA's fp32 accumulation is not
    # correctly rounded and not sign-symmetric in the last bit (measured on
    # MI355X: 183 of 51,200 outputs of v_mfma_f32_16x16x32_bf16 differ when
    # A is negated)
    yn = run(upload(x, packed ^ np.uint8(0x88), scales, sel, p, zero, dtype), flags=flags)
    assert_close(host64(yn), -host64(y), dtype, "sign flip")
    # every scale + 1 doubles the routed part exactly
    y2 = run(upload(x, packed, scales + np.uint8(1), sel, p, zero, dtype), flags=flags)
    assert torch.equal(y2, 2 * y)
    # swapping the nibbles of every byte equals swapping inputs 2j <-> 2j+1
    xs = x.copy()
    xs[:, 0::2], xs[:, 1::2] = x[:, 1::2], x[:, 0::2]
    sw = ((packed & 0x0F) << 4) | (packed >> 4)
    ys = run(upload(xs, sw, scales, sel, p, zero, dtype), flags=flags)
    assert_close(host64(ys), host64(y), dtype, "nibble swap")
    # linear in p
    p2 = np.random.default_rng(2).random(p.shape).astype(np.float32)
    ya = host64(run(d, p=torch.from_numpy(p2).to(DEV), flags=flags))
    yb = host64(run(d, p=torch.from_numpy(p + p2).to(DEV), flags=flags))
    ref = oracle.expert_linear(x, packed, scales, sel, p + p2, zero)
    assert_close(yb, ref, dtype, "p1+p2")
    assert_close(host64(y) + ya, ref, dtype, "y(p1)+y(p2)")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_inputs_untouched_and_in_place(dtype):
    host = random_case(9, 4, 6, 2, 3, 50, dtype)
    d = upload(*host, dtype)
    before = [t.clone() for t in (d.x, d.packed, d.scales, d.sel, d.p, d.shared)]
    y = run(d)
    for a, b in zip((d.x, d.packed, d.scales, d.sel, d.p, d.shared), before):
        assert torch.equal(a, b)
    assert y.data_ptr() != d.shared.data_ptr()
    out = d.shared.clone()
    y2 = run(d, out=None)
    y3 = mx.moe_linear(d.x, d.packed, d.scales, d.sel, d.p, out, out=out)  # y == shared
    torch.cuda.synchronize()
    assert y3.data_ptr() == out.data_ptr() and torch.equal(y3, y2)


def test_out_of_range_index_reported_with_check_flag():
    x, packed, scales, sel, p, shared = random_case(11, 5, 7, 2, 2, 24, "fp32")
    sel[2, 1] = 7
    sel[4, 0] = -1
    d = upload(x, packed, scales, sel, p, shared, "fp32")
    with pytest.raises(mx.Mxfp4Error) as e:
        run(d, flags=_abi.FLAG_CHECK)
    assert e.value.status == _abi.ERR_INVALID_INDEX
    y = run(d)  # without the flag: the bad slots contribute nothing
    sel_ok, p_ok = sel.copy(), p.copy()
    for t, k in ((2, 1), (4, 0)):
        sel_ok[t, k], p_ok[t, k] = 0, 0.0
    assert_fp32_close(host64(y), oracle.expert_linear(x, packed, scales, sel_ok, p_ok, shared), "invalid dropped")


def test_plain_entry_points_match_ex():
    lib = _abi.lib()
    for dtype in ("fp32", "bf16"):
        host = random_case(12, 3, 5, 2, 4, 40, dtype)
        d = upload(*host, dtype)
        y_ex = run(d)
        y = torch.empty_like(d.shared)
        fn = lib.mxfp4_moe_linear if dtype == "fp32" else lib.mxfp4_moe_linear_bf16
        st = fn(d.x.data_ptr(), d.packed.data_ptr(), d.scales.data_ptr(), d.sel.data_ptr(), d.p.data_ptr(),
                d.shared.data_ptr(), y.data_ptr(), 3, 5, 40, 4, 2, torch.cuda.current_stream().cuda_stream)
        assert st == 0
        torch.cuda.synchronize()
        assert torch.equal(y, y_ex)
    # prefill-shaped plain call (allocates its workspace on the stream)
    host = random_case(13, 40, 6, 2, 3, 64, "bf16")
    d = upload(*host, "bf16")
    y = torch.empty_like(d.shared)
    st = lib.mxfp4_moe_linear_bf16(d.x.data_ptr(), d.packed.data_ptr(), d.scales.data_ptr(), d.sel.data_ptr(),
                                   d.p.data_ptr(), d.shared.data_ptr(), y.data_ptr(), 40, 6, 64, 3, 2,
                                   torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    assert torch.equal(y, run(d))


# ------------------------------------------------------------------ SwiGLU expert block

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


def upload_swiglu(x, gu_p, gu_s, dn_p, dn_s, sel, p, shared):
    def u8(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV).to(torch.bfloat16)

    return (bf(x), u8(gu_p), u8(gu_s), u8(dn_p), u8(dn_s), u8(sel.astype(np.int32)),
            torch.from_numpy(np.ascontiguousarray(p, dtype=np.float32)).to(DEV), bf(shared))


def run_swiglu(d, out=None):
    y = mx.moe_swiglu(*d, out=out)
    torch.cuda.synchronize()
    return y


SWIGLU_CASES = [
    # T, E, K, G, F, O, distinct
    (1, 3, 1, 1, 32, 8, True),
    (5, 4, 2, 2, 64, 40, True),
    (33, 6, 3, 3, 96, 130, True),     # F = 1.5 feature tiles, ragged N-tile of the down projection
    (70, 16, 4, 5, 160, 72, True),    # P spans several 128-row M-tiles, odd G
    (40, 3, 2, 17, 64, 33, False),    # duplicates within a token, G over two scale chunks
]


@pytest.mark.parametrize("case", SWIGLU_CASES, ids=lambda c: "T{}E{}K{}G{}F{}O{}{}".format(*c[:6], "" if c[6] else "dup"))
def test_swiglu_against_oracle(case):
    T, E, K, G, F, O, distinct = case
    say(f"swiglu {case}")
    host = swiglu_case(sum(case[:6]), T, E, K, G, F, O, distinct=distinct)
    y = run_swiglu(upload_swiglu(*host))
    assert y.dtype == torch.bfloat16 and tuple(y.shape) == (T, O)
    assert_bf16_close(host64(y), oracle.expert_swiglu(*host), f"swiglu {case}")


def test_swiglu_invariants():
    host = list(swiglu_case(7, 24, 10, 3, 3, 96, 50))
    x, gu_p, gu_s, dn_p, dn_s, sel, p, shared = host
    d = upload_swiglu(*host)
    y = run_swiglu(d)
    assert torch.equal(y, run_swiglu(d)), "not deterministic"
    # unselected experts do not matter, bit for bit
    gu2, dn2, gs2, ds2 = gu_p.copy(), dn_p.copy(), gu_s.copy(), dn_s.copy()
    rng = np.random.default_rng(8)
    for e in set(range(10)) - set(np.unique(sel).tolist()):
        gu2[e] = rng.integers(0, 256, gu2[e].shape)
        dn2[e] = rng.integers(0, 256, dn2[e].shape)
        gs2[e] = 255
        ds2[e] = 255
    assert torch.equal(run_swiglu(upload_swiglu(x, gu2, gs2, dn2, ds2, sel, p, shared)), y)
    # in place on shared
    y2 = d[7].clone()
    run_swiglu(d[:7] + (y2,), out=y2)
    assert torch.equal(y2, y)
    # zero gate rows: the routed part vanishes, y = shared exactly
    gz = gu_p.copy()
    gz[:, :96] = 0
    assert torch.equal(run_swiglu(upload_swiglu(x, gz, gu_s, dn_p, dn_s, sel, p, shared)), d[7])


def test_swiglu_full_shapes_sampled():
    # the gate/up shape of the decode8 workload (I = 7168, 2F = 4096) feeding
    # the skewed workload's down shape (F = 2048 -> O = 7168), E = 384, K = 8;
    # only the selected experts are drawn (the others are never read), and the
    # oracle checks two tokens on a sample of output rows
    T, E, K, G, F, O = 8, 384, 8, 224, 2048, 7168
    rng = np.random.default_rng(2026)
    x = workloads.round_to_bf16(rng.standard_normal((T, 32 * G)).astype(np.float32))
    shared = workloads.round_to_bf16(rng.standard_normal((T, O)).astype(np.float32))
    sel = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    p = rng.random((T, K)).astype(np.float32)
    used = np.unique(sel)
    gu_p = torch.empty((E, 2 * F, G, 16), dtype=torch.uint8, device=DEV)
    gu_s = torch.empty((E, 2 * F, G), dtype=torch.uint8, device=DEV)
    dn_p = torch.empty((E, O, F // 32, 16), dtype=torch.uint8, device=DEV)
    dn_s = torch.empty((E, O, F // 32), dtype=torch.uint8, device=DEV)
    hp = {}
    for e in used:
        r = np.random.default_rng(int(e) + 99)
        hp[e] = (r.integers(0, 256, (2 * F, G, 16), dtype=np.uint8), r.integers(118, 125, (2 * F, G), dtype=np.uint8),
                 r.integers(0, 256, (O, F // 32, 16), dtype=np.uint8), r.integers(118, 125, (O, F // 32), dtype=np.uint8))
        for dst, src in zip((gu_p, gu_s, dn_p, dn_s), hp[e]):
            dst[int(e)].copy_(torch.from_numpy(src))
    bf = lambda a: torch.from_numpy(a).to(DEV).to(torch.bfloat16)  # noqa: E731
    d = (bf(x), gu_p, gu_s, dn_p, dn_s, torch.from_numpy(sel).to(DEV), torch.from_numpy(p).to(DEV), bf(shared))
    y = host64(run_swiglu(d))
    toks = [0, 5]
    rows = np.sort(np.random.default_rng(3).choice(O, 96, replace=False))

    class Lazy:
        def __init__(self, i):
            self.i = i

        def __len__(self):
            return E

        def __getitem__(self, e):
            return hp[int(e)][self.i]

    ref = oracle.expert_swiglu_rows(x[toks], Lazy(0), Lazy(1), Lazy(2), Lazy(3), sel[toks], p[toks], shared[toks], rows)
    assert_bf16_close(y[toks][:, rows], ref, "swiglu full shapes, 2 tokens x 96 rows")
