"""GPU parity of the prefill-shaped grouped GEMM (canonical and prepared
weights) around the M-tile boundary: experts whose pair count just passes a multiple of the
128-pair tile (129, 144, 145, 261 pairs, ...), where the few pairs left over
form a partial tile of their own in the bucketing's tile list.

Two checks per case, through the C ABI:
* the whole layer against the float64 oracle at the bf16 bar (relative L2
  <= 1e-2, every output within 1e-2 (|y_ref| + rms(y_ref)));
* a pair's partial row depends only on its token and expert - every tile
  adds the same products in the same order - so the tokens of the pairs
  left over past an expert's full tiles give the same bits when they are
  run on their own (then in small tiles of their own).
The SwiGLU block rounds its hidden activations h to bf16 between the two
GEMMs (the oracle keeps them in float64): each lands within one bf16 unit
(2^-8 relative) of its exact value, as its fp32 value may sit on the other
side of a rounding boundary, so that case's elementwise bound adds
2^-8 sum_k p_k sum_f |D_e[o, f]| |h_f| (heavy-tailed h makes this term
matter for a few outputs of the largest case).
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
BF16_ELEM = 1e-2
MT = 128  # pairs per full M-tile


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def host64(y):
    return y.float().cpu().numpy().astype(np.float64)


def assert_bf16_close(y, ref, what, extra=0.0):
    r = float(np.linalg.norm(y - ref) / max(np.linalg.norm(ref), 1e-300))
    err = np.abs(y - ref)
    bound = BF16_ELEM * (np.abs(ref) + float(np.sqrt(np.mean(ref * ref)))) + extra
    worst = float(np.max(err / np.maximum(bound, 1e-300)))
    say(f"  {what}: rel L2 {r:.3e}, max err/elementwise bound {worst:.3f}")
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    assert r <= BF16_REL_L2, f"{what}: relative L2 {r:.3e}"
    assert np.all(err <= bound), f"{what}: an output misses the elementwise bound by {worst:.3g}x"


def routing_with_counts(counts, K, seed):
    """sel [T, K] with exactly counts[e] pairs on expert e and distinct experts
    within a token (T = sum(counts) / K; needs max(counts) <= T)."""
    P = int(sum(counts))
    assert P % K == 0
    T = P // K
    assert max(counts) <= T
    flat = np.repeat(np.arange(len(counts)), counts)  # sorted by expert
    sel = flat.reshape(K, T).T.copy()                 # slot k of token t: flat[k T + t]
    rng = np.random.default_rng(seed)
    sel = sel[rng.permutation(T)]                     # tokens in random order
    for t in range(T):
        assert len(set(sel[t].tolist())) == K
    return sel.astype(np.int32)


def leftover_tokens(sel, counts):
    """Tokens of the pairs past each expert's full tiles when fewer than 32
    pairs are left over: the pairs (in pair order t K + k) of expert e at
    sorted positions 128 floor(c / 128) .. c - 1."""
    K = sel.shape[1]
    toks = set()
    flat = sel.reshape(-1)
    for e, c in enumerate(counts):
        r = c % MT
        if c >= MT and 0 < r < 32:
            pairs = np.nonzero(flat == e)[0]
            toks.update((pairs[c - r:] // K).tolist())
    return np.array(sorted(toks), dtype=np.int64)


def linear_case(seed, counts, K, G, O, xscale=1.0, scale_lo=118, scale_hi=130, big_expert=None):
    rng = np.random.default_rng(seed)
    sel = routing_with_counts(counts, K, seed)
    T, E = sel.shape[0], len(counts)
    x = workloads.round_to_bf16((rng.standard_normal((T, 32 * G)) * xscale).astype(np.float32))
    shared = workloads.round_to_bf16(rng.standard_normal((T, O)).astype(np.float32))
    packed = rng.integers(0, 256, (E, O, G, 16), dtype=np.uint8)
    scales = rng.integers(scale_lo, scale_hi + 1, (E, O, G), dtype=np.uint8)
    if big_expert is not None:
        # scale bytes up to 254 on one expert: the kernel's shifted decode
        scales[big_expert] = rng.integers(244, 255, (O, G), dtype=np.uint8)
    p = rng.random((T, K)).astype(np.float32)
    return x, packed, scales, sel, p, shared


def run_linear(x, packed, scales, sel, p, shared, layout="canonical"):
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV).to(torch.bfloat16)  # noqa: E731
    dv = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)  # noqa: E731
    if layout == "canonical":
        y = mx.moe_linear(bf(x), dv(packed), dv(scales), dv(sel), dv(p), bf(shared), flags=_abi.FLAG_FORCE_GEMM)
    else:
        prep = mx.prepare_bf16(dv(packed), dv(scales))
        y = mx.moe_linear_prepared(bf(x), prep, dv(sel), dv(p), bf(shared))
    torch.cuda.synchronize()
    return y


LINEAR_CASES = [  # seed, counts per expert, K, G, O
    (1, [145, 144, 129, 261, 16, 128, 90, 1], 2, 7, 520),  # left over 17, 16, 1, 5; a lone 16; exactly 128
    (2, [130, 140, 200, 12], 1, 90, 1028),                 # the prefill input width, three N-tiles (the last 4 rows)
    (3, [143, 144, 160, 129, 256, 41], 3, 4, 132),         # one chunk of groups, a 4-row last N-tile
]


LAYOUTS = ["canonical", "prepared"]


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("c", LINEAR_CASES, ids=lambda c: "K{}G{}O{}".format(*c[2:]))
def test_partial_tiles_linear(c, layout):
    seed, counts, K, G, O = c
    say(f"tile boundary linear {c} {layout}")
    host = linear_case(seed, counts, K, G, O)
    y = run_linear(*host, layout=layout)
    assert_bf16_close(host64(y), oracle.expert_linear(*host), f"linear {c} {layout}")
    toks = leftover_tokens(host[3], counts)
    assert toks.size > 0
    x, packed, scales, sel, p, shared = host
    y_own = run_linear(x[toks], packed, scales, sel[toks], p[toks], shared[toks], layout=layout)
    assert torch.equal(y[torch.from_numpy(toks).to(DEV)], y_own), "left-over pairs differ when run on their own"


@pytest.mark.parametrize("layout", LAYOUTS)
def test_partial_tiles_largest_scales(layout):
    # expert 1 (144 pairs: 16 left over) with scale bytes 244..254, activations scaled by 2^-100
    counts = [145, 144, 129, 30]
    say(f"tile boundary largest scales {layout}")
    host = linear_case(9, counts, 2, 6, 260, xscale=2.0 ** -100, big_expert=1)
    y = run_linear(*host, layout=layout)
    assert_bf16_close(host64(y), oracle.expert_linear(*host), f"largest scales {layout}")
    toks = leftover_tokens(host[3], counts)
    x, packed, scales, sel, p, shared = host
    y_own = run_linear(x[toks], packed, scales, sel[toks], p[toks], shared[toks], layout=layout)
    assert torch.equal(y[torch.from_numpy(toks).to(DEV)], y_own)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_partial_tiles_swiglu(layout):
    # the SwiGLU block: the down projection runs over the sorted rows with the same tile list
    counts = [145, 144, 129, 261, 16, 128, 90, 1]
    K, G, F, O = 2, 5, 160, 520
    rng = np.random.default_rng(11)
    sel = routing_with_counts(counts, K, 11)
    T, E = sel.shape[0], len(counts)
    x = workloads.round_to_bf16(rng.standard_normal((T, 32 * G)).astype(np.float32))
    shared = workloads.round_to_bf16(rng.standard_normal((T, O)).astype(np.float32))
    gu_p = rng.integers(0, 256, (E, 2 * F, G, 16), dtype=np.uint8)
    gu_s = rng.integers(118, 127, (E, 2 * F, G), dtype=np.uint8)
    dn_p = rng.integers(0, 256, (E, O, F // 32, 16), dtype=np.uint8)
    dn_s = rng.integers(118, 127, (E, O, F // 32), dtype=np.uint8)
    p = rng.random((T, K)).astype(np.float32)

    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV).to(torch.bfloat16)  # noqa: E731
    dv = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)  # noqa: E731
    prep = mx.prepare_swiglu(dv(gu_p), dv(gu_s), dv(dn_p), dv(dn_s)) if layout == "prepared" else None
    say(f"tile boundary swiglu {layout}")

    def run(rows):
        if prep is None:
            y = mx.moe_swiglu(bf(x[rows]), dv(gu_p), dv(gu_s), dv(dn_p), dv(dn_s), dv(sel[rows]), dv(p[rows]),
                              bf(shared[rows]))
        else:
            y = mx.moe_swiglu_prepared(bf(x[rows]), prep, dv(sel[rows]), dv(p[rows]), bf(shared[rows]))
        torch.cuda.synchronize()
        return y

    y = run(np.arange(T))
    toks = leftover_tokens(sel, counts)
    assert torch.equal(y[torch.from_numpy(toks).to(DEV)], run(toks)), "left-over pairs differ when run on their own"
    ref = oracle.expert_swiglu(x, gu_p, gu_s, dn_p, dn_s, sel, p, shared)
    # sum_k p_k |D_e| |h| per output: the reach of the bf16 rounding of h
    reach = np.zeros((T, O))
    x64 = x.astype(np.float64)
    for e in np.unique(sel):
        ts, ks = np.nonzero(sel == e)
        h = np.abs(oracle.swiglu_hidden(x64[ts], gu_p[e], gu_s[e]))
        D = np.abs(oracle.decode_expert(dn_p[e], dn_s[e]))
        np.add.at(reach, ts, p[ts, ks].astype(np.float64)[:, None] * (h @ D.T))
    assert_bf16_close(host64(y), ref, f"swiglu {layout}", extra=2.0 ** -8 * reach)
