"""GPU parity of the router (mxfp4_moe_route, through its C ABI) against the
float64 oracle.

Bars (written in each check):
* softmax router: the ranking key is the fp32 logit itself, exact on both
  sides, so sel is bit-exact against the oracle, tie order included.
* sigmoid router: the key sigmoid(l) + bias is fp32 on the GPU and float64 in
  the oracle, so keys closer than EPS_KEY may rank either way. A token whose
  oracle keys around the cut and between the chosen are all more than
  EPS_KEY apart must match the oracle exactly; for the others the GPU's
  choice must be valid: K distinct experts in [0, E), descending within
  EPS_KEY, no unchosen key above the smallest chosen key by more than EPS_KEY.
  EPS_KEY = 1e-6: the fp32 exponential is good to a few ulp, the sigmoid and
  the bias add each round once, and |key| < 4 here (ulp 4.8e-7).
* p: |p - p_ref| <= 1e-5 |p_ref| + 1e-9, with p_ref the oracle's weights for
  the GPU's own selection (fp32 exponentials and a sum of at most 1024 terms:
  the relative error is a few 1e-7).
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

DEV = torch.device("cuda:0")
EPS_KEY = 1e-6
P_RTOL, P_ATOL = 1e-5, 1e-9


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def run(logits, K, mode, bias=None, scale=1.0):
    dl = torch.from_numpy(logits).to(DEV)
    db = None if bias is None else torch.from_numpy(bias).to(DEV)
    sel, p = mx.route(dl, K, mode, db, scale)
    torch.cuda.synchronize()
    return sel.cpu().numpy(), p.cpu().numpy()


def check_selection(sel, keys, K, exact_sel=None):
    """Validity of the GPU's selection against float64 keys; exact agreement
    with ``exact_sel`` wherever the keys leave no room (see module doc)."""
    T, E = keys.shape
    assert sel.shape == (T, K)
    assert sel.min() >= 0 and sel.max() < E
    for t in range(T):
        assert len(set(sel[t].tolist())) == K, f"token {t}: repeated expert {sel[t]}"
    chosen = np.take_along_axis(keys, sel.astype(np.int64), 1)
    assert np.all(np.diff(chosen, axis=1) <= EPS_KEY), "not descending"
    rest = keys.copy()
    np.put_along_axis(rest, sel.astype(np.int64), -np.inf, 1)
    if K < E:
        assert np.all(rest.max(1) <= chosen.min(1) + EPS_KEY), "an unchosen key beats a chosen one"
    n_exact = 0
    if exact_sel is not None:
        srt = -np.sort(-keys, axis=1)[:, :min(K + 1, E)]
        clear = np.all(np.abs(np.diff(srt, axis=1)) > EPS_KEY, axis=1)
        n_exact = int(clear.sum())
        bad = np.nonzero(clear & np.any(sel != exact_sel, axis=1))[0]
        assert bad.size == 0, f"tokens {bad[:5]} differ from the oracle with no near tie"
    return n_exact


def check_weights(p, logits, sel, mode, scale):
    ref = oracle.route_weights(logits, sel, mode, scale)
    err = np.abs(p.astype(np.float64) - ref)
    assert np.all(err <= P_RTOL * np.abs(ref) + P_ATOL), f"max err {err.max():.3g}"


SHAPES = [  # T, E, K
    (1, 8, 1), (7, 8, 2), (33, 64, 4), (100, 65, 3), (1000, 128, 4), (129, 128, 8),
    (64, 256, 8), (17, 384, 6), (50, 1000, 16), (40, 1024, 64), (5, 64, 64), (3, 1, 1),
]


@pytest.mark.parametrize("T,E,K", SHAPES)
def test_softmax_router_against_oracle(T, E, K):
    say(f"softmax router T={T} E={E} K={K}")
    logits, _ = workloads.router_logits(T, E, seed=E + K, std=2.0)
    sel, p = run(logits, K, "softmax", scale=1.0)
    want_sel, _ = oracle.route_softmax(logits, K)
    assert np.array_equal(sel, want_sel)
    check_weights(p, logits, sel, "softmax", 1.0)


@pytest.mark.parametrize("T,E,K", SHAPES)
def test_sigmoid_router_against_oracle(T, E, K):
    say(f"sigmoid router T={T} E={E} K={K}")
    logits, bias = workloads.router_logits(T, E, seed=7 * E + K, std=1.5, bias_std=0.1)
    sel, p = run(logits, K, "sigmoid", bias, scale=2.5)
    want_sel, _ = oracle.route_sigmoid(logits, bias, K)
    n = check_selection(sel, oracle.route_keys(logits, bias, "sigmoid"), K, want_sel)
    assert n >= 0.9 * T, f"only {n} of {T} tokens clear of near ties: the case proves little"
    check_weights(p, logits, sel, "sigmoid", 2.5)


@pytest.mark.parametrize("mode", ["softmax", "sigmoid"])
def test_router_exact_ties(mode):
    """Logits on a 1/4 grid (and no bias): many exact ties among the largest,
    identical on both sides, which must go to the lower index in order."""
    T, E, K = 300, 96, 6
    say(f"router ties {mode}")
    logits, _ = workloads.router_logits(T, E, seed=11, std=1.0, grid=0.25)
    sel, p = run(logits, K, mode)
    want_sel, _ = (oracle.route_softmax(logits, K) if mode == "softmax" else oracle.route_sigmoid(logits, None, K))
    ties = sum(len(set(np.sort(r)[-K - 1:].tolist())) < K + 1 for r in logits)
    assert ties > T // 2
    assert np.array_equal(sel, want_sel)
    check_weights(p, logits, sel, mode, 1.0)


def test_sigmoid_router_bias_ties():
    """Grid logits and a grid bias: experts with equal logits and equal bias
    have equal keys on both sides (the same inputs through the same steps),
    so those ties must go to the lower index; other keys are checked within
    EPS_KEY."""
    T, E, K = 200, 64, 4
    logits, bias = workloads.router_logits(T, E, seed=12, std=1.0, grid=0.25, bias_std=0.2)
    sel, p = run(logits, K, "sigmoid", bias)
    want_sel, _ = oracle.route_sigmoid(logits, bias, K)
    check_selection(sel, oracle.route_keys(logits, bias, "sigmoid"), K, want_sel)
    check_weights(p, logits, sel, "sigmoid", 1.0)


def test_router_nan_and_infinite_logits():
    """A NaN key counts as -inf: never chosen over a larger number, tied
    with -inf by index; -inf logits are still valid, distinct choices."""
    T, E, K = 64, 32, 4
    logits, _ = workloads.router_logits(T, E, seed=13)
    logits[:, 5] = np.nan
    logits[:8, :] = -np.inf
    logits[:8, 9] = np.nan
    sel, _ = run(logits, K, "sigmoid")
    assert sel.min() >= 0 and sel.max() < E
    for t in range(T):
        assert len(set(sel[t].tolist())) == K
        assert 5 not in sel[t].tolist()
    assert sel[:8].tolist() == [[0, 1, 2, 3]] * 8  # all -inf or NaN: ties to the lower index
    finite = logits[8:].copy()
    finite[:, 5] = -np.inf  # the reading of a NaN key
    want, _ = oracle.route_sigmoid(finite, None, K)
    check_selection(sel[8:], oracle.route_keys(finite, None, "sigmoid"), K, want)
    sel_s, _ = run(logits, K, "softmax")
    assert np.array_equal(sel_s[8:], oracle.route_softmax(finite, K)[0])


@pytest.mark.parametrize("name,mode", [("prefill", "softmax"), ("skewed", "sigmoid")])
def test_router_at_full_batch(name, mode):
    """The routers at the token counts and expert counts of the prefill
    (4096 x 128, K = 4) and skewed (8192 x 384, K = 8) batches."""
    w = workloads.WORKLOADS[name]
    say(f"router {mode} at {name}: T={w.T} E={w.E} K={w.K}")
    logits, bias = workloads.router_logits(w.T, w.E, seed=21 + w.index, std=2.0,
                                           bias_std=0.1 if mode == "sigmoid" else None)
    sel, p = run(logits, w.K, mode, bias, scale=1.0)
    want_sel, _ = (oracle.route_softmax(logits, w.K) if mode == "softmax"
                   else oracle.route_sigmoid(logits, bias, w.K))
    if mode == "softmax":
        assert np.array_equal(sel, want_sel)
    else:
        n = check_selection(sel, oracle.route_keys(logits, bias, mode), w.K, want_sel)
        assert n >= 0.9 * w.T
    check_weights(p, logits, sel, mode, 1.0)


def test_router_empty_batch():
    sel, p = mx.route(torch.empty((0, 16), dtype=torch.float32, device=DEV), 2)
    assert sel.shape == (0, 2) and p.shape == (0, 2)


def test_router_rejects_bad_arguments():
    lg = torch.zeros((4, 8), dtype=torch.float32, device=DEV)
    with pytest.raises(mx.Mxfp4Error):
        mx.route(lg, 9)
    with pytest.raises(mx.Mxfp4Error):
        mx.route(lg, 2, "softmax", torch.zeros(8, dtype=torch.float32, device=DEV))
    with pytest.raises(ValueError):
        mx.route(lg, 2, "tanh")
