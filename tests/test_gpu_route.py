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


# ------------------------------------------------------------- group-limited sigmoid router

EPS_GROUP = 2e-6  # a group score is a sum of two keys: twice their EPS_KEY


def run_grouped(logits, K, n_group, topk_group, bias=None, scale=1.0, renorm=True):
    dl = torch.from_numpy(logits).to(DEV)
    db = None if bias is None else torch.from_numpy(bias).to(DEV)
    sel, p = mx.route_grouped(dl, K, n_group, topk_group, db, scale, renorm)
    torch.cuda.synchronize()
    return sel.cpu().numpy(), p.cpu().numpy()


def check_grouped(sel, p, logits, bias, K, n_group, topk_group, scale, renorm):
    """Exact agreement with the oracle on tokens whose group scores around the
    topk_group cut and whose kept keys around the K cut are more than the
    fp32 margins apart; a valid choice within those margins elsewhere."""
    T, E = logits.shape
    eg = E // n_group
    want_sel, want_p = oracle.route_sigmoid_grouped(logits, bias, K, n_group, topk_group, scale, renorm)
    keys = oracle.route_keys(logits, bias, "sigmoid")
    keys = np.where(np.isnan(keys), -np.inf, keys)
    gsc = -np.sort(-keys.reshape(T, n_group, eg), axis=2)[:, :, :2].sum(2)
    gsorted = -np.sort(-gsc, axis=1)
    cut = gsorted[:, topk_group - 1]
    g_clear = (topk_group == n_group) | (np.abs(gsorted[:, topk_group - 1] - gsorted[:, min(topk_group, n_group - 1)])
                                         > EPS_GROUP)
    kept = gsc >= cut[:, None]
    masked = np.where(np.repeat(kept, eg, axis=1), keys, -np.inf)
    ks = -np.sort(-masked, axis=1)[:, :K + 1]
    k_clear = np.all(np.abs(np.diff(ks, axis=1)) > EPS_KEY, axis=1)
    clear = g_clear & k_clear
    assert sel.shape == (T, K) and sel.min() >= 0 and sel.max() < E
    for t in range(T):
        assert len(set(sel[t].tolist())) == K, f"token {t}: repeated expert"
        # every chosen expert's group is within the margin of the kept set
        assert np.all(gsc[t, sel[t] // eg] >= cut[t] - EPS_GROUP), f"token {t}: a group below the cut"
        ck = keys[t, sel[t]]
        assert np.all(np.diff(ck) <= EPS_KEY), f"token {t}: not descending"
    bad = np.nonzero(clear & np.any(sel != want_sel, axis=1))[0]
    assert bad.size == 0, f"tokens {bad[:5]} differ from the oracle with no near tie"
    same = np.all(sel == want_sel, axis=1)
    err = np.abs(p[same].astype(np.float64) - want_p[same])
    assert np.all(err <= P_RTOL * np.abs(want_p[same]) + P_ATOL), f"weights: max err {err.max():.3g}"
    return int(clear.sum())


GROUPED_SHAPES = [  # T, E, K, n_group, topk_group
    (1, 8, 2, 4, 2), (33, 64, 4, 8, 2), (100, 256, 8, 8, 4), (129, 128, 6, 4, 1), (50, 1000, 16, 8, 3),
    (17, 384, 8, 12, 4), (40, 1024, 64, 64, 32), (3, 2, 1, 1, 1), (64, 160, 6, 10, 10),
]


@pytest.mark.parametrize("renorm", [True, False])
@pytest.mark.parametrize("T,E,K,n_group,topk_group", GROUPED_SHAPES)
def test_grouped_router_against_oracle(T, E, K, n_group, topk_group, renorm):
    say(f"grouped router T={T} E={E} K={K} groups {n_group} keep {topk_group} renorm={renorm}")
    logits, bias = workloads.router_logits(T, E, seed=3 * E + K + n_group, std=1.5, bias_std=0.1)
    sel, p = run_grouped(logits, K, n_group, topk_group, bias, 1.75, renorm)
    n = check_grouped(sel, p, logits, bias, K, n_group, topk_group, 1.75, renorm)
    assert n >= 0.85 * T, f"only {n} of {T} tokens clear of near ties: the case proves little"


def test_grouped_router_worked_example():
    # biases on a 1/8 grid and logits 0: every score exact on both sides;
    # group scores 1.0, 1.5, 1.0, 0.9375 keep groups 1 and 0 (tie with 2 to
    # the lower index), so the best expert overall (7) is dropped
    logits = np.zeros((3, 8), np.float32)
    bias = np.array([0.375, -0.375, 0.25, 0.25, 0.0, 0.0, -0.5, 0.4375], np.float32)
    sel, p = run_grouped(logits, 2, 4, 2, bias, 3.0)
    assert sel.tolist() == [[0, 2]] * 3
    assert np.all(p == 1.5)
    sel1, _ = run_grouped(logits, 2, 4, 1, bias)  # one group kept: group 1 (1.5)
    assert sel1.tolist() == [[2, 3]] * 3


def test_grouped_router_every_group_kept_is_the_sigmoid_router():
    T, E, K = 300, 256, 8
    logits, bias = workloads.router_logits(T, E, seed=31, std=1.5, bias_std=0.1)
    sel_g, p_g = run_grouped(logits, K, 8, 8, bias, 2.0)
    sel_s, p_s = run(logits, K, "sigmoid", bias, scale=2.0)
    assert np.array_equal(sel_g, sel_s)
    assert np.array_equal(p_g, p_s)


def test_grouped_router_full_batch_and_nan():
    # 4096 tokens over 256 experts in 8 groups, 4 kept, top 8 (the shape of
    # the large group-limited routers), then NaN logits that never win
    T, E, K = 4096, 256, 8
    logits, bias = workloads.router_logits(T, E, seed=32, std=2.0, bias_std=0.1)
    sel, p = run_grouped(logits, K, 8, 4, bias)
    n = check_grouped(sel, p, logits, bias, K, 8, 4, 1.0, True)
    assert n >= 0.9 * T
    bad = logits[:64].copy()
    bad[:, 3] = np.nan
    sel, p = run_grouped(bad, K, 8, 4, bias)
    assert not np.any(sel == 3)
    check_grouped(sel, p, bad, bias, K, 8, 4, 1.0, True)


def test_grouped_router_rejects_bad_arguments():
    lg = torch.zeros((4, 12), dtype=torch.float32, device=DEV)
    for args in ((2, 5, 1), (2, 4, 5), (2, 12, 1), (7, 4, 1), (0, 4, 1)):  # 5 does not divide 12; one per group; K too big
        with pytest.raises(mx.Mxfp4Error):
            mx.route_grouped(lg, *args)
    sel, p = mx.route_grouped(torch.empty((0, 12), dtype=torch.float32, device=DEV), 2, 4, 2)
    assert sel.shape == (0, 2)
