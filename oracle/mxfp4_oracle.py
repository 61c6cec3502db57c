"""Float64 CPU oracle for the MXFP4 routed-expert linear.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
baseline may import this module. The GPU library never imports it, and this
module imports nothing from the library: the two share no code.

What is computed. Page "MXFP4 Routed Expert Linear" (Kimi K3), section
"Route, weight, and add the shared path", defines for every token t

    y_t = y_t^shared + sum over selected experts e of p_{t,e} * W_e x_t

where W_e (O rows by I = 32G columns) is held as packed bytes (E, O, G, 16)
and scale bytes (E, O, G) (page "MXFP4 Experts", shape paragraph; page
"MXFP4 Dequant", "How it works": the scale array has the packed array's
shape without its last axis). The method has no approximation step: the
decoded weights are exact, so this float64 oracle is the defining formula
written out, and its only rounding is float64 accumulation.

Decoding follows the pages:

* one group is 16 bytes = 32 four-bit E2M1 codes plus one E8M0 scale byte
  (page "MXFP4 Routed Expert Linear", "What is stored in one group");
* every byte gives its low nibble first, then its high nibble, i.e.
  n_lo = b mod 16, n_hi = floor(b / 16) (same section; page "MXFP4 Dequant",
  "How it works");
* a code indexes the 16-entry E2M1 table printed in the starter code;
* each decoded value of a group is multiplied by 2^(s - 127) for the group's
  scale byte s ("Apply the shared group scale"); the scale belongs to one
  expert, one output row and one group;
* group g fills input columns 32g .. 32g+31, and output coordinate o is the
  dot product of the token with row o ("Reconstruct the matrix in the right
  orientation").

The steps of ``expert_linear`` follow the page's "Implementation order":
start from a copy of the shared output, decode each selected expert once,
multiply each token by its selected experts, weight and accumulate the
contributions, then add them to the shared output.

Readings taken where the pages are silent:

* every scale byte 0..255 follows 2^(s-127); 255 is not treated as NaN;
* a token that lists the same expert twice gets both contributions
  (the page speaks of a list of selected experts);
* the mixture weights are used as given, never renormalised;
* an expert index outside [0, E) violates a stated precondition; the oracle
  raises ValueError.

The SwiGLU expert block (``expert_swiglu``, at the end of this module)
composes two such projections per routed pair with silu(gate) * up between
them (page "MoE Expert Kernels: Grouped Prefill and Mixed-Quant Compact
Experts", section 1; gate and up stacked along the output rows, gate first).

Parity status: every function here is pinned by tests against values the
pages print, closed forms, invariants and a brute-force scalar version.
"""

from __future__ import annotations

import numpy as np

# The 16-entry E2M1 value table of the starter code (page "MXFP4 Routed
# Expert Linear", "Starter Code"; the same table is printed in page
# "MXFP4 Dequant", "How it works"). Index 8 is negative zero.
E2M1_VALUES = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
               -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0)
E2M1_TABLE = np.array(E2M1_VALUES, dtype=np.float64)

SCALE_BIAS = 127  # "Apply the shared group scale": factor 2^(s - 127)
GROUP_BYTES = 16  # "What is stored in one group": sixteen bytes
GROUP_VALUES = 32  # ... holding 32 four-bit codes


# ---------------------------------------------------------------- decoding

def split_nibbles(packed: np.ndarray):
    """Low and high nibble of every byte: (b & 0xF, b >> 4).

    Page "MXFP4 Routed Expert Linear", hints: a bit mask for the low nibble,
    a right shift then the same mask for the high one.
    """
    b = np.asarray(packed, dtype=np.uint8)
    return b & 0x0F, (b >> 4) & 0x0F


def group_codes(packed: np.ndarray) -> np.ndarray:
    """Codes of each 16-byte group in decode order: (..., 16) -> (..., 32).

    Position 2j holds byte j's low nibble and position 2j+1 its high nibble
    (decode the low nibble first, then the high nibble; interleave before
    flattening).
    """
    lo, hi = split_nibbles(packed)
    codes = np.stack([lo, hi], axis=-1)  # (..., 16, 2)
    return codes.reshape(codes.shape[:-2] + (2 * codes.shape[-2],))


def scale_factor(scales: np.ndarray) -> np.ndarray:
    """2^(s - 127) for each scale byte, in float64 (exact for all 0..255)."""
    s = np.asarray(scales, dtype=np.uint8).astype(np.int64)
    return np.ldexp(np.ones(s.shape, dtype=np.float64), s - SCALE_BIAS)


def decode_rows(packed_rows: np.ndarray, scales_rows: np.ndarray) -> np.ndarray:
    """Decode rows of one expert: packed (R, G, 16), scales (R, G) -> (R, 32G).

    Each group's 32 table values are multiplied by its own scale factor and
    the groups are concatenated in order along the input axis.
    """
    packed_rows = np.asarray(packed_rows, dtype=np.uint8)
    scales_rows = np.asarray(scales_rows, dtype=np.uint8)
    if packed_rows.ndim != 3 or packed_rows.shape[-1] != GROUP_BYTES:
        raise ValueError("packed rows must have shape (R, G, 16)")
    if scales_rows.shape != packed_rows.shape[:-1]:
        raise ValueError("scales must have the packed shape without its last axis")
    values = E2M1_TABLE[group_codes(packed_rows)]  # (R, G, 32)
    values = values * scale_factor(scales_rows)[..., None]
    R, G = scales_rows.shape
    return values.reshape(R, G * GROUP_VALUES)


def decode_expert(packed_e: np.ndarray, scales_e: np.ndarray) -> np.ndarray:
    """The full (O, 32G) float64 matrix W_e of one expert."""
    return decode_rows(packed_e, scales_e)


# --------------------------------------------------------------- bucketing

def bucket_pairs(sel: np.ndarray, E: int) -> dict:
    """Count-sort of (token, slot) pairs by expert, keeping pair order.

    The pairs are numbered i = t*K + k. ``count[e]`` is how many pairs chose
    e; ``offsets`` is the exclusive prefix sum of the counts (length E+1);
    expert e owns the sorted positions offsets[e] .. offsets[e+1]-1, filled
    with its pairs in increasing pair number (histogram, then scatter, as
    the bucketed expert prefill does on page "MoE Expert Kernels: Grouped
    Prefill and Mixed-Quant Compact Experts", section 2).
    ``perm[position] = pair`` and ``slot_of_pair[pair] = position``.
    A pair whose index is outside [0, E) gets no position
    (slot_of_pair = -1) and is counted in ``n_invalid``.
    """
    flat = np.asarray(sel).reshape(-1).astype(np.int64)
    P = flat.size
    count = np.zeros(E, dtype=np.int64)
    n_invalid = 0
    for e in flat:  # histogram
        if 0 <= e < E:
            count[e] += 1
        else:
            n_invalid += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):  # exclusive prefix sum
        offsets[e + 1] = offsets[e] + count[e]
    cursor = offsets[:-1].copy()
    perm = np.full(offsets[-1], -1, dtype=np.int64)
    slot_of_pair = np.full(P, -1, dtype=np.int64)
    for i, e in enumerate(flat):  # stable scatter in pair order
        if 0 <= e < E:
            perm[cursor[e]] = i
            slot_of_pair[i] = cursor[e]
            cursor[e] += 1
    return {
        "count": count.astype(np.int32),
        "offsets": offsets.astype(np.int32),
        "perm": perm.astype(np.int32),
        "slot_of_pair": slot_of_pair.astype(np.int32),
        "n_invalid": int(n_invalid),
    }


# ------------------------------------------------------------- the layer

def _check(x, sel, p, shared, E):
    x = np.asarray(x)
    sel = np.asarray(sel)
    p = np.asarray(p)
    shared = np.asarray(shared)
    if x.ndim != 2 or x.shape[1] % GROUP_VALUES != 0 or x.shape[1] == 0:
        raise ValueError("x must be (T, 32G) with G >= 1")
    if sel.shape != p.shape or sel.ndim != 2 or sel.shape[0] != x.shape[0]:
        raise ValueError("selected experts and mixture weights must both be (T, K)")
    if shared.ndim != 2 or shared.shape[0] != x.shape[0]:
        raise ValueError("shared output must be (T, O)")
    if sel.size and (sel.min() < 0 or sel.max() >= E):
        raise ValueError("selected expert index out of range")
    return x, sel, p, shared


def expert_linear(x, packed, scales, sel, p, shared) -> np.ndarray:
    """y = shared + sum_k p[t,k] * W_{sel[t,k]} x_t, in float64.

    ``packed`` and ``scales`` are anything that returns expert e's arrays for
    ``packed[e]`` (O, G, 16) and ``scales[e]`` (O, G) - a NumPy array or a
    lazily drawn tensor - so only the selected experts are ever read.
    Returns a new float64 (T, O) array; no input is modified.
    """
    E = len(packed)
    x, sel, p, shared = _check(x, sel, p, shared, E)
    T, K = sel.shape
    O = shared.shape[1]
    x64 = x.astype(np.float64)
    p64 = p.astype(np.float64)
    y = shared.astype(np.float64, copy=True)  # a non-mutating copy of shared
    contrib = np.zeros((T, K, O), dtype=np.float64)
    for e in np.unique(sel):  # each selected expert is decoded once
        W = decode_expert(packed[e], scales[e])
        if W.shape != (O, x.shape[1]):
            raise ValueError("expert matrix shape does not match x and shared")
        ts, ks = np.nonzero(sel == e)
        contrib[ts, ks, :] = x64[ts] @ W.T  # each row of W dotted with the token
    routed = np.zeros((T, O), dtype=np.float64)
    for k in range(K):  # weighted accumulation over the selected list
        routed += p64[:, k:k + 1] * contrib[:, k, :]
    return y + routed


def expert_linear_rows(x, packed, scales, sel, p, shared, rows) -> np.ndarray:
    """The same as ``expert_linear`` restricted to output coordinates ``rows``.

    Returns (T, len(rows)) float64: column j is output coordinate rows[j].
    Only those rows of the selected experts are decoded, which makes the
    oracle usable at full size on a sample of outputs.
    """
    E = len(packed)
    x, sel, p, shared = _check(x, sel, p, shared, E)
    rows = np.asarray(rows, dtype=np.int64)
    T, K = sel.shape
    x64 = x.astype(np.float64)
    p64 = p.astype(np.float64)
    y = shared[:, rows].astype(np.float64)
    contrib = np.zeros((T, K, rows.size), dtype=np.float64)
    for e in np.unique(sel):
        W = decode_rows(np.asarray(packed[e])[rows], np.asarray(scales[e])[rows])
        ts, ks = np.nonzero(sel == e)
        contrib[ts, ks, :] = x64[ts] @ W.T
    routed = np.zeros((T, rows.size), dtype=np.float64)
    for k in range(K):
        routed += p64[:, k:k + 1] * contrib[:, k, :]
    return y + routed


def expert_linear_scalar(x, packed, scales, sel, p, shared) -> list:
    """Brute force with plain Python numbers and loops (tiny shapes only).

    Reads every weight from its byte and scale directly, with no arrays, no
    table of decoded groups and no matrix products; returns a list of lists.
    """
    T = len(x)
    K = len(sel[0]) if T else 0
    O = len(shared[0]) if T else 0
    out = []
    for t in range(T):
        row = []
        for o in range(O):
            acc = float(shared[t][o])
            for k in range(K):
                e = int(sel[t][k])
                dot = 0.0
                G = len(packed[e][o])
                for g in range(G):
                    factor = 2.0 ** (int(scales[e][o][g]) - SCALE_BIAS)
                    for j in range(GROUP_BYTES):
                        byte = int(packed[e][o][g][j])
                        low, high = byte % 16, byte // 16
                        dot += E2M1_VALUES[low] * factor * float(x[t][32 * g + 2 * j])
                        dot += E2M1_VALUES[high] * factor * float(x[t][32 * g + 2 * j + 1])
                acc += float(p[t][k]) * dot
            row.append(acc)
        out.append(row)
    return out


# ------------------------------------------------------- the SwiGLU expert
#
# Page "MoE Expert Kernels: Grouped Prefill and Mixed-Quant Compact Experts",
# section "1. The shared building blocks: routers and the SwiGLU expert
# shape": every routed expert is a SwiGLU - gate and up projections of the
# token, silu(gate) times up elementwise, then the down projection - and the
# routed outputs are weighted by the mixture weights and accumulated. The exo
# pull request page ("Summary") stacks each expert's gate and up matrices
# along their output rows; the plainest reading, taken here, is gate rows
# first: rows [0, F) of the stacked matrix are the gate, rows [F, 2F) the up
# projection. Both matrices are MXFP4 like the routed linear's. The oracle
# keeps the intermediate exact in float64.

def silu(v):
    """silu(v) = v * sigmoid(v) = v / (1 + e^-v), float64 (0 for v -> -inf)."""
    v = np.asarray(v, dtype=np.float64)
    with np.errstate(over="ignore"):
        return v / (1.0 + np.exp(-v))


def _swiglu_shapes(gu_packed, dn_packed, x, shared):
    two_f = np.asarray(gu_packed[0]).shape[0]
    if two_f % 2 != 0:
        raise ValueError("the stacked gate/up matrix needs an even row count")
    F = two_f // 2
    if np.asarray(dn_packed[0]).shape[1] * GROUP_VALUES != F:
        raise ValueError("the down projection's input width must be F")
    if np.asarray(gu_packed[0]).shape[1] * GROUP_VALUES != np.asarray(x).shape[1]:
        raise ValueError("the gate/up input width must match x")
    if np.asarray(dn_packed[0]).shape[0] != np.asarray(shared).shape[1]:
        raise ValueError("the down projection's output width must match shared")
    return F


def swiglu_hidden(x_rows, gu_packed_e, gu_scales_e):
    """h = silu(gate x) * (up x) for the token rows x_rows (n, I) of one
    expert: (n, F) float64."""
    W = decode_expert(gu_packed_e, gu_scales_e)  # (2F, I)
    F = W.shape[0] // 2
    gu = np.asarray(x_rows, dtype=np.float64) @ W.T
    return silu(gu[:, :F]) * gu[:, F:]


def expert_swiglu(x, gu_packed, gu_scales, dn_packed, dn_scales, sel, p, shared) -> np.ndarray:
    """y_t = shared_t + sum_k p[t,k] * D_e (silu(Gate_e x_t) * (Up_e x_t)),
    e = sel[t,k], in float64. gu_packed (E, 2F, G, 16) / gu_scales (E, 2F, G)
    hold gate then up; dn_packed (E, O, F/32, 16) / dn_scales (E, O, F/32)
    the down projection. Returns a new (T, O) float64 array."""
    E = len(gu_packed)
    x, sel, p, shared = _check(x, sel, p, shared, E)
    _swiglu_shapes(gu_packed, dn_packed, x, shared)
    T, K = sel.shape
    O = shared.shape[1]
    x64 = x.astype(np.float64)
    p64 = p.astype(np.float64)
    y = shared.astype(np.float64, copy=True)
    contrib = np.zeros((T, K, O), dtype=np.float64)
    for e in np.unique(sel):
        ts, ks = np.nonzero(sel == e)
        h = swiglu_hidden(x64[ts], gu_packed[e], gu_scales[e])
        D = decode_expert(dn_packed[e], dn_scales[e])  # (O, F)
        contrib[ts, ks, :] = h @ D.T
    routed = np.zeros((T, O), dtype=np.float64)
    for k in range(K):
        routed += p64[:, k:k + 1] * contrib[:, k, :]
    return y + routed


def expert_swiglu_rows(x, gu_packed, gu_scales, dn_packed, dn_scales, sel, p, shared, rows) -> np.ndarray:
    """``expert_swiglu`` restricted to output coordinates ``rows``: every
    pair's full hidden vector, but only those rows of the down projections."""
    E = len(gu_packed)
    x, sel, p, shared = _check(x, sel, p, shared, E)
    rows = np.asarray(rows, dtype=np.int64)
    T, K = sel.shape
    x64 = x.astype(np.float64)
    p64 = p.astype(np.float64)
    y = shared[:, rows].astype(np.float64)
    contrib = np.zeros((T, K, rows.size), dtype=np.float64)
    for e in np.unique(sel):
        ts, ks = np.nonzero(sel == e)
        h = swiglu_hidden(x64[ts], gu_packed[e], gu_scales[e])
        D = decode_rows(np.asarray(dn_packed[e])[rows], np.asarray(dn_scales[e])[rows])
        contrib[ts, ks, :] = h @ D.T
    routed = np.zeros((T, rows.size), dtype=np.float64)
    for k in range(K):
        routed += p64[:, k:k + 1] * contrib[:, k, :]
    return y + routed


def expert_swiglu_scalar(x, gu_packed, gu_scales, dn_packed, dn_scales, sel, p, shared) -> list:
    """Brute force with plain Python numbers and loops (tiny shapes only)."""
    import math

    def weight(packed, scales, e, o, i):
        byte = int(packed[e][o][i // 32][(i % 32) // 2])
        code = byte % 16 if i % 2 == 0 else byte // 16
        return E2M1_VALUES[code] * 2.0 ** (int(scales[e][o][i // 32]) - SCALE_BIAS)

    T = len(x)
    K = len(sel[0]) if T else 0
    O = len(shared[0]) if T else 0
    I = len(x[0]) if T else 0
    F = len(gu_packed[0]) // 2
    out = []
    for t in range(T):
        row = [float(shared[t][o]) for o in range(O)]
        for k in range(K):
            e = int(sel[t][k])
            h = []
            for f in range(F):
                g = sum(weight(gu_packed, gu_scales, e, f, i) * float(x[t][i]) for i in range(I))
                u = sum(weight(gu_packed, gu_scales, e, F + f, i) * float(x[t][i]) for i in range(I))
                h.append(g / (1.0 + math.exp(-g)) * u)
            for o in range(O):
                d = sum(weight(dn_packed, dn_scales, e, o, f) * h[f] for f in range(F))
                row[o] += float(p[t][k]) * d
        out.append(row)
    return out


# ----------------------------------------------------------------- routers
#
# What produces sel and p upstream of the layer. Two routers are described:
# the CPU kernels page (section 1) gives a softmax router - softmax over all
# experts, the top k of it, their probabilities divided by
# max(their sum, 6.103515625e-5), times a scaling factor - and a sigmoid
# router whose correction bias steers the selection only (the weights are
# gathered from the unbiased scores); the Metal PR page ("Summary", the
# router bullets) ranks with ties going to the lower expert index, keeps the
# selection in that descending order, sums the chosen scores left to right,
# divides by (sum + 1e-20) and multiplies by the scaling factor. Readings:
# the selection is made on the exact (float64) quantities - for the softmax
# router that is the logits themselves, which rank exactly like the exact
# probabilities - and the sigmoid router has no expert groups (one group).

SOFTMAX_MASS_FLOOR = 6.103515625e-5  # the CPU kernels page's lower bound on the selected mass
SIGMOID_EPS = 1e-20                  # the Metal PR page's addend to the sum of the chosen scores


def _topk_desc(keys: np.ndarray, K: int) -> np.ndarray:
    """Indices of the K largest keys per row, largest first, ties to the
    lower index (a stable sort of the negated keys)."""
    return np.argsort(-keys, axis=1, kind="stable")[:, :K]


def _logits2d(logits, K: int) -> np.ndarray:
    l = np.asarray(logits, dtype=np.float64)
    if l.ndim != 2 or not 1 <= K <= l.shape[1]:
        raise ValueError("logits must be (T, E) with 1 <= K <= E")
    return l


def _sigmoid(l: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-l))


def route_keys(logits, bias, mode: str) -> np.ndarray:
    """The float64 quantity each router ranks by: the logits (softmax; they
    order like the exact probabilities) or sigmoid(logits) + bias."""
    l = np.asarray(logits, dtype=np.float64)
    if mode == "softmax":
        return l.copy()
    if mode == "sigmoid":
        b = np.zeros(l.shape[1]) if bias is None else np.asarray(bias, dtype=np.float64)
        return _sigmoid(l) + b[None, :]
    raise ValueError(f"unknown router {mode!r}")


def route_weights(logits, sel, mode: str, scale: float = 1.0) -> np.ndarray:
    """float64 mixture weights (T, K) of the selection ``sel``: the chosen
    softmax probabilities over max(their sum, floor), or the chosen sigmoid
    scores over (their left-to-right sum + 1e-20); times ``scale``."""
    l = np.asarray(logits, dtype=np.float64)
    sel = np.asarray(sel, dtype=np.int64)
    if mode == "softmax":
        z = np.exp(l - l.max(axis=1, keepdims=True))
        prob = z / z.sum(axis=1, keepdims=True)
        chosen = np.take_along_axis(prob, sel, axis=1)
        return chosen / np.maximum(chosen.sum(axis=1, keepdims=True), SOFTMAX_MASS_FLOOR) * scale
    if mode == "sigmoid":
        chosen = np.take_along_axis(_sigmoid(l), sel, axis=1)
        total = np.zeros((l.shape[0], 1))
        for k in range(sel.shape[1]):  # left to right
            total += chosen[:, k:k + 1]
        return chosen / (total + SIGMOID_EPS) * scale
    raise ValueError(f"unknown router {mode!r}")


def route_softmax(logits, K: int, scale: float = 1.0):
    """Softmax router: returns (sel int32 [T, K], p float64 [T, K])."""
    l = _logits2d(logits, K)
    sel = _topk_desc(route_keys(l, None, "softmax"), K)
    return sel.astype(np.int32), route_weights(l, sel, "softmax", scale)


def route_sigmoid(logits, bias, K: int, scale: float = 1.0):
    """Sigmoid router with a selection-only bias: returns (sel, p)."""
    l = _logits2d(logits, K)
    sel = _topk_desc(route_keys(l, bias, "sigmoid"), K)
    return sel.astype(np.int32), route_weights(l, sel, "sigmoid", scale)


def _group_scores(keys: np.ndarray, n_group: int) -> np.ndarray:
    """(T, n_group): the sum of the two largest keys of each group of
    E / n_group consecutive experts."""
    T, E = keys.shape
    two = -np.sort(-keys.reshape(T, n_group, E // n_group), axis=2)[:, :, :2]
    return two[:, :, 0] + two[:, :, 1]


def route_sigmoid_grouped(logits, bias, K: int, n_group: int, topk_group: int, scale: float = 1.0,
                          renormalize: bool = True):
    """Group-limited sigmoid router (the CPU kernels page, section 1, its
    first router): the choice score of expert e is sigmoid(logit) + bias[e];
    the E experts form n_group groups of E / n_group consecutive experts; a
    group's score is the sum of its two largest choice scores; the topk_group
    groups with the largest scores are kept (ties to the lower group index);
    the K experts with the largest choice scores inside the kept groups are
    chosen (descending, ties to the lower expert index); their weights are
    gathered from the unbiased scores sigmoid(logit). Readings, the page
    being silent: a NaN choice score counts as -inf everywhere (also in its
    group's sum); with renormalize the gathered scores are divided by their
    left-to-right sum + 1e-20 as the ungrouped sigmoid router does (the page
    stops at the gather: renormalize=False), then times ``scale``. Needs
    n_group | E, E / n_group >= 2, 1 <= topk_group <= n_group and
    K <= topk_group * E / n_group. Returns (sel int32 [T, K], p float64)."""
    l = _logits2d(logits, K)
    T, E = l.shape
    if n_group < 1 or E % n_group or E // n_group < 2 or not 1 <= topk_group <= n_group:
        raise ValueError("need n_group | E, E / n_group >= 2 and 1 <= topk_group <= n_group")
    eg = E // n_group
    if K > topk_group * eg:
        raise ValueError("K exceeds the experts of the kept groups")
    keys = route_keys(l, bias, "sigmoid")
    keys = np.where(np.isnan(keys), -np.inf, keys)
    groups = _topk_desc(_group_scores(keys, n_group), topk_group)
    kept = np.zeros((T, n_group), dtype=bool)
    np.put_along_axis(kept, groups, True, axis=1)
    masked = np.where(np.repeat(kept, eg, axis=1), keys, -np.inf)
    sel = np.empty((T, K), dtype=np.int64)
    for t in range(T):  # the largest K of the kept experts; an -inf key may be chosen only inside a kept group
        order = [e for e in np.argsort(-masked[t], kind="stable") if kept[t, e // eg]]
        sel[t] = order[:K]
    chosen = np.take_along_axis(_sigmoid(l), sel, axis=1)
    if renormalize:
        total = np.zeros((T, 1))
        for k in range(K):  # left to right
            total += chosen[:, k:k + 1]
        chosen = chosen / (total + SIGMOID_EPS)
    return sel.astype(np.int32), chosen * scale


def route_scalar(logits, bias, K: int, mode: str, scale: float = 1.0):
    """Brute force with plain Python numbers (tiny shapes): repeated
    selection of the largest remaining key, lower index on ties."""
    import math
    out_sel, out_p = [], []
    for row in logits:
        E = len(row)
        if mode == "softmax":
            m = max(row)
            z = [math.exp(float(v) - m) for v in row]
            prob = [v / sum(z) for v in z]
            keys = [float(v) for v in row]
        else:
            prob = [1.0 / (1.0 + math.exp(-float(v))) for v in row]
            keys = [prob[e] + (0.0 if bias is None else float(bias[e])) for e in range(E)]
        left = list(range(E))
        sel = []
        for _ in range(K):
            best = left[0]
            for e in left[1:]:
                if keys[e] > keys[best]:
                    best = e
            sel.append(best)
            left.remove(best)
        mass = 0.0
        for e in sel:
            mass += prob[e]
        den = max(mass, SOFTMAX_MASS_FLOOR) if mode == "softmax" else mass + SIGMOID_EPS
        out_sel.append(sel)
        out_p.append([prob[e] / den * scale for e in sel])
    return out_sel, out_p


def route_grouped_scalar(logits, bias, K: int, n_group: int, topk_group: int, scale: float = 1.0,
                         renormalize: bool = True):
    """Brute force of route_sigmoid_grouped with plain Python numbers (tiny
    shapes): group scores by scanning each group for its two largest scores,
    then repeated selection of the largest remaining group and expert."""
    import math
    out_sel, out_p = [], []
    for row in logits:
        E = len(row)
        eg = E // n_group
        raw = [1.0 / (1.0 + math.exp(-float(v))) for v in row]
        keys = [raw[e] + (0.0 if bias is None else float(bias[e])) for e in range(E)]
        keys = [-math.inf if k != k else k for k in keys]
        gscore = []
        for g in range(n_group):
            a = b = -math.inf
            for e in range(g * eg, (g + 1) * eg):
                if keys[e] > a:
                    a, b = keys[e], a
                elif keys[e] > b:
                    b = keys[e]
            gscore.append(a + b)
        gleft, kept = list(range(n_group)), []
        for _ in range(topk_group):
            best = gleft[0]
            for g in gleft[1:]:
                if gscore[g] > gscore[best]:
                    best = g
            kept.append(best)
            gleft.remove(best)
        left = [e for e in range(E) if e // eg in kept]
        sel = []
        for _ in range(K):
            best = left[0]
            for e in left[1:]:
                if keys[e] > keys[best]:
                    best = e
            sel.append(best)
            left.remove(best)
        w = [raw[e] for e in sel]
        if renormalize:
            mass = 0.0
            for v in w:
                mass += v
            w = [v / (mass + SIGMOID_EPS) for v in w]
        out_sel.append(sel)
        out_p.append([v * scale for v in w])
    return out_sel, out_p


# ------------------------------------------- MXFP8 activations (variant)
#
# The block-scaled variant multiplies the packed weights as they are by
# activations that are themselves block-scaled. The pages fix the family and
# its block structure: MXFP4 is a member of the OCP Microscaling formats, in
# which blocks of 32 element codes share one E8M0 scale byte (page "MXFP4
# Dequant", "Overview"); the CPU kernels page quantises activations to 8-bit
# blocks of 32 for its integer dot products (its Q8_1 row provider). Readings
# for the activations, the pages being silent:
#
# * element format: the 8-bit float of that family with 4 exponent bits
#   (bias 7) and 3 mantissa bits, subnormals with quantum 2^-9, largest
#   finite value 448 = 1.75 * 2^8, no infinities, S.1111.111 the only NaN;
# * block: 32 consecutive inputs of one token (input columns 32b .. 32b+31,
#   the same columns as weight group b);
# * scale: the smallest power of two 2^X with max|block| <= 448 * 2^X, so no
#   element saturates; X clamped to [-127, 127] and stored as the byte
#   X + 127; an all-zero block takes X = -127;
# * elements: v / 2^X rounded to the nearest representable value, ties to
#   the even code, then clamped to +-448 (reachable only through the clamp of
#   X); the sign of v is kept, also when the magnitude rounds to zero.
#
# The variant's defining result is the routed linear of the dequantised
# activations, exact in float64: expert_linear(dequantize(quantize(x)), ...).

E4M3_MAX = 448.0
E4M3_MIN_NORMAL_EXP = -6   # smallest normal 2^-6
E4M3_MANTISSA_BITS = 3
E4M3_BIAS = 7


def e4m3_value(code: int) -> float:
    """Real value of one E4M3 code (NaN for 0x7f and 0xff)."""
    code = int(code)
    sign = -1.0 if code & 0x80 else 1.0
    e, m = (code >> 3) & 15, code & 7
    if e == 15 and m == 7:
        return float("nan")
    if e == 0:
        return sign * m * 2.0 ** (E4M3_MIN_NORMAL_EXP - E4M3_MANTISSA_BITS)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - E4M3_BIAS)


E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def mxfp8_block_exponent(amax) -> np.ndarray:
    """Smallest integer X with amax <= 448 * 2^X, clamped to [-127, 127];
    -127 for amax == 0. Exact: amax = f * 2^e with f in [0.5, 1), and
    448 = 0.875 * 2^9, so X = e - 9 when f <= 0.875 and e - 8 otherwise."""
    a = np.asarray(amax, dtype=np.float64)
    f, e = np.frexp(a)
    X = np.where(f <= 0.875, e - 9, e - 8)
    X = np.where(a == 0, -127, X)
    return np.clip(X, -127, 127).astype(np.int64)


def quantize_e4m3(v) -> np.ndarray:
    """E4M3 codes of float64 values already divided by their block scale:
    round to nearest, ties to even, clamp to +-448, keep the sign."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, e = np.frexp(a)                       # a = f * 2^e, f in [0.5, 1): exponent e - 1
    E = np.maximum(e - 1, E4M3_MIN_NORMAL_EXP)
    quantum = np.ldexp(1.0, E - E4M3_MANTISSA_BITS)
    aq = np.minimum(np.rint(a / quantum) * quantum, E4M3_MAX)   # np.rint: ties to even
    # encode the exact grid value: below 2^-6 the code is aq / 2^-9 (0..8,
    # and 8 is also the code of 2^-6); above, exponent and 3 mantissa bits
    _, eq = np.frexp(aq)
    Eq = eq - 1
    normal = aq >= 2.0 ** E4M3_MIN_NORMAL_EXP
    mant = np.where(normal, np.ldexp(aq, -Eq) - 1.0, 0.0) * 8.0
    code = np.where(normal, ((Eq + E4M3_BIAS) << 3) | mant.astype(np.int64),
                    np.ldexp(aq, 9).astype(np.int64))
    return (code | np.where(np.signbit(v), 0x80, 0)).astype(np.uint8)


def quantize_mxfp8(x) -> tuple:
    """Activations (T, I), I a multiple of 32 -> (codes uint8 (T, I),
    scale bytes uint8 (T, I/32)), one scale per token and block of 32."""
    x = np.asarray(x, dtype=np.float64)
    T, I = x.shape
    if I % GROUP_VALUES:
        raise ValueError("the input width must be a multiple of 32")
    blocks = x.reshape(T, I // GROUP_VALUES, GROUP_VALUES)
    X = mxfp8_block_exponent(np.abs(blocks).max(axis=2))
    codes = quantize_e4m3(blocks / np.ldexp(1.0, X)[:, :, None])
    return codes.reshape(T, I), (X + SCALE_BIAS).astype(np.uint8)


def dequantize_mxfp8(codes, scale_bytes) -> np.ndarray:
    """float64 values of MXFP8 activations: E4M3 value times 2^(s - 127)."""
    codes = np.asarray(codes)
    T, I = codes.shape
    vals = E4M3_TABLE[codes].reshape(T, I // GROUP_VALUES, GROUP_VALUES)
    f = np.ldexp(1.0, np.asarray(scale_bytes, dtype=np.int64) - SCALE_BIAS)
    return (vals * f[:, :, None]).reshape(T, I)


def expert_linear_mxfp8(x, packed, scales, sel, p, shared) -> np.ndarray:
    """The block-scaled variant: the routed linear of the MXFP8-quantised
    activations, exact in float64."""
    xh = dequantize_mxfp8(*quantize_mxfp8(x))
    return expert_linear(xh, packed, scales, sel, p, shared)


def expert_linear_mxfp8_rows(x, packed, scales, sel, p, shared, rows) -> np.ndarray:
    """expert_linear_mxfp8 restricted to the output rows ``rows``."""
    xh = dequantize_mxfp8(*quantize_mxfp8(x))
    return expert_linear_rows(xh, packed, scales, sel, p, shared, rows)


# ------------------------------------------- MXFP4 activations (variant)
#
# The same block-scaled variant with the activations in the weights' own
# format, so that both operands of the scaled multiply are FP4: E2M1 codes
# (the table above), blocks of 32 sharing one E8M0 scale byte (page "MXFP4
# Dequant", "Overview": the format is defined for blocks of 32 values, not
# for weights only). The pages say nothing of how activations would be
# quantised to it; the readings follow the MXFP8 ones above:
#
# * element: E2M1, the 4-bit code sign << 3 | index of the magnitude in
#   (0, 0.5, 1, 1.5, 2, 3, 4, 6);
# * block: 32 consecutive inputs of one token (the same columns as weight
#   group b);
# * scale: the smallest power of two 2^X with max|block| <= 6 * 2^X, so no
#   element saturates; X clamped to [-127, 127] and stored as the byte
#   X + 127; an all-zero block takes X = -127;
# * elements: v / 2^X rounded to the nearest E2M1 magnitude, ties to the
#   even code, clamped to 6 (reachable only through the clamp of X); the
#   sign kept, also when the magnitude rounds to zero (code 8);
# * two codes per byte, low nibble first, as the weights are packed.
#
# The variant's defining result is the routed linear of the dequantised
# activations, exact in float64: expert_linear(dequantize(quantize(x)), ...).

E2M1_MAX = 6.0
E2M1_MAGNITUDES = E2M1_TABLE[:8]  # 0, 0.5, 1, 1.5, 2, 3, 4, 6: codes 0..7


def mxfp4_block_exponent(amax) -> np.ndarray:
    """Smallest integer X with amax <= 6 * 2^X, clamped to [-127, 127];
    -127 for amax == 0. Exact: amax = f * 2^e with f in [0.5, 1), and
    6 = 0.75 * 2^3, so X = e - 3 when f <= 0.75 and e - 2 otherwise."""
    a = np.asarray(amax, dtype=np.float64)
    f, e = np.frexp(a)
    X = np.where(f <= 0.75, e - 3, e - 2)
    X = np.where(a == 0, -127, X)
    return np.clip(X, -127, 127).astype(np.int64)


def quantize_e2m1(v) -> np.ndarray:
    """E2M1 codes of float64 values already divided by their block scale:
    round to nearest, ties to even, clamp to +-6, keep the sign. Below 2 the
    magnitudes are multiples of 0.5, in [2, 4) of 1, in [4, 6] of 2, and in
    each step the even multiple has the even code."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, e = np.frexp(a)                           # a = f * 2^e, f in [0.5, 1)
    quantum = np.ldexp(1.0, np.maximum(e - 1, 0) - 1)
    aq = np.minimum(np.rint(a / quantum) * quantum, E2M1_MAX)   # np.rint: ties to even
    idx = np.searchsorted(E2M1_MAGNITUDES, aq)   # aq is one of the magnitudes
    return (idx | np.where(np.signbit(v), 8, 0)).astype(np.uint8)


def quantize_mxfp4(x) -> tuple:
    """Activations (T, I), I a multiple of 32 -> (codes uint8 (T, I) with
    values 0..15, one per input, and scale bytes uint8 (T, I/32))."""
    x = np.asarray(x, dtype=np.float64)
    T, I = x.shape
    if I % GROUP_VALUES:
        raise ValueError("the input width must be a multiple of 32")
    blocks = x.reshape(T, I // GROUP_VALUES, GROUP_VALUES)
    X = mxfp4_block_exponent(np.abs(blocks).max(axis=2))
    codes = quantize_e2m1(blocks / np.ldexp(1.0, X)[:, :, None])
    return codes.reshape(T, I), (X + SCALE_BIAS).astype(np.uint8)


def pack_codes(codes) -> np.ndarray:
    """Four-bit codes (T, I) -> bytes (T, I/2), code 2j in the low nibble of
    byte j (the weights' order)."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def dequantize_mxfp4(codes, scale_bytes) -> np.ndarray:
    """float64 values of MXFP4 activations: E2M1 value times 2^(s - 127)."""
    codes = np.asarray(codes)
    T, I = codes.shape
    vals = E2M1_TABLE[codes].reshape(T, I // GROUP_VALUES, GROUP_VALUES)
    f = np.ldexp(1.0, np.asarray(scale_bytes, dtype=np.int64) - SCALE_BIAS)
    return (vals * f[:, :, None]).reshape(T, I)


def expert_linear_mxfp4act(x, packed, scales, sel, p, shared) -> np.ndarray:
    """The block-scaled variant with MXFP4 activations: the routed linear of
    the quantised activations, exact in float64."""
    xh = dequantize_mxfp4(*quantize_mxfp4(x))
    return expert_linear(xh, packed, scales, sel, p, shared)


def expert_linear_mxfp4act_rows(x, packed, scales, sel, p, shared, rows) -> np.ndarray:
    """expert_linear_mxfp4act restricted to the output rows ``rows``."""
    xh = dequantize_mxfp4(*quantize_mxfp4(x))
    return expert_linear_rows(xh, packed, scales, sel, p, shared, rows)
