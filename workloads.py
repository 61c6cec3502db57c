"""Seeded synthetic inputs for the MXFP4 routed-expert linear.

This module only draws random inputs. It holds none of the method's
arithmetic: no nibble split, no table lookup, no scaling, no products and
no combine. The float64 oracle (under ``oracle/``) and the GPU library (under
``mxfp4_block_scaled_amd/``) both take their inputs from here and from nowhere
else, so the two sides never share code.

The five routed-linear workloads are the shapes and value distributions of
the problem statement on the pages (page "MXFP4 Routed Expert Linear", section
"Route, weight, and add the shared path"; page "MXFP4 Experts", the shape
paragraph): latent tokens x (T, I=32G), selected experts and mixture weights
(T, K), shared output (T, O), packed codes (E, O, G, 16) and scale bytes
(E, O, G), both unsigned bytes.

Recipe (fixed order, NumPy PCG64):

* ``SeedSequence(20261202 + index).spawn(8)`` gives the streams
  [0] x, [1] shared, [2] packed, [3] scales, [4] routing, [5] logits, and
  for the SwiGLU expert block [6] and [7], the down projection's packed and
  scale bytes ([2] and [3] then hold the stacked gate/up matrices).
* Packed codes and scale bytes are drawn per expert, each expert from its own
  child of stream [2] / [3], so any expert can be regenerated alone.
* x and shared are standard normal, drawn in float64, stored as float32; for
  bfloat16 workloads they are then rounded to bfloat16 (round to nearest
  even) and kept as float32 arrays that hold bfloat16-exact values.
* Packed bytes are uniform on 0..255; scale bytes uniform on [lo, hi]
  (inclusive).
* Routing draws K distinct experts per token by Gumbel-top-k, which is
  sequential sampling without replacement with weights w_e ("uniform":
  w = 1; Zipf(s): w_e = (e+1)^-s). Ties go to the lower expert index.
* Mixture weights are the softmax over K of N(0, std^2) logits (float64,
  stored as float32).
* Further routing draws (for timing runs that must not reuse the same
  experts call after call) continue streams [4] and [5].
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np

SEED_BASE = 20261202


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int  # seeds the streams: SeedSequence(SEED_BASE + index)
    T: int
    E: int
    K: int
    G: int
    O: int
    dtype: str  # "fp32" or "bf16": dtype of x, shared and y
    scale_lo: int
    scale_hi: int
    routing: str = "uniform"  # "uniform" or "zipf"
    zipf_s: float = 0.0
    logit_std: float = 1.0
    F: int = 0  # SwiGLU expert block: intermediate width (0: the routed linear alone)

    @property
    def I(self) -> int:  # noqa: E743 - the pages' name for the input width
        return 32 * self.G

    @property
    def P(self) -> int:
        return self.T * self.K

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The workloads. Names say what each is; sizes are in the fields.
WORKLOADS = {
    "tiny": Workload("tiny", 0, T=4, E=4, K=2, G=2, O=32, dtype="fp32",
                     scale_lo=124, scale_hi=130),
    "decode": Workload("decode", 1, T=1, E=128, K=4, G=90, O=5760, dtype="fp32",
                       scale_lo=118, scale_hi=128),
    "decode8": Workload("decode8", 2, T=8, E=384, K=8, G=224, O=4096, dtype="bf16",
                        scale_lo=118, scale_hi=128, routing="zipf", zipf_s=1.1),
    "prefill": Workload("prefill", 3, T=4096, E=128, K=4, G=90, O=5760, dtype="bf16",
                        scale_lo=118, scale_hi=128),
    "skewed": Workload("skewed", 4, T=8192, E=384, K=8, G=64, O=7168, dtype="bf16",
                       scale_lo=110, scale_hi=135, routing="zipf", zipf_s=1.2,
                       logit_std=math.sqrt(2.0)),
    # the prefill shape with fp32 activations (the prefill workload's seeds):
    # the grouped GEMM on the three-piece bf16 split
    "prefill_fp32": Workload("prefill_fp32", 3, T=4096, E=128, K=4, G=90, O=5760, dtype="fp32",
                             scale_lo=118, scale_hi=128),
    # SwiGLU expert block: decode8's gate/up shape (I = 7168, 2F = 4096)
    # feeding the skewed workload's down shape (F = 2048 -> O = 7168), with
    # the skewed workload's tokens and routing
    "swiglu": Workload("swiglu", 5, T=8192, E=384, K=8, G=224, O=7168, dtype="bf16",
                       scale_lo=118, scale_hi=128, routing="zipf", zipf_s=1.2,
                       logit_std=math.sqrt(2.0), F=2048),
}


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even).

    Returns float32 values that bfloat16 holds exactly. Inputs here are finite
    normal draws, so NaN handling is not needed.
    """
    bits = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    bits = (bits + 0x7FFF + ((bits >> 16) & 1)) & 0xFFFF0000
    return bits.astype(np.uint32).view(np.float32)


class ExpertTensor:
    """A lazily drawn per-expert uint8 tensor of shape (E, *inner).

    ``t[e]`` draws expert e from its own seeded stream, so a caller that
    needs only the selected experts never draws the rest.
    """

    def __init__(self, seq: np.random.SeedSequence, E: int, inner: tuple, lo: int, hi: int):
        self.E = E
        self.inner = tuple(inner)
        self.lo = lo
        self.hi = hi
        self._children = seq.spawn(E)
        self.shape = (E,) + self.inner
        self.dtype = np.dtype(np.uint8)

    def __len__(self) -> int:
        return self.E

    def __getitem__(self, e) -> np.ndarray:
        e = int(e)
        if not 0 <= e < self.E:
            raise IndexError(e)
        rng = np.random.Generator(np.random.PCG64(self._children[e]))
        return rng.integers(self.lo, self.hi + 1, size=self.inner, dtype=np.uint8)

    def materialize(self) -> np.ndarray:
        out = np.empty(self.shape, dtype=np.uint8)
        for e in range(self.E):
            out[e] = self[e]
        return out


def _log_weights(w: Workload) -> np.ndarray:
    if w.routing == "uniform":
        return np.zeros(w.E)
    if w.routing == "zipf":
        return -w.zipf_s * np.log(np.arange(1, w.E + 1, dtype=np.float64))
    raise ValueError(f"unknown routing {w.routing!r}")


def _draw_routing(w: Workload, rng_route, rng_logit, logw):
    key = rng_route.gumbel(size=(w.T, w.E)) + logw
    # descending key; stable so that equal keys keep the lower expert first
    sel = np.argsort(-key, axis=1, kind="stable")[:, : w.K].astype(np.int32)
    logits = rng_logit.normal(0.0, w.logit_std, size=(w.T, w.K))
    z = np.exp(logits - logits.max(axis=1, keepdims=True))
    p = (z / z.sum(axis=1, keepdims=True)).astype(np.float32)
    return np.ascontiguousarray(sel), np.ascontiguousarray(p)


@dataclasses.dataclass
class Inputs:
    workload: Workload
    x: np.ndarray  # float32 (T, I); bfloat16-exact values for bf16 workloads
    shared: np.ndarray  # float32 (T, O); bfloat16-exact for bf16 workloads
    packed: ExpertTensor  # (E, O, G, 16) uint8, lazily drawn; SwiGLU: gate/up (E, 2F, G, 16)
    scales: ExpertTensor  # (E, O, G) uint8, lazily drawn; SwiGLU: (E, 2F, G)
    sel: np.ndarray  # int32 (T, K)
    p: np.ndarray  # float32 (T, K)
    routing_sets: list  # further (sel, p) draws; [0] is (sel, p)
    dn_packed: ExpertTensor | None = None  # SwiGLU: down projection (E, O, F/32, 16)
    dn_scales: ExpertTensor | None = None  # SwiGLU: (E, O, F/32)


def make_inputs(w: Workload | str, n_routing_sets: int = 1) -> Inputs:
    """Draw the inputs of workload ``w`` (a Workload or a name in WORKLOADS)."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    if w.scale_lo < 0 or w.scale_hi > 255 or w.scale_lo > w.scale_hi:
        raise ValueError("scale range must lie in 0..255")
    if w.routing != "uniform" and w.K > w.E:
        raise ValueError("K distinct experts need K <= E")
    # children 0..5 as always; 6 and 7 draw the SwiGLU down projection
    s_x, s_sh, s_pk, s_sc, s_rt, s_lg, s_dp, s_ds = np.random.SeedSequence(SEED_BASE + w.index).spawn(8)
    x = np.random.Generator(np.random.PCG64(s_x)).standard_normal((w.T, w.I)).astype(np.float32)
    shared = np.random.Generator(np.random.PCG64(s_sh)).standard_normal((w.T, w.O)).astype(np.float32)
    if w.dtype == "bf16":
        x = round_to_bf16(x)
        shared = round_to_bf16(shared)
    elif w.dtype != "fp32":
        raise ValueError(f"unknown dtype {w.dtype!r}")
    rows = 2 * w.F if w.F else w.O
    packed = ExpertTensor(s_pk, w.E, (rows, w.G, 16), 0, 255)
    scales = ExpertTensor(s_sc, w.E, (rows, w.G), w.scale_lo, w.scale_hi)
    dn_packed = dn_scales = None
    if w.F:
        if w.F % 32:
            raise ValueError("the SwiGLU intermediate width must be a multiple of 32")
        dn_packed = ExpertTensor(s_dp, w.E, (w.O, w.F // 32, 16), 0, 255)
        dn_scales = ExpertTensor(s_ds, w.E, (w.O, w.F // 32), w.scale_lo, w.scale_hi)
    rng_route = np.random.Generator(np.random.PCG64(s_rt))
    rng_logit = np.random.Generator(np.random.PCG64(s_lg))
    logw = _log_weights(w)
    sets = [_draw_routing(w, rng_route, rng_logit, logw) for _ in range(max(1, n_routing_sets))]
    return Inputs(w, x, shared, packed, scales, sets[0][0], sets[0][1], sets, dn_packed, dn_scales)


def router_logits(T: int, E: int, seed: int, std: float = 1.0, grid: float | None = None,
                  bias_std: float | None = None):
    """Router inputs: logits (T, E) float32 ~ N(0, std^2) and, when bias_std
    is given, a per-expert bias (E,) float32 ~ N(0, bias_std^2), else None.
    ``grid`` rounds the logits to multiples of itself (and the bias to
    multiples of grid / 16), which plants exact ties. Streams: children 0
    (logits) and 1 (bias) of SeedSequence(SEED_BASE + 1000 + seed)."""
    s_l, s_b = np.random.SeedSequence(SEED_BASE + 1000 + seed).spawn(2)
    logits = np.random.Generator(np.random.PCG64(s_l)).normal(0.0, std, size=(T, E))
    bias = None
    if bias_std is not None:
        bias = np.random.Generator(np.random.PCG64(s_b)).normal(0.0, bias_std, size=E)
    if grid is not None:
        logits = np.round(logits / grid) * grid
        if bias is not None:
            bias = np.round(bias / (grid / 16)) * (grid / 16)
    logits = np.ascontiguousarray(logits.astype(np.float32))
    return logits, (None if bias is None else np.ascontiguousarray(bias.astype(np.float32)))


def unique_experts(sel: np.ndarray) -> np.ndarray:
    """Sorted distinct expert indices that appear in ``sel`` (routing summary)."""
    return np.unique(np.asarray(sel).ravel())
