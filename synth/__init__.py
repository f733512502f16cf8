"""Seeded synthetic inputs for the MoE-layer forward pass.

This module only *draws and encodes input data*: it holds no step of the
layer's arithmetic (no routing, no scoring, no FFN).  Both the float64 oracle
and the HIP path are fed from it, and neither imports the other.

Recipe (the same for every workload):

* every tensor is drawn from ``numpy.random.default_rng(SeedSequence([seed,
  tensor_id, expert]))`` so that one expert's weights can be regenerated
  without drawing the others;
* normal variates are drawn in float32 (``standard_normal``), scaled by the
  standard deviation in float32, then rounded once to bfloat16
  (round-to-nearest-even) for the bf16 workloads; the fp32 toy keeps float32;
* the bf16 *bits* are what the GPU receives; ``bf16_to_f64`` gives the oracle
  the exact same values.

Distributions follow the workload descriptions: weights N(0, 0.02), tokens
N(0, 1), selection biases U(-0.1, 0.1) in float32, image tokens N(0.5, 1.5)
(standard deviation 1.5).  The fp32 toy reproduces the draws of the NumPy
MoE-layer listing of the "Mixture of Experts" fiche (dataistudio.com, code
section): ``default_rng(42)``, W1, W2 and the router N(0, 0.1), tokens N(0, 1),
drawn in that order.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os
from dataclasses import dataclass, field, replace
from typing import Callable, Optional

import numpy as np

# tensor ids used in SeedSequence([seed, tensor_id, expert])
T_X, T_ROUTER, T_WGATE, T_WUP, T_WDOWN, T_SGATE, T_SUP, T_SDOWN = range(8)
T_SELBIAS, T_MODALITY, T_X_DECODE, T_X_IMAGE, T_X_IMAGE_DECODE = 8, 9, 10, 11, 12
T_DY = 13


@dataclass(frozen=True)
class Workload:
    """Shape and recipe of one MoE-layer workload."""
    name: str
    N: int                 # tokens
    d: int                 # model width
    E: int                 # routed experts
    k: int                 # experts per token
    I: int                 # expert inner size
    S: int = 0             # shared experts (same inner size I)
    f: float = 0.0         # capacity factor; <= 0 means unlimited
    gating: str = "softmax"      # "softmax" | "sigmoid"
    activation: str = "swiglu"   # "swiglu" | "relu"
    clip: float = 0.0            # 0 = no clamp of the SwiGLU product
    dtype: str = "bf16"          # "bf16" | "f32"
    n_bias_sets: int = 0         # 0, 1, or 2 (per modality)
    zipf_offset: float = 0.0     # s of the per-expert logit offset (e+1)^-s; 0 = none
    image_frac: float = 0.0      # fraction of image tokens (contiguous blocks)
    decode: bool = False         # decode token stream (same weights as prefill)
    seed: int = 0
    w_std: float = 0.02
    toy_draws: bool = False      # reproduce the NumPy fiche's draw order (toy layer)
    renormalize: bool = True     # gate weights renormalised over the k chosen
    overflow: str = "drop"       # "drop" | "reroute": fate of assignments past capacity
    notes: str = ""


# The named workloads.  Sizes are the ones the MoE-layer descriptions give.
WORKLOADS = {
    "toy": Workload("toy", N=1000, d=64, E=8, k=2, I=256, S=0, gating="softmax",
                    activation="relu", dtype="f32", seed=42, w_std=0.1, toy_draws=True,
                    notes="NumPy MoE fiche toy: 8 two-layer ReLU experts, top-2"),
    "cap": Workload("cap", N=16384, d=2048, E=64, k=2, I=1408, S=1, f=1.0,
                    gating="softmax", zipf_offset=1.1, seed=1,
                    notes="capacity/drop layer, C=ceil(N*k/E)"),
    "mix-P": Workload("mix-P", N=8192, d=4096, E=8, k=2, I=14336, seed=2,
                      notes="Mixtral-shaped prefill"),
    "mix-D": Workload("mix-D", N=16, d=4096, E=8, k=2, I=14336, seed=2, decode=True,
                      notes="Mixtral-shaped decode"),
    "ds-P": Workload("ds-P", N=8192, d=7168, E=256, k=8, I=2048, S=1,
                     gating="sigmoid", n_bias_sets=1, seed=3,
                     notes="DeepSeek-V3-shaped prefill"),
    "ds-D": Workload("ds-D", N=32, d=7168, E=256, k=8, I=2048, S=1,
                     gating="sigmoid", n_bias_sets=1, seed=3, decode=True,
                     notes="DeepSeek-V3-shaped decode"),
    "v41": Workload("v41", N=16384, d=5120, E=384, k=6, I=2304, S=1,
                    gating="sigmoid", n_bias_sets=2, clip=10.0, image_frac=0.3,
                    seed=4, notes="DeepSeek-V4.1-Flash-shaped multimodal layer"),
}

# Small members of each family: several tiles per dimension plus ragged tails,
# sized so that the float64 oracle finishes in well under a second.
SMALL = {
    "toy-s": replace(WORKLOADS["toy"], name="toy-s", N=203, seed=7),
    "cap-s": replace(WORKLOADS["cap"], name="cap-s", N=1000, d=320, E=16, I=200, seed=11),
    "mix-s": replace(WORKLOADS["mix-P"], name="mix-s", N=777, d=256, E=8, I=392, seed=12),
    "mixd-s": replace(WORKLOADS["mix-D"], name="mixd-s", N=5, d=256, E=8, I=392, seed=12),
    "ds-s": replace(WORKLOADS["ds-P"], name="ds-s", N=530, d=448, E=64, k=8, I=136, seed=13),
    "v41-s": replace(WORKLOADS["v41"], name="v41-s", N=1100, d=320, E=96, k=6, I=144,
                     seed=14),
    "relu-bf16-s": replace(WORKLOADS["cap"], name="relu-bf16-s", N=300, d=192, E=6, k=2,
                           I=264, S=1, f=1.25, activation="relu", zipf_offset=0.0, seed=15),
    # many experts averaging more than 256 rows, with a skewed spread (one empty
    # expert, ~60 above 256 rows, remainders past the last 256-row tile both
    # below and above 128 rows): the grouped-GEMM tile plan of the DeepSeek-
    # and V4.1-shaped prefill layers at a size the oracle runs in seconds
    "ds-split-s": replace(WORKLOADS["ds-P"], name="ds-split-s", N=6000, d=320, E=160, k=8,
                          I=200, seed=16),
    # the V4.1-shaped small layer with the activation clip lowered to 0.06, so
    # that the clamp is active on a large share of the hidden elements
    "v41-clip-s": replace(WORKLOADS["v41"], name="v41-clip-s", N=1100, d=320, E=96, k=6,
                          I=144, clip=0.06, seed=14),
}

ALL = {**WORKLOADS, **SMALL}


def get(name: str) -> Workload:
    return ALL[name]


# ---------------------------------------------------------------------------
# encoding helpers (data representation only)

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    b = a.view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(bits).astype(np.float64)


def _rng(seed: int, tensor: int, expert: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, tensor, expert]))


def _normal(rng, shape, mean, std) -> np.ndarray:
    v = rng.standard_normal(shape, dtype=np.float32)
    v *= np.float32(std)
    if mean:
        v += np.float32(mean)
    return v


def _encode(w: Workload, a32: np.ndarray) -> np.ndarray:
    return f32_to_bf16_bits(a32) if w.dtype == "bf16" else np.ascontiguousarray(a32)


def to_f64(w: Workload, arr: np.ndarray) -> np.ndarray:
    """Exact float64 values of an encoded array (bf16 bits or float32)."""
    return bf16_to_f64(arr) if (w.dtype == "bf16" and arr.dtype == np.uint16) else \
        np.asarray(arr, dtype=np.float64)


# ---------------------------------------------------------------------------
# per-tensor generators

def modality_flags(w: Workload) -> Optional[np.ndarray]:
    """uint8 [N]: 0 = text, 1 = image.  The tokens are split into segments of
    2048 (fewer if N is smaller); each segment holds one contiguous image block
    of floor(image_frac * segment) tokens at a seeded start."""
    if w.n_bias_sets != 2:
        return None
    if w.N == 0:
        return np.zeros(0, dtype=np.uint8)
    seg = min(2048, w.N)
    nseg = max(1, w.N // seg)
    flags = np.zeros(w.N, dtype=np.uint8)
    rng = _rng(w.seed, T_MODALITY, 1 if w.decode else 0)
    for s in range(nseg):
        lo = s * seg
        hi = w.N if s == nseg - 1 else lo + seg
        n = hi - lo
        blk = int(np.floor(w.image_frac * n))
        if blk <= 0:
            continue
        start = int(rng.integers(0, n - blk + 1))
        flags[lo + start: lo + start + blk] = 1
    return flags


def tokens(w: Workload) -> np.ndarray:
    """x [N, d], encoded (bf16 bits or float32)."""
    if w.toy_draws:
        return _toy_draws(w)["tokens"]
    t_id = T_X_DECODE if w.decode else T_X
    x = _normal(_rng(w.seed, t_id), (w.N, w.d), 0.0, 1.0)
    flags = modality_flags(w)
    if flags is not None and flags.any():
        img = _normal(_rng(w.seed, T_X_IMAGE_DECODE if w.decode else T_X_IMAGE),
                      (int(flags.sum()), w.d), 0.5, 1.5)
        x[flags.astype(bool)] = img
    return _encode(w, x)


def router(w: Workload) -> np.ndarray:
    """Router weights in the library layout [E][d] (row e scores expert e)."""
    if w.toy_draws:
        return _toy_draws(w)["router"]
    return _encode(w, _normal(_rng(w.seed, T_ROUTER), (w.E, w.d), 0.0, w.w_std))


def logit_offset(w: Workload) -> Optional[np.ndarray]:
    """float32 [E] per-expert logit offset (e+1)^-s (Zipf skew), or None."""
    if not w.zipf_offset:
        return None
    e = np.arange(1, w.E + 1, dtype=np.float64)
    return (e ** (-w.zipf_offset)).astype(np.float32)


def upstream_grad(w: Workload) -> np.ndarray:
    """float32 [N][d] ~ N(0, 1): the gradient dL/dy fed to the backward pass."""
    return _normal(_rng(w.seed, T_DY), (w.N, w.d), 0.0, 1.0)


def selection_bias(w: Workload) -> Optional[np.ndarray]:
    """float32 [n_bias_sets][E] ~ U(-0.1, 0.1), or None."""
    if w.n_bias_sets == 0:
        return None
    rng = _rng(w.seed, T_SELBIAS)
    return rng.uniform(-0.1, 0.1, size=(w.n_bias_sets, w.E)).astype(np.float32)


def expert_weights(w: Workload, e: int, shared: bool = False):
    """(w_gate [I][d] or None, w_up [I][d], w_down [d][I]) for routed expert e or
    shared expert e, encoded.  For ReLU experts w_up = W1^T and w_down = W2^T."""
    if w.toy_draws:
        t = _toy_draws(w)
        return None, t["w_up"][e], t["w_down"][e]
    tg, tu, td = (T_SGATE, T_SUP, T_SDOWN) if shared else (T_WGATE, T_WUP, T_WDOWN)
    wg = None
    if w.activation == "swiglu":
        wg = _encode(w, _normal(_rng(w.seed, tg, e), (w.I, w.d), 0.0, w.w_std))
    wu = _encode(w, _normal(_rng(w.seed, tu, e), (w.I, w.d), 0.0, w.w_std))
    wd = _encode(w, _normal(_rng(w.seed, td, e), (w.d, w.I), 0.0, w.w_std))
    return wg, wu, wd


_TOY_CACHE: dict = {}


def _toy_draws(w: Workload) -> dict:
    """Draws of the NumPy fiche's toy layer (default_rng(seed); W1 (E,d,h), W2
    (E,h,d), router (d,E), tokens (N,d), in that order), cast to float32 and
    laid out for the library ([E][d] router, W1^T, W2^T)."""
    key = (w.seed, w.N, w.d, w.E, w.I)
    if key not in _TOY_CACHE:
        rng = np.random.default_rng(w.seed)
        W1 = rng.normal(0, w.w_std, (w.E, w.d, w.I))
        W2 = rng.normal(0, w.w_std, (w.E, w.I, w.d))
        R = rng.normal(0, w.w_std, (w.d, w.E))
        X = rng.normal(0, 1, (w.N, w.d))
        _TOY_CACHE[key] = {
            "tokens": np.ascontiguousarray(X.astype(np.float32)),
            "router": np.ascontiguousarray(R.T.astype(np.float32)),
            "w_up": np.ascontiguousarray(np.transpose(W1, (0, 2, 1)).astype(np.float32)),
            "w_down": np.ascontiguousarray(np.transpose(W2, (0, 2, 1)).astype(np.float32)),
        }
    return _TOY_CACHE[key]


# ---------------------------------------------------------------------------
# bundles

@dataclass
class Inputs:
    """All inputs of one workload.  Expert weights are produced lazily, one
    expert at a time, by ``expert(e)`` / ``shared(s)`` (encoded arrays)."""
    w: Workload
    x: np.ndarray
    w_router: np.ndarray
    logit_bias: Optional[np.ndarray]
    sel_bias: Optional[np.ndarray]
    modality: Optional[np.ndarray]
    _cache: dict = field(default_factory=dict)

    def expert(self, e: int):
        key = ("r", e)
        if key in self._cache:
            return self._cache[key]
        return expert_weights(self.w, e, shared=False)

    def shared(self, s: int):
        key = ("s", s)
        if key in self._cache:
            return self._cache[key]
        return expert_weights(self.w, s, shared=True)

    def materialize(self, threads: Optional[int] = None) -> "Inputs":
        """Generate and keep every expert's weights (threaded)."""
        jobs = [("r", e) for e in range(self.w.E)] + [("s", s) for s in range(self.w.S)]
        todo = [j for j in jobs if j not in self._cache]
        nthr = threads or min(16, os.cpu_count() or 1)
        with _cf.ThreadPoolExecutor(nthr) as ex:
            res = ex.map(lambda j: expert_weights(self.w, j[1], shared=(j[0] == "s")), todo)
            for j, r in zip(todo, res):
                self._cache[j] = r
        return self

    def stacked(self, which: str, shared: bool = False) -> Optional[np.ndarray]:
        """Stack one weight kind over all (routed or shared) experts: which in
        {"gate", "up", "down"}.  Materialises the weights if needed."""
        n = self.w.S if shared else self.w.E
        if n == 0:
            return None
        pos = {"gate": 0, "up": 1, "down": 2}[which]
        arrs = [(self.shared(i) if shared else self.expert(i))[pos] for i in range(n)]
        if arrs[0] is None:
            return None
        return np.stack(arrs)


def make_inputs(name_or_w, materialize: bool = False) -> Inputs:
    w = get(name_or_w) if isinstance(name_or_w, str) else name_or_w
    inp = Inputs(w=w, x=tokens(w), w_router=router(w), logit_bias=logit_offset(w),
                 sel_bias=selection_bias(w), modality=modality_flags(w))
    if materialize:
        inp.materialize()
    return inp


def derive(w: Workload, **changes) -> Workload:
    """A workload with some fields changed (used by tests for edge cases)."""
    return replace(w, **changes)
