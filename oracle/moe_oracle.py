"""Float64 oracle of one Mixture-of-Experts FFN layer's forward pass.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the library.  It shares no code with the
HIP path.

Every function computes the plain definition in float64, step by step in the
order the pages give it, with NumPy's matmul/argsort/cumsum as the only library
primitives.  Citations name the page and the section the step comes from:

  [Основы]   "Основы MoE" (ai.flicky.cc, stage 5.3)
  [Routage]  "Mixture-of-Experts : routage et capacité" (cours.spawnkit.ai, session 19)
  [Groupe]   "Le groupe d'experts (MoE)" (aiengineeringfromscratch.com, phase 07 lesson 11)
  [V4.1]     "Mixture-of-Experts" (mkdocs.reaper.mx, DeepSeek-V4.1-Flash / fondations)
  [Fiche]    "Mixture of Experts" fiche (dataistudio.com)

Readings of points the pages leave open (also listed in the design doc):

* Softmax gating selects on ``z + b`` (bias added to the raw router scores, as
  in [Groupe] "Étape 1: le routeur"); sigmoid gating selects on ``sigmoid(z) +
  b[modality]`` ([V4.1] "L'équilibrage de charge"); gate weights never include
  the selection bias.
* A logit offset ``o_e`` (an input) is added to the logits themselves and so
  affects both selection and weights.
* Ties between equal keys go to the lower expert index ([Основы] "Практика",
  the ``topk_route`` docstring: stable descending sort).
* Capacity ``C = ceil(T*k/E * f)`` is the exact ceiling of the rational value
  ([Routage] "L'idée — Capacité"); per expert the first C tokens in token order
  are kept; a dropped assignment contributes nothing and the surviving weights
  are not renormalised ([Routage] "Cas guidé — trace complète").
* SwiGLU expert: ``(silu(x W_gate) * (x W_up)) W_down`` with ``silu(a) =
  a*sigmoid(a)``; the V4.1 clip bounds that product to [-clip, clip]
  ([V4.1] table "Les chiffres de DeepSeek-V4.1-Flash": "écrêtée à 10").
* The shared expert has weight 1 and is added outside the renormalisation
  ([Routage] "L'idée — Top-k et mélange").
* Residual and normalisation around the layer are not part of it.

Weight layout (the library's): router ``[E][d]``, gate/up ``[E][I][d]``, down
``[E][d][I]`` -- each row is one output unit, i.e. the transpose of the pages'
``x @ W`` orientation.  For ReLU experts ``w_up = W1^T`` and ``w_down = W2^T``.
"""
from __future__ import annotations

import math
from fractions import Fraction
from typing import Callable, Optional, Sequence

import numpy as np

SOFTMAX, SIGMOID = "softmax", "sigmoid"
SWIGLU, RELU = "swiglu", "relu"

NEAR_TIE_REL = 1e-6


# ---------------------------------------------------------------------------
# 1. router projection and scoring

def router_logits(x: np.ndarray, w_router: np.ndarray,
                  logit_bias: Optional[np.ndarray] = None) -> np.ndarray:
    """z = x W_g (+ o): one logit per expert, a single linear layer without bias.

    [Основы] "Как устроен MoE-слой", step 1 (logits z = x W_g);
    [Groupe] "Étape 1: le routeur" (one dot product per expert).
    ``w_router`` is [E][d] (row e = column e of W_g)."""
    z = np.asarray(x, np.float64) @ np.asarray(w_router, np.float64).T
    if logit_bias is not None:
        z = z + np.asarray(logit_bias, np.float64)[None, :]
    return z


def softmax(z: np.ndarray) -> np.ndarray:
    """Max-subtracted softmax over the last axis ([Основы] "Практика", the
    ``softmax`` helper; [Routage] "Cas guidé — trace complète")."""
    z = np.asarray(z, np.float64)
    e = np.exp(z - z.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def sigmoid(z: np.ndarray) -> np.ndarray:
    """s = 1 / (1 + exp(-z)) -- the DeepSeek-V3 replacement of softmax
    ([Основы] "Как устроен MoE-слой", paragraph on model variants)."""
    z = np.asarray(z, np.float64)
    return 1.0 / (1.0 + np.exp(-z))


def scores(z: np.ndarray, gating: str) -> np.ndarray:
    if gating == SOFTMAX:
        return softmax(z)
    if gating == SIGMOID:
        return sigmoid(z)
    raise ValueError(gating)


def selection_keys(z: np.ndarray, s: np.ndarray, gating: str,
                   sel_bias: Optional[np.ndarray] = None,
                   modality: Optional[np.ndarray] = None) -> np.ndarray:
    """Keys that choose the experts.  The per-expert bias only moves the
    selection ([Groupe] "Étape 1: le routeur"; [V4.1] "L'équilibrage de
    charge"); with two bias sets each token uses its modality's set ([V4.1]
    "La nouveauté de V4.1 : l'équilibrage par modalité").
    Softmax gating: z + b.  Sigmoid gating: sigmoid(z) + b."""
    base = np.asarray(z if gating == SOFTMAX else s, np.float64)
    if sel_bias is None:
        return base.copy()
    b = np.asarray(sel_bias, np.float64)
    if b.ndim == 1:
        b = b[None, :]
    if b.shape[0] == 1:
        return base + b[0][None, :]
    if modality is None:
        raise ValueError("two bias sets need a modality flag per token")
    return base + b[np.asarray(modality, np.int64)]


# ---------------------------------------------------------------------------
# 2. top-k and gate weights

def topk(keys: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest keys per row, in descending key order; equal
    keys go to the lower index ([Основы] "Практика": ``np.argsort(-p,
    kind='stable')``).  Returns int64 [N, k]."""
    order = np.argsort(-np.asarray(keys, np.float64), axis=-1, kind="stable")
    return order[:, :k]


def gate_weights(s: np.ndarray, idx: np.ndarray, renormalize: bool = True) -> np.ndarray:
    """Renormalise the chosen (unbiased) scores: g_i = s_i / sum_{j in T} s_j.

    [Основы] "Как устроен MoE-слой", step 3; [Routage] "L'idée — Top-k et
    mélange" (0.529, 0.392 -> 0.574, 0.426).  For sigmoid gating the same rule
    applies to the sigmoid scores ([V4.1] "L'équilibrage de charge": combine
    weights come from the unbiased scores).

    ``renormalize=False`` keeps the chosen scores as they are: the Switch
    Transformer weight with k = 1 is the router probability p_i itself, not 1
    ([Основы] "Как устроен MoE-слой", paragraph on model variants; the
    ``MoE.forward`` code in "Эксперимент на PyTorch")."""
    chosen = np.take_along_axis(np.asarray(s, np.float64), idx, axis=-1)
    if not renormalize:
        return chosen
    return chosen / chosen.sum(axis=-1, keepdims=True)


def softmax_over_chosen(z: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Softmax taken over the chosen logits only ([Groupe] "Étape 1: le
    routeur"; [Fiche] code section).  Equal to ``gate_weights(softmax(z), idx)``
    in exact arithmetic."""
    return softmax(np.take_along_axis(np.asarray(z, np.float64), idx, axis=-1))


def route(x, w_router, k: int, gating: str, logit_bias=None, sel_bias=None,
          modality=None, check_softmax_identity: bool = True,
          renormalize: bool = True) -> dict:
    """Steps 1-4 of [Основы] "Как устроен MoE-слой" with the selection bias.

    Returns z, s (scores), keys, idx [N,k] int64 and g [N,k]."""
    z = router_logits(x, w_router, logit_bias)
    s = scores(z, gating)
    keys = selection_keys(z, s, gating, sel_bias, modality)
    idx = topk(keys, k)
    g = gate_weights(s, idx, renormalize)
    if gating == SOFTMAX and renormalize and check_softmax_identity and idx.size:
        alt = softmax_over_chosen(z, idx)
        if not np.allclose(alt, g, rtol=0, atol=1e-12):
            raise AssertionError("renormalised softmax differs from softmax over chosen")
    return {"z": z, "s": s, "keys": keys, "idx": idx, "g": g}


def near_ties(keys: np.ndarray, z: np.ndarray, k: int, rel: float = NEAR_TIE_REL):
    """Tokens whose top-k is not decided robustly in fp32-level arithmetic.

    With the float64 keys of token t sorted descending (ties to the lower
    index), let S_t = max(|key_(k)|, |key_(k+1)|, RMS_e z_te).  A token is
    *boundary-ambiguous* if |key_(k) - key_(k+1)| <= rel * S_t and
    *order-ambiguous* if two adjacent keys inside the top k meet the same test.
    Returns (boundary_mask [N], order_mask [N])."""
    keys = np.asarray(keys, np.float64)
    N, E = keys.shape
    if N == 0:
        return np.zeros(0, bool), np.zeros(0, bool)
    srt = -np.sort(-keys, axis=-1)
    rms = np.sqrt(np.mean(np.asarray(z, np.float64) ** 2, axis=-1))
    boundary = np.zeros(N, bool)
    if k < E:
        a, b = srt[:, k - 1], srt[:, k]
        S = np.maximum(np.maximum(np.abs(a), np.abs(b)), rms)
        boundary = np.abs(a - b) <= rel * S
    order = np.zeros(N, bool)
    for j in range(k - 1):
        a, b = srt[:, j], srt[:, j + 1]
        S = np.maximum(np.maximum(np.abs(a), np.abs(b)), rms)
        order |= np.abs(a - b) <= rel * S
    return boundary, order


# ---------------------------------------------------------------------------
# 3. dispatch: counts, capacity, token-order drops, slot rows

def capacity(f: float, N: int, k: int, E: int) -> Optional[int]:
    """C = ceil(T*k/E * f), computed exactly on the rational value of the
    binary double f ([Routage] "L'idée — Capacité" and "Cas guidé — trace
    complète").  f <= 0 means unlimited (returns None).  C >= 1 when f > 0."""
    if f is None or f <= 0:
        return None
    c = Fraction(N * k, E) * Fraction(f)
    return max(1, math.ceil(c))


def dispatch(idx: np.ndarray, E: int, C: Optional[int],
             modality: Optional[np.ndarray] = None) -> dict:
    """Per-expert demand, capacity and slot assignment in token order.

    Follows the per-expert structure of [Основы] "Эксперимент на PyTorch"
    (find the tokens that chose expert e, process them together) and the rule
    of [Routage] "Cas guidé — trace complète": tokens arrive in batch order and
    each expert keeps its first C arrivals; the rest are dropped.

    Returns counts [E] (demand, before capacity), modality_counts [2][E] or
    None, offsets [E+1] (prefix sums of kept counts), row_of [N,k] (slot row
    or -1 when dropped), token_of_row [A], drop_mask [N,k] (uint8).

    A replayed routing may hold indices outside [0, E): such an assignment
    goes to no expert, is not counted and is marked dropped (a definition for
    replay; routing itself never produces one)."""
    idx = np.asarray(idx, np.int64)
    N, k = idx.shape if idx.ndim == 2 else (0, 0)
    counts = np.zeros(E, np.int64)
    kept = np.zeros(E, np.int64)
    rank_of = np.full(idx.shape, -1, np.int64)
    for e in range(E):
        hit = idx == e                       # [N,k]; at most one True per row
        took = hit.any(axis=1)               # tokens that chose e
        counts[e] = int(took.sum())
        rank = np.cumsum(took) - 1           # arrival rank among tokens that chose e
        rank_of[hit] = np.broadcast_to(rank[:, None], hit.shape)[hit]
        kept[e] = counts[e] if C is None else min(counts[e], C)
    offsets = np.zeros(E + 1, np.int64)
    offsets[1:] = np.cumsum(kept)
    row_of = np.full(idx.shape, -1, np.int64)
    token_of_row = np.full(int(offsets[E]), -1, np.int64)
    drop = np.zeros(idx.shape, np.uint8)
    for e in range(E):
        hit = idx == e
        ranks = rank_of[hit]
        ok = ranks < (kept[e])
        rows = np.where(ok, offsets[e] + ranks, -1)
        row_of[hit] = rows
        drop[hit] = (~ok).astype(np.uint8)
        toks = np.nonzero(hit.any(axis=1))[0]          # token order
        tk = toks[: kept[e]]
        token_of_row[offsets[e]: offsets[e] + len(tk)] = tk
    mod_counts = None
    if modality is not None:
        mod = np.asarray(modality, np.int64)
        mod_counts = np.zeros((2, E), np.int64)
        for m in (0, 1):
            sel = idx[mod == m]
            for e in range(E):
                mod_counts[m, e] = int((sel == e).any(axis=1).sum()) if sel.size else 0
    drop[(idx < 0) | (idx >= E)] = 1
    return {"counts": counts, "modality_counts": mod_counts, "offsets": offsets,
            "row_of": row_of, "token_of_row": token_of_row, "drop_mask": drop,
            "C": C}


def alternates(keys: np.ndarray, k: int) -> np.ndarray:
    """The experts ranked k+1 .. 2k by key (same order and tie rule as topk);
    -1 where fewer than 2k experts exist.  int64 [N, k]."""
    keys = np.asarray(keys, np.float64)
    N, E = keys.shape
    order = np.argsort(-keys, axis=-1, kind="stable")
    alt = np.full((N, k), -1, np.int64)
    m = max(0, min(k, E - k))
    alt[:, :m] = order[:, k:k + m]
    return alt


def dispatch_reroute(idx: np.ndarray, alt: np.ndarray, E: int, C: Optional[int]) -> dict:
    """The overflow policy that hands a dropped assignment to the token's next
    expert ([Routage] "Politiques de débordement", row "Report sur E2/E3": t6,
    over capacity at E1, is processed by its third-best expert).

    Reading: first every expert keeps its first C arrivals in token order (the
    drop dispatch).  Then, walking the assignments in token order (slot order
    within a token), the q-th dropped slot of token t goes to alt[t, q] -- the
    token's (k+1+q)-th best expert -- if that expert still has room (C minus
    its first-round rows minus earlier rerouted rows), else it stays dropped.
    A rerouted slot keeps its gate weight.  Expert e's rows are its first-round
    rows (token order) followed by its rerouted rows (token order).

    Returns the drop dispatch's fields with row_of / token_of_row / drop_mask /
    offsets for the final placement, plus final_idx [N,k] (the expert that
    processes each slot, -1 if dropped)."""
    idx = np.asarray(idx, np.int64)
    alt = np.asarray(alt, np.int64)
    N, k = idx.shape
    first = dispatch(idx, E, C)
    drop1 = first["drop_mask"].astype(bool)
    kept1 = np.diff(first["offsets"])
    room = np.zeros(E, np.int64) if C is None else C - kept1
    taken = np.zeros(E, np.int64)
    final = np.where(drop1, -1, idx)
    rank2 = np.full((N, k), -1, np.int64)
    for t in range(N):
        q = 0
        for j in range(k):
            if not drop1[t, j]:
                continue
            c = alt[t, q] if q < k else -1
            q += 1
            if C is not None and 0 <= c < E and taken[c] < room[c]:
                final[t, j] = c
                rank2[t, j] = taken[c]
                taken[c] += 1
    total = kept1 + taken
    offsets = np.zeros(E + 1, np.int64)
    offsets[1:] = np.cumsum(total)
    row_of = np.full((N, k), -1, np.int64)
    token_of_row = np.full(int(offsets[E]), -1, np.int64)
    for t in range(N):
        for j in range(k):
            if not drop1[t, j]:
                e = idx[t, j]
                r = offsets[e] + (first["row_of"][t, j] - first["offsets"][e])
            elif rank2[t, j] >= 0:
                e = final[t, j]
                r = offsets[e] + kept1[e] + rank2[t, j]
            else:
                continue
            row_of[t, j] = r
            token_of_row[r] = t
    out = dict(first)
    out.update({"offsets": offsets, "row_of": row_of, "token_of_row": token_of_row,
                "drop_mask": (row_of < 0).astype(np.uint8), "final_idx": final})
    return out


def hash_route(token_ids, E: int, k: int):
    """A router without parameters ([Groupe] "Exercices", Medium: a
    deterministic hash-based router).  Reading: h = splitmix64(id) (S. Vigna's
    published 64-bit mixer: add the golden-ratio increment, then two
    xor-shift-multiply rounds and a final xor-shift); the token's experts are
    h mod E, h mod E + 1, ... (mod E) -- k distinct experts -- with equal
    weights 1/k.  Returns idx [N,k] int64 and g [N,k]."""
    M = (1 << 64) - 1
    ids = [int(v) & M for v in np.asarray(token_ids, np.int64).ravel()]
    idx = np.zeros((len(ids), k), np.int64)
    for t, v in enumerate(ids):
        z = (v + 0x9E3779B97F4A7C15) & M
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M
        z = z ^ (z >> 31)
        base = z % E
        idx[t] = [(base + j) % E for j in range(k)]
    return idx, np.full(idx.shape, 1.0 / k)


# ---------------------------------------------------------------------------
# 4. experts and combine

def silu(a: np.ndarray) -> np.ndarray:
    return a / (1.0 + np.exp(-a))


def expert_ffn(xr: np.ndarray, w_gate, w_up, w_down, activation: str,
               clip: float = 0.0) -> np.ndarray:
    """One expert on a block of rows.

    SwiGLU: h = silu(x W_gate) * (x W_up), clamped to [-clip, clip] when clip
    > 0, out = h W_down (three matrices per expert: [V4.1] "Le compte des
    paramètres"; clip: [V4.1] table).  ReLU: out = max(x W1, 0) W2 ([Fiche]
    code section)."""
    xr = np.asarray(xr, np.float64)
    up = xr @ np.asarray(w_up, np.float64).T
    if activation == SWIGLU:
        a = xr @ np.asarray(w_gate, np.float64).T
        h = silu(a) * up
        if clip and clip > 0:
            h = np.clip(h, -clip, clip)
    elif activation == RELU:
        h = np.maximum(up, 0.0)
    else:
        raise ValueError(activation)
    return h @ np.asarray(w_down, np.float64).T


def forward(x, k: int, E: int, gating: str, activation: str,
            get_expert: Callable[[int], Sequence], n_shared: int = 0,
            get_shared: Optional[Callable[[int], Sequence]] = None,
            w_router=None, clip: float = 0.0, f: float = 0.0,
            logit_bias=None, sel_bias=None, modality=None,
            forced_idx: Optional[np.ndarray] = None,
            tokens: Optional[np.ndarray] = None, renormalize: bool = True,
            forced_w: Optional[np.ndarray] = None, overflow: str = "drop") -> dict:
    """The whole layer: y_t = sum_{j kept} g_tj FFN_{e_tj}(x_t) + sum_s FFN_s(x_t).

    [Основы] "Как устроен MoE-слой", step 4; shared expert and drops:
    [Routage] "L'idée — Top-k et mélange" and "Cas guidé — trace complète".

    ``get_expert(e)`` returns float64 (w_gate, w_up, w_down) of routed expert e
    (w_gate None for ReLU); ``get_shared(s)`` likewise.  ``forced_idx`` replays
    a given routing: with ``forced_w`` the weights are taken as given (the
    router is not evaluated), otherwise they are recomputed from the scores.
    ``tokens`` restricts the output to those token rows (routing and capacity
    are still decided over the whole batch); the result 'y' then has
    len(tokens) rows.  ``overflow="reroute"`` applies dispatch_reroute with the
    router's alternates instead of dropping."""
    x = np.asarray(x, np.float64)
    N = x.shape[0]
    if forced_w is not None:
        r = {"z": None, "s": None, "keys": None}
        idx = np.asarray(forced_idx, np.int64)
        g = np.asarray(forced_w, np.float64)
    else:
        r = route(x, w_router, k, gating, logit_bias, sel_bias, modality,
                  renormalize=renormalize)
        idx = r["idx"] if forced_idx is None else np.asarray(forced_idx, np.int64)
        g = gate_weights(r["s"], np.clip(idx, 0, E - 1), renormalize)
    C = capacity(f, N, k, E)
    if overflow == "reroute":
        disp = dispatch_reroute(idx, alternates(r["keys"], k), E, C)
        if modality is not None:
            disp["modality_counts"] = dispatch(idx, E, C, modality)["modality_counts"]
        proc = disp["final_idx"]                            # expert processing each slot
    else:
        disp = dispatch(idx, E, C, modality)
        proc = idx
    want = np.arange(N) if tokens is None else np.asarray(tokens, np.int64)
    pos = {int(t): i for i, t in enumerate(want)}
    y = np.zeros((len(want), x.shape[1]), np.float64)
    row_of = disp["row_of"]
    for e in range(E):
        hit = (proc[want] == e) & (row_of[want] >= 0)       # kept assignments to e
        rows, slot = np.nonzero(hit)
        if rows.size == 0:
            continue
        wg, wu, wd = get_expert(e)
        out = expert_ffn(x[want[rows]], wg, wu, wd, activation, clip)
        np.add.at(y, rows, g[want[rows], slot][:, None] * out)
    for s_ in range(n_shared):
        wg, wu, wd = get_shared(s_)
        y += expert_ffn(x[want], wg, wu, wd, activation, clip)
    del pos
    return {"y": y, "z": r["z"], "s": r["s"], "keys": r["keys"], "idx": idx, "g": g,
            **disp}


# ---------------------------------------------------------------------------
# 4b. backward pass (gradients of L = sum(dy * y) for a given upstream dy)
#
# The pages give no backward; it is the chain rule through the forward above,
# with the selection (top-k, capacity, reroute) held fixed -- it is piecewise
# constant -- so the router is reached only through the gate weights (the
# reason the Switch top-1 weight is p_i and not 1: [Основы] "Как устроен
# MoE-слой", variants paragraph).  The clamp passes the gradient where
# -clip <= silu(a)*u <= clip and stops it outside.  Pinned by central finite
# differences of the forward.

def expert_ffn_backward(xr, w_gate, w_up, w_down, activation: str, clip: float,
                        d_out: np.ndarray):
    """Gradients of out = FFN(xr) for d(out) = d_out: (dx, dW_gate or None,
    dW_up, dW_down), float64, weights in the library layout."""
    xr = np.asarray(xr, np.float64)
    wu = np.asarray(w_up, np.float64)
    wd = np.asarray(w_down, np.float64)
    d_out = np.asarray(d_out, np.float64)
    up = xr @ wu.T
    if activation == SWIGLU:
        wg = np.asarray(w_gate, np.float64)
        a = xr @ wg.T
        sg = sigmoid(a)
        act = a * sg
        hpre = act * up
        h = np.clip(hpre, -clip, clip) if clip and clip > 0 else hpre
        dh = d_out @ wd
        if clip and clip > 0:
            dh = dh * (np.abs(hpre) <= clip)
        d_up = dh * act
        d_a = dh * up * (sg * (1.0 + a * (1.0 - sg)))
        return d_a @ wg + d_up @ wu, d_a.T @ xr, d_up.T @ xr, d_out.T @ h
    h = np.maximum(up, 0.0)
    d_up = (d_out @ wd) * (up > 0)
    return d_up @ wu, None, d_up.T @ xr, d_out.T @ h


def gate_backward(s: np.ndarray, z: np.ndarray, idx: np.ndarray, dg: np.ndarray,
                  gating: str, renormalize: bool = True) -> np.ndarray:
    """dz [N, E] from the gate weights' gradient dg [N, k] (gate_weights above,
    differentiated).  Only the chosen experts (and, for raw softmax weights,
    every expert through the softmax denominator) receive a gradient."""
    z = np.asarray(z, np.float64)
    N, E = z.shape
    dz = np.zeros((N, E))
    if N == 0:
        return dz
    s = np.asarray(s, np.float64)
    rows = np.arange(N)[:, None]
    if gating == SOFTMAX:
        if renormalize:
            g = softmax_over_chosen(z, idx)
            dz[rows, idx] = g * (dg - np.sum(g * dg, axis=1, keepdims=True))
        else:
            dp = np.zeros((N, E))
            dp[rows, idx] = dg
            dz = s * (dp - np.sum(s * dp, axis=1, keepdims=True))
    else:
        sc = np.take_along_axis(s, idx, axis=1)
        if renormalize:
            tot = sc.sum(axis=1, keepdims=True)
            g = sc / tot
            ds = (dg - np.sum(g * dg, axis=1, keepdims=True)) / tot
        else:
            ds = dg
        dz[rows, idx] = ds * sc * (1.0 - sc)
    return dz


def backward(x, k: int, E: int, gating: str, activation: str,
             get_expert: Callable[[int], Sequence], n_shared: int = 0,
             get_shared: Optional[Callable[[int], Sequence]] = None,
             w_router=None, clip: float = 0.0, f: float = 0.0,
             logit_bias=None, sel_bias=None, modality=None, dy=None,
             renormalize: bool = True, overflow: str = "drop") -> dict:
    """Gradients of L = sum(dy * y) w.r.t. x, every expert's weights, the
    shared experts, the router and the logit offset, for the routing the
    forward pass decides.  Returns dx, dW_gate/dW_up/dW_down (lists over
    experts; None for experts with no kept row), dWs_* (lists over shared
    experts), dW_router, d_logit_bias, dz, dg."""
    x = np.asarray(x, np.float64)
    dy = np.asarray(dy, np.float64)
    N, d = x.shape
    r = route(x, w_router, k, gating, logit_bias, sel_bias, modality,
              renormalize=renormalize, check_softmax_identity=False)
    idx = r["idx"]
    g = gate_weights(r["s"], idx, renormalize)
    C = capacity(f, N, k, E)
    if overflow == "reroute":
        disp = dispatch_reroute(idx, alternates(r["keys"], k), E, C)
        proc = disp["final_idx"]
    else:
        disp = dispatch(idx, E, C)
        proc = idx
    row_of = disp["row_of"]
    dx = np.zeros_like(x)
    dg = np.zeros((N, k))
    dWg, dWu, dWd = [None] * E, [None] * E, [None] * E
    for e in range(E):
        hit = (proc == e) & (row_of >= 0)
        rows, slot = np.nonzero(hit)
        if rows.size == 0:
            continue
        wg, wu, wd = get_expert(e)
        out = expert_ffn(x[rows], wg, wu, wd, activation, clip)
        dg[rows, slot] = np.sum(dy[rows] * out, axis=1)
        d_out = g[rows, slot][:, None] * dy[rows]
        dxe, dWg[e], dWu[e], dWd[e] = expert_ffn_backward(x[rows], wg, wu, wd, activation,
                                                          clip, d_out)
        np.add.at(dx, rows, dxe)
    dWsg, dWsu, dWsd = [], [], []
    for s_ in range(n_shared):
        wg, wu, wd = get_shared(s_)
        dxs, a_, b_, c_ = expert_ffn_backward(x, wg, wu, wd, activation, clip, dy)
        dx += dxs
        dWsg.append(a_)
        dWsu.append(b_)
        dWsd.append(c_)
    dz = gate_backward(r["s"], r["z"], idx, dg, gating, renormalize)
    dWr = dz.T @ x
    dx += dz @ np.asarray(w_router, np.float64)
    return {"dx": dx, "dW_gate": dWg, "dW_up": dWu, "dW_down": dWd, "dWs_gate": dWsg,
            "dWs_up": dWsu, "dWs_down": dWsd, "dW_router": dWr, "d_logit_bias": dz.sum(0),
            "dz": dz, "dg": dg, "route": r, **disp}


# ---------------------------------------------------------------------------
# 5. load-balancing statistics and the aux-loss-free bias update

def expert_load(counts, N: int, k: int) -> np.ndarray:
    """f_i = count_i / (T k): the share of the batch's assignments that went to
    expert i; sums to 1 ([Основы] "Практика", ``expert_load``).  An empty
    batch has no assignments: every share is 0 there (a reading)."""
    c = np.asarray(counts, np.float64)
    if N * k == 0:
        return np.zeros_like(c)
    return c / float(N * k)


def mean_router_probs(z: np.ndarray, gating: str) -> np.ndarray:
    """P_i: the batch mean of the probability the router gives expert i
    ([Основы] "Вспомогательный лосс Switch Transformer").  Softmax gating: the
    softmax of the logits.  Sigmoid gating (no softmax on the pages for it):
    the sigmoid scores normalised over all experts -- a reading."""
    z = np.asarray(z, np.float64)
    if z.shape[0] == 0:
        return np.zeros(z.shape[1])
    if gating == SOFTMAX:
        p = softmax(z)
    else:
        s = sigmoid(z)
        p = s / s.sum(axis=-1, keepdims=True)
    return p.mean(axis=0)


def switch_aux(f: np.ndarray, P: np.ndarray, alpha: float = 1.0) -> float:
    """alpha * N * sum_i f_i P_i with N the number of experts ([Основы]
    "Вспомогательный лосс Switch Transformer"; 1 when uniform, -> N on
    collapse)."""
    f = np.asarray(f, np.float64)
    return float(alpha * len(f) * np.sum(f * np.asarray(P, np.float64)))


def bias_update(bias, counts, n_tokens: int, k: int, gamma: float = 0.001) -> np.ndarray:
    """Aux-loss-free balancing step: an expert above its target load (n_tokens *
    k / E assignments) has its selection bias lowered by gamma, one below
    raised by gamma, one exactly on target left alone ([Groupe] "Le problème
    de l'équilibre de la charge", "Étape 2"; [V4.1] "L'équilibrage de charge";
    gamma = 0.001 in [V4.1] "La nouveauté de V4.1").  The comparison is exact
    (count * E against n_tokens * k in integers); the update is one float32
    addition, as the biases are float32."""
    counts = np.asarray(counts, np.int64)
    E = counts.shape[-1]
    diff = counts * E - n_tokens * k
    sgn = np.sign(diff).astype(np.float32)
    b = np.asarray(bias, np.float32)
    return (b - np.float32(gamma) * sgn).astype(np.float32)


def bias_update_by_modality(bias2, modality_counts, k: int, gamma: float = 0.001) -> np.ndarray:
    """Two independent bias sets, each updated from its own modality's loads and
    target N_m k / E ([V4.1] "La nouveauté de V4.1 : l'équilibrage par
    modalité").  N_m k is the modality's total number of assignments."""
    mc = np.asarray(modality_counts, np.int64)
    out = np.empty((2, mc.shape[1]), np.float32)
    for m in (0, 1):
        n_m = int(mc[m].sum()) // k
        out[m] = bias_update(np.asarray(bias2)[m], mc[m], n_m, k, gamma)
    return out


# ---------------------------------------------------------------------------
# closed forms (parameter counts)

def expert_params(d: int, I: int, activation: str = SWIGLU) -> int:
    """Parameters of one expert: 3*d*I for SwiGLU ([V4.1] "Le compte des
    paramètres"; [Основы] "Всего параметров и активных параметров"), 2*d*I for
    the two-layer ReLU expert ([Fiche] code section)."""
    return (3 if activation == SWIGLU else 2) * d * I


def layer_params(d: int, I: int, E: int, k: int, S: int, activation: str = SWIGLU):
    """(expert_total, expert_active, router) of one MoE layer: (E+S) experts
    stored, (k+S) run per token, plus the d*E router ([Основы] "Всего
    параметров и активных параметров")."""
    pe = expert_params(d, I, activation)
    return (E + S) * pe, (k + S) * pe, d * E
