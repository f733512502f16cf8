"""Pure-Python brute force of the MoE layer for tiny inputs.

TEST INFRASTRUCTURE ONLY.  Standard library only (no NumPy): every token is
handled on its own with explicit loops, the way the pages' per-token router
([Groupe] "Étape 1: le routeur") and the per-token loop of the NumPy fiche
([Fiche] code section) describe it.  Top-k is found by enumerating *every*
k-subset of the experts, not by sorting, so it checks ``moe_oracle.topk``
independently; the capacity rule is simulated by walking the batch in arrival
order with one counter per expert ([Routage] "Cas guidé — trace complète").

Inputs are nested lists of floats; weights use the library layout (router
[E][d], gate/up [E][I][d], down [E][d][I]).
"""
from __future__ import annotations

import itertools
import math


def dot(a, b):
    s = 0.0
    for u, v in zip(a, b):
        s += u * v
    return s


def best_subset(keys, k):
    """The k-subset with the largest key sum; among subsets of equal sum the
    lexicographically smallest index tuple wins (lower index first).  Returned
    in descending key order, equal keys by lower index."""
    E = len(keys)
    best, best_sum = None, -math.inf
    for comb in itertools.combinations(range(E), k):
        ssum = math.fsum(keys[i] for i in comb)
        if ssum > best_sum:          # strict: earlier (lexicographically smaller) wins ties
            best, best_sum = comb, ssum
    # order inside the subset: descending key, equal keys by lower index
    return sorted(best, key=lambda i: (-keys[i], i))


def route_token(x, w_router, k, gating, logit_bias=None, sel_bias=None, mod=0,
                renormalize=True):
    E = len(w_router)
    z = [dot(x, w_router[e]) + (logit_bias[e] if logit_bias is not None else 0.0)
         for e in range(E)]
    if gating == "softmax":
        m = max(z)
        ex = [math.exp(v - m) for v in z]
        tot = sum(ex)
        s = [v / tot for v in ex]
        base = z
    else:
        s = [1.0 / (1.0 + math.exp(-v)) for v in z]
        base = s
    if sel_bias is None:
        keys = list(base)
    else:
        b = sel_bias[mod] if isinstance(sel_bias[0], (list, tuple)) else sel_bias
        keys = [base[e] + b[e] for e in range(E)]
    chosen = best_subset(keys, k)
    if renormalize:
        tot = sum(s[e] for e in chosen)
        g = [s[e] / tot for e in chosen]
    else:                 # the scores themselves (Switch, k = 1: the probability p_i)
        g = [s[e] for e in chosen]
    return z, chosen, g


def ffn(x, wg, wu, wd, activation, clip=0.0):
    I = len(wu)
    h = [0.0] * I
    for i in range(I):
        u = dot(x, wu[i])
        if activation == "swiglu":
            a = dot(x, wg[i])
            v = a / (1.0 + math.exp(-a)) * u
            if clip and clip > 0:
                v = min(max(v, -clip), clip)
        else:
            v = u if u > 0.0 else 0.0
        h[i] = v
    return [dot(h, wd[j]) for j in range(len(wd))]


def layer(xs, w_router, experts, shared, k, gating, activation, clip=0.0,
          C=None, logit_bias=None, sel_bias=None, modality=None, renormalize=True):
    """Full layer over a tiny batch.  ``experts[e]`` / ``shared[s]`` are
    (wg, wu, wd) nested lists.  Returns (ys, chosen, gates, kept_flags)."""
    E = len(w_router)
    used = [0] * E
    ys, chosen_all, gates_all, kept_all = [], [], [], []
    for t, x in enumerate(xs):
        mod = modality[t] if modality is not None else 0
        _, chosen, g = route_token(x, w_router, k, gating, logit_bias, sel_bias, mod,
                                   renormalize)
        y = [0.0] * len(x)
        kept = []
        for e, w in zip(chosen, g):
            ok = C is None or used[e] < C
            used[e] += 1
            kept.append(ok)
            if ok:
                out = ffn(x, *experts[e], activation, clip)
                y = [a + w * b for a, b in zip(y, out)]
        for sh in shared:
            out = ffn(x, *sh, activation, clip)
            y = [a + b for a, b in zip(y, out)]
        ys.append(y)
        chosen_all.append(chosen)
        gates_all.append(g)
        kept_all.append(kept)
    return ys, chosen_all, gates_all, kept_all
