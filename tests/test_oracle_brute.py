"""The NumPy oracle against the pure-Python brute force on tiny inputs, and
mutation checks showing that plausible mistakes in the oracle are caught."""
import numpy as np
import pytest

import synth
from oracle import brute
from oracle import moe_oracle as O


def _case(seed, N, d, E, k, I, S, gating, activation, clip=0.0, f=0.0,
          n_bias_sets=0, logit=False, dup=False, renormalize=True):
    rng = np.random.default_rng(seed)
    x = rng.normal(size=(N, d))
    if n_bias_sets == 2:
        x[rng.random(N) < 0.3] += 0.5
    w_router = rng.normal(size=(E, d)) * 0.6
    if dup:
        # experts 0, 2 and 3 share one router row: their logits tie exactly,
        # so the lower-index-first rule decides the order and the boundary
        w_router[2] = w_router[0]
        w_router[3] = w_router[0]
    W = {e: ((rng.normal(size=(I, d)) if activation == "swiglu" else None),
             rng.normal(size=(I, d)), rng.normal(size=(d, I))) for e in range(E)}
    SH = [((rng.normal(size=(I, d)) if activation == "swiglu" else None),
           rng.normal(size=(I, d)), rng.normal(size=(d, I))) for _ in range(S)]
    lb = rng.normal(size=E) * 0.3 if logit else None
    sb = rng.uniform(-0.1, 0.1, size=(n_bias_sets, E)) if n_bias_sets else None
    mod = (rng.random(N) < 0.4).astype(np.uint8) if n_bias_sets == 2 else None
    return dict(x=x, w_router=w_router, W=W, SH=SH, k=k, E=E, gating=gating,
                activation=activation, clip=clip, f=f, lb=lb, sb=sb, mod=mod,
                renormalize=renormalize)


CASES = [
    dict(seed=1, N=12, d=5, E=6, k=2, I=4, S=0, gating="softmax", activation="swiglu"),
    dict(seed=2, N=16, d=6, E=8, k=3, I=5, S=1, gating="softmax", activation="swiglu", f=1.0),
    dict(seed=3, N=10, d=4, E=5, k=2, I=7, S=1, gating="sigmoid", activation="swiglu",
         n_bias_sets=1, clip=1.5),
    dict(seed=4, N=14, d=7, E=8, k=3, I=3, S=1, gating="sigmoid", activation="swiglu",
         n_bias_sets=2, clip=2.0, f=1.25),
    dict(seed=5, N=9, d=8, E=4, k=2, I=6, S=0, gating="softmax", activation="relu", logit=True),
    dict(seed=6, N=11, d=3, E=7, k=1, I=5, S=2, gating="softmax", activation="relu", f=0.5),
    dict(seed=7, N=8, d=4, E=4, k=4, I=3, S=0, gating="sigmoid", activation="swiglu"),
    dict(seed=8, N=12, d=3, E=5, k=2, I=3, S=0, gating="softmax", activation="swiglu", dup=True),
    # weights without renormalisation: Switch top-1 and a sigmoid top-2
    dict(seed=9, N=13, d=5, E=6, k=1, I=4, S=1, gating="softmax", activation="swiglu",
         f=1.0, renormalize=False),
    dict(seed=10, N=10, d=4, E=6, k=2, I=3, S=0, gating="sigmoid", activation="swiglu",
         n_bias_sets=1, renormalize=False),
]


def compare(c, oracle=O):
    """Max |oracle - brute| over y, plus whether indices/weights/drops agree."""
    xs = c["x"].tolist()
    experts = [tuple(None if a is None else a.tolist() for a in c["W"][e]) for e in range(c["E"])]
    shared = [tuple(None if a is None else a.tolist() for a in s) for s in c["SH"]]
    C = None                      # the brute force's own exact integer ceiling
    if c["f"] > 0:
        num, den = float(c["f"]).as_integer_ratio()
        C = max(1, -(-(len(xs) * c["k"] * num) // (c["E"] * den)))
    sb = None if c["sb"] is None else (c["sb"][0].tolist() if c["sb"].shape[0] == 1
                                       else [r.tolist() for r in c["sb"]])
    ys, chosen, gates, kept = brute.layer(
        xs, c["w_router"].tolist(), experts, shared, c["k"], c["gating"], c["activation"],
        c["clip"], C, None if c["lb"] is None else c["lb"].tolist(), sb,
        None if c["mod"] is None else c["mod"].tolist(), c["renormalize"])
    out = oracle.forward(c["x"], c["k"], c["E"], c["gating"], c["activation"],
                         get_expert=lambda e: c["W"][e], n_shared=len(c["SH"]),
                         get_shared=lambda s: c["SH"][s], w_router=c["w_router"],
                         clip=c["clip"], f=c["f"], logit_bias=c["lb"], sel_bias=c["sb"],
                         modality=c["mod"], renormalize=c["renormalize"])
    same_idx = out["idx"].tolist() == chosen
    dg = float(np.max(np.abs(out["g"] - np.array(gates))))
    same_drop = (out["drop_mask"] == 0).tolist() == kept
    dy = float(np.max(np.abs(out["y"] - np.array(ys)))) if len(ys) else 0.0
    return same_idx, dg, same_drop, dy


@pytest.mark.parametrize("spec", CASES, ids=lambda s: f"{s['gating']}-{s['activation']}-k{s['k']}-S{s['S']}-{s['seed']}"
                         + ("" if s.get("renormalize", True) else "-raw"))
def test_oracle_matches_brute_force(spec):
    c = _case(**spec)
    same_idx, dg, same_drop, dy = compare(c)
    assert same_idx
    assert dg < 1e-14
    assert same_drop
    assert dy < 1e-10


def test_capacity_bites_in_brute_cases():
    # the capacity cases above really drop something, so drops are exercised
    c = _case(**CASES[5])
    C = O.capacity(c["f"], 11, 1, 7)
    out = O.forward(c["x"], 1, 7, "softmax", "relu", get_expert=lambda e: c["W"][e],
                    w_router=c["w_router"], f=c["f"])
    assert C == 1 and out["drop_mask"].sum() > 0


def test_toy_fiche_layer_reexecuted():
    # The fiche's toy layer (8 two-layer ReLU experts, top-2, softmax over the
    # two chosen logits), re-executed per token in pure Python on the exact
    # float32 draws, against the oracle on the whole 1000-token batch.
    w = synth.get("toy")
    inp = synth.make_inputs(w)
    x = inp.x.astype(np.float64)
    wr = inp.w_router.astype(np.float64)
    W = {e: tuple(None if a is None else a.astype(np.float64) for a in inp.expert(e))
         for e in range(w.E)}
    out = O.forward(x, w.k, w.E, "softmax", "relu", get_expert=lambda e: W[e], w_router=wr)
    toks = list(range(0, 1000, 41))
    experts = [tuple(None if a is None else a.tolist() for a in W[e]) for e in range(w.E)]
    ys, chosen, gates, _ = brute.layer(x[toks].tolist(), wr.tolist(), experts, [], w.k,
                                       "softmax", "relu")
    assert out["idx"][toks].tolist() == chosen
    assert np.max(np.abs(out["y"][toks] - np.array(ys))) < 1e-12
    # every expert gets work; loads sum to one (the fiche's load printout)
    load = np.bincount(out["idx"].ravel(), minlength=w.E) / (w.N * w.k)
    assert abs(load.sum() - 1) < 1e-15 and np.all(load > 0)


# ---------------------------------------------------------------------------
# mutation checks: plant a mistake in (a copy of) the oracle, on the CPU, and
# make sure the brute-force comparison or a pin notices it.

class _Mutant:
    """A copy of the oracle module's namespace with some functions replaced.
    All functions share one globals dict, so helpers called indirectly (e.g.
    ``sigmoid`` via ``scores`` via ``route``) see the mutation too."""

    def __init__(self, **over):
        import types
        ns = dict(vars(O))
        ns.update(over)
        for name, val in list(ns.items()):
            if isinstance(val, types.FunctionType) and name not in over \
                    and val.__module__ == O.__name__:
                ns[name] = types.FunctionType(val.__code__, ns, val.__name__,
                                              val.__defaults__, val.__closure__)
        self.__dict__.update(ns)


def _any_case_differs(mut):
    for spec in CASES:
        c = _case(**spec)
        try:
            same_idx, dg, same_drop, dy = compare(c, mut)
        except Exception:
            return True
        if not same_idx or dg > 1e-12 or not same_drop or dy > 1e-8:
            return True
    return False


MUTANTS = {
    "topk ascending": dict(topk=lambda keys, k: np.argsort(np.asarray(keys), axis=-1,
                                                           kind="stable")[:, ::-1][:, :k]),
    "weights from keys": dict(gate_weights=lambda s, idx: np.take_along_axis(s, idx, -1)
                              * 0 + 1.0 / idx.shape[1]),
    "silu without sigmoid": dict(silu=lambda a: a),
    "sigmoid sign": dict(sigmoid=lambda z: 1.0 / (1.0 + np.exp(np.asarray(z, np.float64)))),
    "no renormalisation": dict(gate_weights=lambda s, idx: np.take_along_axis(s, idx, -1)),
    "capacity floor": dict(capacity=lambda f, N, k, E: None if f <= 0 else max(1, int(N * k / E * f) - 1)),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes_are_caught(name):
    mut = _Mutant(**MUTANTS[name])
    assert _any_case_differs(mut), f"mutation '{name}' went unnoticed"


def test_transposed_weight_is_caught():
    # a transposed down projection (d x I read as I x d) changes y on the
    # non-square shapes the brute-force cases use
    def bad_ffn(xr, wg, wu, wd, activation, clip=0.0):
        return O.expert_ffn(xr, wg, wu, np.asarray(wd).T.reshape(np.asarray(wd).shape),
                            activation, clip)
    mut = _Mutant(expert_ffn=bad_ffn)
    assert _any_case_differs(mut)
