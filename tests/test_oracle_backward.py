"""Pins of the oracle's backward pass: central finite differences of the
forward oracle (L = sum(dy * y)) for every parameter kind, on tiny cases
whose routing does not change under the perturbation."""
import numpy as np
import pytest

from oracle import moe_oracle as O

H = 1e-6


def _case(seed, N=7, d=5, E=5, k=2, I=4, S=1, gating="softmax", activation="swiglu",
          clip=0.0, f=0.0, renormalize=True, overflow="drop", logit=True, bias=False):
    rng = np.random.default_rng(seed)
    c = dict(x=rng.normal(size=(N, d)), wr=rng.normal(size=(E, d)) * 0.7,
             W=[[rng.normal(size=(I, d)) * 0.6 if activation == "swiglu" else None,
                 rng.normal(size=(I, d)) * 0.6, rng.normal(size=(d, I)) * 0.6] for _ in range(E)],
             SH=[[rng.normal(size=(I, d)) * 0.6 if activation == "swiglu" else None,
                  rng.normal(size=(I, d)) * 0.6, rng.normal(size=(d, I)) * 0.6] for _ in range(S)],
             lb=rng.normal(size=E) * 0.3 if logit else None,
             sb=rng.uniform(-0.1, 0.1, size=(1, E)) if bias else None,
             dy=rng.normal(size=(N, d)), N=N, E=E, k=k, gating=gating, activation=activation,
             clip=clip, f=f, renormalize=renormalize, overflow=overflow, S=S)
    return c


def _fwd(c):
    return O.forward(c["x"], c["k"], c["E"], c["gating"], c["activation"],
                     get_expert=lambda e: c["W"][e], n_shared=c["S"],
                     get_shared=lambda s: c["SH"][s], w_router=c["wr"], clip=c["clip"],
                     f=c["f"], logit_bias=c["lb"], sel_bias=c["sb"],
                     renormalize=c["renormalize"], overflow=c["overflow"])


def _loss(c):
    out = _fwd(c)
    return float(np.sum(c["dy"] * out["y"])), out["idx"], out["row_of"]


def _bwd(c):
    return O.backward(c["x"], c["k"], c["E"], c["gating"], c["activation"],
                      get_expert=lambda e: c["W"][e], n_shared=c["S"],
                      get_shared=lambda s: c["SH"][s], w_router=c["wr"], clip=c["clip"],
                      f=c["f"], logit_bias=c["lb"], sel_bias=c["sb"], dy=c["dy"],
                      renormalize=c["renormalize"], overflow=c["overflow"])


def _fd_check(c, getter, analytic, n_probe=12, rng=None):
    """Central differences of L over n_probe random entries of the array
    getter(c) (modified in place), against the analytic gradient."""
    rng = rng or np.random.default_rng(0)
    arr = getter(c)
    L0, idx0, row0 = _loss(c)
    flat = arr.reshape(-1)
    picks = rng.choice(flat.size, size=min(n_probe, flat.size), replace=False)
    worst = 0.0
    for p in picks:
        v = flat[p]
        flat[p] = v + H
        Lp, ip, rp = _loss(c)
        flat[p] = v - H
        Lm, im, rm = _loss(c)
        flat[p] = v
        assert np.array_equal(ip, idx0) and np.array_equal(im, idx0), "routing moved"
        assert np.array_equal(rp, row0) and np.array_equal(rm, row0), "dispatch moved"
        num = (Lp - Lm) / (2 * H)
        ana = float(np.asarray(analytic).reshape(-1)[p])
        worst = max(worst, abs(num - ana) / max(1.0, abs(ana)))
    return worst


CASES = {
    "softmax-swiglu": dict(seed=1),
    "softmax-raw-clip": dict(seed=2, renormalize=False, clip=0.8),
    "sigmoid-renorm": dict(seed=3, gating="sigmoid", bias=True),
    "sigmoid-raw": dict(seed=4, gating="sigmoid", renormalize=False, bias=True),
    "relu-capacity": dict(seed=5, activation="relu", f=0.75, N=9),
    "reroute": dict(seed=6, f=0.75, N=9, overflow="reroute"),
    "switch-k1": dict(seed=7, k=1, renormalize=False, S=0),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_gradients_match_finite_differences(name):
    c = _case(**CASES[name])
    g = _bwd(c)
    tol = 2e-6
    assert _fd_check(c, lambda c: c["x"], g["dx"]) < tol
    assert _fd_check(c, lambda c: c["wr"], g["dW_router"]) < tol
    if c["lb"] is not None:
        assert _fd_check(c, lambda c: c["lb"], g["d_logit_bias"]) < tol
    for e in range(c["E"]):
        if g["dW_up"][e] is None:
            continue
        assert _fd_check(c, lambda c: c["W"][e][1], g["dW_up"][e], n_probe=6) < tol
        assert _fd_check(c, lambda c: c["W"][e][2], g["dW_down"][e], n_probe=6) < tol
        if c["activation"] == "swiglu":
            assert _fd_check(c, lambda c: c["W"][e][0], g["dW_gate"][e], n_probe=6) < tol
    for s in range(c["S"]):
        assert _fd_check(c, lambda c: c["SH"][s][1], g["dWs_up"][s], n_probe=6) < tol
        assert _fd_check(c, lambda c: c["SH"][s][2], g["dWs_down"][s], n_probe=6) < tol
        if c["activation"] == "swiglu":
            assert _fd_check(c, lambda c: c["SH"][s][0], g["dWs_gate"][s], n_probe=6) < tol


def test_cases_exercise_drops_clip_and_reroute():
    c = _case(**CASES["relu-capacity"])
    assert _fwd(c)["drop_mask"].sum() > 0
    c = _case(**CASES["reroute"])
    out = _fwd(c)
    assert np.any((out["final_idx"] != out["idx"]) & (out["final_idx"] >= 0))
    c = _case(**CASES["softmax-raw-clip"])
    hp = []
    for e in range(c["E"]):
        wg, wu, _ = c["W"][e]
        a = c["x"] @ wg.T
        hp.append(np.abs(O.silu(a) * (c["x"] @ wu.T)))
    assert max(float(v.max()) for v in hp) > 0.8       # the clamp is active somewhere


def test_selection_bias_gets_no_gradient_and_dropped_slots_none():
    # a dropped slot contributes nothing: its dg is 0; the selection bias only
    # moves the choice, so L does not change with it while the choice holds
    c = _case(**CASES["relu-capacity"])
    g = _bwd(c)
    assert np.all(g["dg"][g["drop_mask"] == 1] == 0)
    c = _case(**CASES["sigmoid-renorm"])
    L0, idx0, _ = _loss(c)
    c["sb"][0, 0] += 1e-7
    L1, idx1, _ = _loss(c)
    assert np.array_equal(idx0, idx1) and L1 == L0
