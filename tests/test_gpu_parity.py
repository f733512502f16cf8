"""GPU parity: the HIP library (through its C ABI) against the float64 oracle.

Small members of every workload family (several tiles per dimension and ragged
tails), the fp32 toy at its full size, and the edge cases of the method."""
import numpy as np
import pytest
import torch

import synth
from synth import device as sdev

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


SMALL = ["toy", "toy-s", "cap-s", "mix-s", "mixd-s", "ds-s", "v41-s", "relu-bf16-s"]


@pytest.mark.parametrize("name", SMALL)
def test_forward_parity_small(name):
    import parity
    w = synth.get(name)
    _say(f"[parity] {name} N={w.N} d={w.d} E={w.E} k={w.k} I={w.I} S={w.S}")
    rep, *_ = parity.full_check(w)
    _say(f"[parity] {name} {rep}")


def test_capacity_drops_really_happen():
    import parity
    w = synth.get("cap-s")
    rep, *_ = parity.full_check(w)
    assert rep["dropped"] > 0


EDGE = {
    "single-token": dict(base="ds-s", N=1),
    "one-expert": dict(base="mix-s", E=1, k=1, N=300),
    "k-equals-E": dict(base="mix-s", E=4, k=4, N=200),
    "capacity-one": dict(base="cap-s", f=1e-6, N=300),
    "many-empty-experts": dict(base="ds-s", N=9),
    "sigmoid-k1": dict(base="ds-s", k=1, N=257),
    "tail-rows-129": dict(base="cap-s", N=129, f=0.0),
    "no-shared-relu": dict(base="relu-bf16-s", S=0),
    "two-shared": dict(base="ds-s", S=2, N=200),
    # small batches split the router's reduction over several blocks
    "split-k-router": dict(base="mixd-s", N=8, d=1024),
    "split-k-router-ragged": dict(base="ds-s", N=3, d=1000, E=40, k=4),
    "f32-swiglu-clip": dict(base="toy-s", activation="swiglu", clip=0.05, S=1, N=150,
                            toy_draws=False),
    "f32-sigmoid-2bias": dict(base="toy-s", gating="sigmoid", n_bias_sets=2, image_frac=0.3,
                              N=300, toy_draws=False),
}


@pytest.mark.parametrize("case", sorted(EDGE))
def test_edge_cases(case):
    import parity
    spec = dict(EDGE[case])
    base = synth.get(spec.pop("base"))
    w = synth.derive(base, name=f"{base.name}-{case}", **spec)
    _say(f"[edge] {case} {w}")
    rep, *_ = parity.full_check(w)
    _say(f"[edge] {case} {rep}")


def test_collapse_to_one_expert_with_capacity():
    """Every token prefers expert 0 (a huge logit offset): with f = 1 the expert
    keeps its first C tokens, later tokens lose it (the Switch-style collapse of
    the MoE basics lesson)."""
    import parity
    w = synth.derive(synth.get("cap-s"), name="collapse", N=400, f=1.0, zipf_offset=0.0)
    inp = synth.make_inputs(w)
    inp.logit_bias = np.zeros(w.E, np.float32)
    inp.logit_bias[0] = 50.0
    rep, y, g, _ = parity.full_check(w, inp=inp)
    C = -(-(w.N * w.k) // w.E)
    assert g["counts"][0] == w.N and g["offsets"][1] == C
    assert rep["dropped"] >= w.N - C


def test_exact_tie_goes_to_lower_index():
    """Two experts with identical router rows have bit-identical logits; the
    lower index must come first (the topk_route rule of the MoE basics lesson)."""
    import parity
    w = synth.derive(synth.get("mix-s"), name="ties", N=256, E=8, k=2)
    inp = synth.make_inputs(w)
    inp.w_router = inp.w_router.copy()
    inp.w_router[5] = inp.w_router[2]
    di = sdev.upload(inp)
    y, out = parity.gpu_forward(w, di)
    g = parity.to_np(out)
    z = g["logits"].reshape(w.N, w.E)
    assert np.array_equal(z[:, 5], z[:, 2])
    idx = g["topk_idx"].reshape(w.N, w.k)
    both = np.all(np.isin(idx, [2, 5]), axis=1)
    first_of_pair = [row.tolist().index(2) < row.tolist().index(5)
                     for row in idx if 2 in row and 5 in row]
    assert all(first_of_pair)
    # with the pair tied, expert 5 can only be chosen together with expert 2
    assert all(2 in row for row in idx.tolist() if 5 in row)
    # a token whose best two are the tied pair chooses (2, 5) in that order
    if both.any():
        assert np.all(idx[both] == np.array([2, 5]))


def test_zero_tokens_is_a_noop():
    from mixture_experts_layer_16_amd import _lib as L
    import parity
    w = synth.derive(synth.get("cap-s"), name="empty", N=0)
    di = sdev.upload(synth.make_inputs(synth.derive(w, N=1)))
    p = parity.problem_of(w)
    y = torch.full((1, w.d), 3.0, dtype=torch.float32, device="cuda")
    ws = L.workspace(p)
    L.moe_forward(p, L.weights(di.w_router, di.w_gate, di.w_up, di.w_down, di.ws_gate, di.ws_up,
                               di.ws_down), di.x, di.logit_bias, None, None, y, None, ws)
    torch.cuda.synchronize()
    assert torch.all(y == 3.0)
