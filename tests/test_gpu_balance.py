"""GPU parity of the load-balancing statistics and the aux-loss-free bias update
(moe_balance) against the oracle.

Every full_check in the other GPU tests already runs moe_balance on its
routing; the cases here add the closed forms (one expert, k = E, collapse),
the size limits (1024 experts, more tokens than the statistics kernel has
blocks), the empty batch, and the training loop the lessons describe: route,
measure the loads, move the biases, route again -- the GPU's biases equal the
oracle's bit for bit at every step and the loads approach uniform."""
import numpy as np
import pytest
import torch

import synth
from synth import device as sdev
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _run(w, inp=None):
    import parity
    rep, y, g, di = parity.full_check(w, inp=inp)
    _say(f"[balance] {w.name} {dict((k, v) for k, v in rep.items() if k != 'modality_counts')}")
    return rep, g


def _stats(w, g, di):
    """Load, P and aux from the GPU for the routing in g (no bias update)."""
    from mixture_experts_layer_16_amd import _lib as L
    import parity
    p = parity.problem_of(w)
    dev = "cuda"
    logits = torch.from_numpy(g["logits"]).to(dev)
    counts = torch.from_numpy(g["counts"]).to(dev)
    load = torch.empty(w.E, dtype=torch.float64, device=dev)
    prob = torch.empty(w.E, dtype=torch.float64, device=dev)
    aux = torch.empty(1, dtype=torch.float64, device=dev)
    L.moe_balance(p, logits, counts, None, load, prob, aux, None, 0.0, L.workspace(p))
    torch.cuda.synchronize()
    return load.cpu().numpy(), prob.cpu().numpy(), float(aux.item())


def test_single_expert_is_uniform():
    w = synth.derive(synth.get("toy-s"), name="bal-one", E=1, k=1, N=300, toy_draws=False)
    rep, g = _run(w)
    assert rep["aux"] == 1.0


def test_k_equals_e_is_on_target():
    # every token takes every expert: all loads equal the target, the biases
    # stay, and (softmax) the statistic is sum_e P_e = 1
    w = synth.derive(synth.get("toy-s"), name="bal-kE", E=4, k=4, N=333, toy_draws=False,
                     n_bias_sets=1)
    rep, g = _run(w)
    assert rep["bias_moved"] == 0
    assert abs(rep["aux"] - 1.0) < 1e-14


def test_collapse_tends_to_e():
    # a huge logit offset sends every token to expert 0 (k = 1): f = e_0 and
    # P_0 -> 1, so the statistic is E * P_0 ~ E
    w = synth.derive(synth.get("toy-s"), name="bal-collapse", k=1, N=500, toy_draws=False,
                     n_bias_sets=1, gating="softmax")
    inp = synth.make_inputs(w)
    inp.logit_bias = np.zeros(w.E, np.float32)
    inp.logit_bias[0] = 40.0
    rep, g = _run(w, inp)
    assert g["counts"][0] == w.N
    assert w.E * (1 - 1e-12) < rep["aux"] <= w.E
    # the overloaded expert's bias goes down, every other one's up
    assert rep["bias_moved"] == w.E


def test_max_experts():
    w = synth.derive(synth.get("toy-s"), name="bal-1024", E=1024, k=4, N=700, I=16,
                     toy_draws=False, gating="sigmoid", n_bias_sets=1)
    _run(w)


def test_more_tokens_than_blocks():
    # 40000 tokens > 512 blocks x 64 tokens: each block takes a longer chunk
    w = synth.derive(synth.get("toy-s"), name="bal-many", N=40000, I=16, toy_draws=False,
                     n_bias_sets=1)
    _run(w)


def test_empty_batch():
    from mixture_experts_layer_16_amd import _lib as L
    import parity
    w = synth.derive(synth.get("ds-s"), name="bal-empty", N=0)
    p = parity.problem_of(w)
    dev = "cuda"
    logits = torch.zeros(1, dtype=torch.float64, device=dev)
    counts = torch.zeros(w.E, dtype=torch.int32, device=dev)
    load = torch.full((w.E,), np.nan, dtype=torch.float64, device=dev)
    prob = torch.full((w.E,), np.nan, dtype=torch.float64, device=dev)
    aux = torch.full((1,), np.nan, dtype=torch.float64, device=dev)
    b0 = torch.from_numpy(synth.selection_bias(w)).to(dev)
    bias = b0.clone()
    L.moe_balance(p, logits, counts, None, load, prob, aux, bias, 0.001, L.workspace(p))
    torch.cuda.synchronize()
    assert torch.all(load == 0) and torch.all(prob == 0) and aux.item() == 0.0
    assert torch.equal(bias, b0)


def test_statistics_are_deterministic():
    w = synth.get("v41-s")
    import parity
    inp = synth.make_inputs(w)
    di = sdev.upload(inp)
    _, out = parity.gpu_forward(w, di)
    g = parity.to_np(out)
    a = _stats(w, g, di)
    b = _stats(w, g, di)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]) and a[2] == b[2]


@pytest.mark.parametrize("sets", [1, 2])
def test_balancing_loop_matches_oracle(sets):
    """Route -> loads -> bias update, repeated: the GPU's float32 biases equal the
    oracle's at every step, and the most loaded expert's excess shrinks."""
    from mixture_experts_layer_16_amd import _lib as L
    import parity
    w = synth.derive(synth.get("toy-s"), name=f"bal-loop-{sets}", N=2000, d=64, E=16, k=2, I=16,
                     toy_draws=False, gating="sigmoid", n_bias_sets=sets, zipf_offset=0.8,
                     image_frac=0.3, seed=31 + sets)
    inp = synth.make_inputs(w)
    inp.sel_bias = np.zeros((sets, w.E), np.float32)
    di = sdev.upload(inp)
    p = parity.problem_of(w)
    ws = L.workspace(p)
    rt = parity.alloc_routing(w)
    dev = "cuda"
    bias = torch.zeros(sets * w.E, dtype=torch.float32, device=dev)
    x64 = synth.to_f64(w, inp.x)
    wr64 = synth.to_f64(w, inp.w_router)
    lb64 = None if inp.logit_bias is None else inp.logit_bias.astype(np.float64)
    mod = inp.modality if sets == 2 else None
    ob = np.zeros((sets, w.E), np.float32)
    gamma = 0.01
    target = w.N * w.k / w.E
    excess = []
    for it in range(30):
        L.moe_route(p, di.x, di.w_router, di.logit_bias, bias, di.modality, rt["topk_idx"],
                    rt["topk_w"], rt["logits"], ws)
        L.moe_permute(p, rt["topk_idx"], di.modality, rt["counts"], rt["modality_counts"],
                      rt["offsets"], rt["row_of"], rt["token_of_row"], rt["drop_mask"], ws)
        L.moe_balance(p, rt["logits"], rt["counts"], rt["modality_counts"], None, None, None,
                      bias, gamma, ws)
        torch.cuda.synchronize()
        r = O.route(x64, wr64, w.k, w.gating, lb64, ob.astype(np.float64), mod)
        d = O.dispatch(r["idx"], w.E, None, mod)
        gc = rt["counts"].cpu().numpy()
        assert np.array_equal(gc, d["counts"]), it
        if sets == 1:
            ob = O.bias_update(ob[0], d["counts"], w.N, w.k, gamma)[None, :]
        else:
            ob = O.bias_update_by_modality(ob, d["modality_counts"], w.k, gamma)
        gb = bias.cpu().numpy().reshape(sets, w.E)
        assert np.array_equal(gb.view(np.uint32), ob.view(np.uint32)), it
        excess.append(gc.max() / target)
    _say(f"[balance] loop sets={sets} max-load/target: {excess[0]:.3f} -> {excess[-1]:.3f}")
    assert excess[-1] < excess[0]
