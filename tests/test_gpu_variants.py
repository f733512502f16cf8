"""GPU parity of the routing variants: gate weights without renormalisation
(Switch top-1 style) and the routing-replay entry point moe_forward_routed."""
import numpy as np
import pytest
import torch

import synth
from synth import device as sdev
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


RAW = {
    # Switch: top-1, weight = p_i, with capacity
    "switch-k1-cap": dict(base="cap-s", k=1, f=1.0, renormalize=False),
    "sigmoid-raw": dict(base="ds-s", renormalize=False),
    "softmax-raw-k2": dict(base="mix-s", renormalize=False),
    "f32-raw": dict(base="toy-s", toy_draws=False, renormalize=False),
    "v41-raw": dict(base="v41-s", renormalize=False),
}


@pytest.mark.parametrize("case", sorted(RAW))
def test_raw_weights(case):
    import parity
    spec = dict(RAW[case])
    base = synth.get(spec.pop("base"))
    w = synth.derive(base, name=f"{base.name}-{case}", **spec)
    _say(f"[raw] {case} {w}")
    rep, y, g, _ = parity.full_check(w)
    _say(f"[raw] {case} {dict((k, v) for k, v in rep.items() if k != 'modality_counts')}")
    # raw softmax weights are probabilities: positive, summing to at most 1
    gw = g["topk_w"][: w.N * w.k].reshape(w.N, w.k)
    assert np.all(gw > 0)
    if w.gating == "softmax":
        assert np.all(gw.sum(1) <= 1.0 + 1e-6)


def _run_routed(w, di, idx_t, w_t, ws=None):
    from mixture_experts_layer_16_amd import _lib as L
    import parity
    p = parity.problem_of(w)
    out = parity.alloc_routing(w, "cuda")
    y = torch.full((max(1, w.N), w.d), float("nan"), dtype=torch.float32, device="cuda")
    r = L.routing(**{k: v for k, v in out.items()
                     if v is not None and k not in ("topk_idx", "topk_w", "logits")})
    L.moe_forward_routed(p, L.weights(None, di.w_gate, di.w_up, di.w_down, di.ws_gate,
                                      di.ws_up, di.ws_down),
                         di.x, idx_t, w_t, di.modality, y, r, ws if ws is not None else L.workspace(p))
    torch.cuda.synchronize()
    return y, parity.to_np(out)


@pytest.mark.parametrize("name", ["cap-s", "v41-s", "toy-s"])
def test_replay_of_own_routing_is_bit_exact(name):
    import parity
    w = synth.get(name)
    inp = synth.make_inputs(w)
    di = sdev.upload(inp)
    y0, out0 = parity.gpu_forward(w, di)
    y1, g1 = _run_routed(w, di, out0["topk_idx"], out0["topk_w"])
    g0 = parity.to_np(out0)
    assert torch.equal(y0, y1)
    for key in ("counts", "offsets", "row_of", "drop_mask"):
        assert np.array_equal(g0[key], g1[key]), key
    A = int(g0["offsets"][-1])
    assert np.array_equal(g0["token_of_row"][:A], g1["token_of_row"][:A])


@pytest.mark.parametrize("name", ["cap-s", "mix-s", "toy-s", "relu-bf16-s"])
def test_replay_of_arbitrary_routing(name):
    """Random distinct experts per token, random weights and a few indices
    outside [0, E): layer and dispatch against the oracle's replay."""
    import parity
    w = synth.get(name)
    inp = synth.make_inputs(w)
    di = sdev.upload(inp)
    rng = np.random.default_rng(7)
    idx = np.stack([rng.permutation(w.E)[: w.k] for _ in range(w.N)]).astype(np.int32)
    idx[rng.random(idx.shape) < 0.05] = -1
    idx[rng.random(idx.shape) < 0.02] = w.E + 3
    gw = rng.uniform(0.05, 1.0, size=idx.shape).astype(np.float32)
    y, g = _run_routed(w, di, torch.from_numpy(idx.ravel()).cuda(),
                       torch.from_numpy(gw.ravel()).cuda())
    ors = parity.OracleSide(inp)
    ref = ors.forward(idx.astype(np.int64), forced_w=gw.astype(np.float64))
    C = O.capacity(w.f, w.N, w.k, w.E)
    d = O.dispatch(idx.astype(np.int64), w.E, C)
    assert np.array_equal(g["counts"], d["counts"])
    assert np.array_equal(g["offsets"], d["offsets"])
    assert np.array_equal(g["row_of"][: w.N * w.k].reshape(w.N, w.k), d["row_of"])
    assert np.array_equal(g["drop_mask"][: w.N * w.k].reshape(w.N, w.k), d["drop_mask"])
    yg = parity.y_to_f64(y)
    rms = float(np.sqrt(np.mean(ref["y"] ** 2)))
    err = np.abs(yg - ref["y"])
    if w.dtype == "bf16":
        m = float(err.max()) / rms
        assert m <= parity.BF16_Y_TOL, m
    else:
        m = float(np.max(err / np.maximum(np.abs(ref["y"]), rms)))
        assert m <= parity.F32_Y_TOL, m
    _say(f"[replay] {name} err {m:.3e} dropped {int(g['drop_mask'][: w.N * w.k].sum())}")


REROUTE = {
    "cap-reroute": dict(base="cap-s", f=1.0),
    "ds-reroute": dict(base="ds-s", f=1.0),
    "v41-reroute": dict(base="v41-s", f=1.25),
    "f32-reroute": dict(base="toy-s", toy_draws=False, f=1.0, zipf_offset=1.0),
    "k1-reroute": dict(base="cap-s", k=1, f=1.0),
}


@pytest.mark.parametrize("case", sorted(REROUTE))
def test_overflow_reroute(case):
    """Overflowing slots go to the token's next experts while they have room
    (routing slides, overflow table, 'Report sur E2/E3')."""
    import parity
    spec = dict(REROUTE[case])
    base = synth.get(spec.pop("base"))
    w = synth.derive(base, name=f"{base.name}-{case}", overflow="reroute", **spec)
    _say(f"[reroute] {case} {w}")
    rep, y, g, _ = parity.full_check(w)
    _say(f"[reroute] {case} {dict((k, v) for k, v in rep.items() if k != 'modality_counts')}")
    assert rep["rerouted"] > 0


def test_reroute_collapse_fills_other_experts():
    # every token prefers expert 0: its overflow spreads over the next experts
    import parity
    w = synth.derive(synth.get("cap-s"), name="collapse-reroute", N=400, f=1.0,
                     zipf_offset=0.0, overflow="reroute")
    inp = synth.make_inputs(w)
    inp.logit_bias = np.zeros(w.E, np.float32)
    inp.logit_bias[0] = 50.0
    rep, y, g, _ = parity.full_check(w, inp=inp)
    assert rep["rerouted"] > 0
    C = -(-(w.N * w.k) // w.E)
    assert np.all(np.diff(g["offsets"]) <= C)


def test_hash_router_and_replay():
    from mixture_experts_layer_16_amd import _lib as L
    import parity
    w = synth.get("cap-s")
    inp = synth.make_inputs(w)
    di = sdev.upload(inp)
    rng = np.random.default_rng(11)
    ids = rng.integers(-(1 << 62), 1 << 62, size=w.N, dtype=np.int64)
    ids[:3] = [0, 1, -1]
    p = parity.problem_of(w)
    idx = torch.full((w.N * w.k,), -7, dtype=torch.int32, device="cuda")
    gw = torch.full((w.N * w.k,), -7.0, dtype=torch.float32, device="cuda")
    L.moe_route_hash(p, torch.from_numpy(ids).cuda(), idx, gw)
    torch.cuda.synchronize()
    ridx, rg = O.hash_route(ids, w.E, w.k)
    assert np.array_equal(idx.cpu().numpy().reshape(w.N, w.k), ridx)
    assert np.all(gw.cpu().numpy() == np.float32(1.0 / w.k))
    # the layer on the hash routing (capacity applies as usual)
    y, g = _run_routed(w, di, idx, gw)
    ors = parity.OracleSide(inp)
    ref = ors.forward(ridx, forced_w=np.full(ridx.shape, float(np.float32(1.0 / w.k))))
    d = O.dispatch(ridx, w.E, O.capacity(w.f, w.N, w.k, w.E))
    assert np.array_equal(g["row_of"][: w.N * w.k].reshape(w.N, w.k), d["row_of"])
    m = float(np.max(np.abs(parity.y_to_f64(y) - ref["y"]))) / float(np.sqrt(np.mean(ref["y"] ** 2)))
    assert m <= parity.BF16_Y_TOL, m
