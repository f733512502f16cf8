"""Helpers shared by the GPU parity tests: run the library through its C ABI
and compare with the float64 oracle on the same synthetic inputs.

The protocol (tolerances are the ones the workload statement fixes):
* routing indices bit-exact on every token that is not a near-tie (a key gap
  within 1e-6 of S_t = max(|key_k|, |key_k+1|, RMS z)); order-only near-ties
  compare the chosen set; gate weights within 1e-5 absolute;
* the logits' error relative to the token's RMS logit (floored at the batch
  RMS) <= 5e-7, so that every possible flip lies inside the excluded near-tie
  set;
* dispatch (counts, per-modality counts, offsets, row map, token map, drops)
  bit-exact against the oracle fed with the GPU's indices;
* layer output: bf16 max|dy| <= 2e-2 * RMS(y); fp32 max_i |dy_i| / max(|y_i|,
  RMS(y)) <= 1e-4 (elementwise with an RMS floor).
"""
from __future__ import annotations

import numpy as np
import torch

import synth
from synth import device as sdev
from oracle import moe_oracle as O
from mixture_experts_layer_16_amd import _lib as L

Z_REL_TOL = 5e-7
W_TOL = 1e-5
BF16_Y_TOL = 2e-2
F32_Y_TOL = 1e-4
# balance statistics from the GPU's own logits: float64 sums of N terms in
# another order, each term within a few ulps -> |dP| <= 1e-11 (N <= 2^24 would
# allow ~N*eps = 2e-9 in the worst case; the sums here have N <= 2^16)
P_ABS_TOL = 1e-11
AUX_REL_TOL = 1e-12
GAMMA = 0.001


def problem_of(w: synth.Workload, **over):
    kw = dict(S=w.S, gating=w.gating, activation=w.activation, dtype=w.dtype,
              n_bias_sets=w.n_bias_sets, act_clip=w.clip, capacity_factor=w.f,
              renormalize=int(w.renormalize), overflow=w.overflow)
    kw.update(over)
    return L.problem(w.N, w.d, w.E, w.k, w.I, **kw)


def alloc_routing(w, dev="cuda"):
    N, k, E = w.N, w.k, w.E
    i32 = torch.int32
    return dict(
        topk_idx=torch.full((max(1, N * k),), -7, dtype=i32, device=dev),
        topk_w=torch.full((max(1, N * k),), -7.0, dtype=torch.float32, device=dev),
        counts=torch.full((E,), -7, dtype=i32, device=dev),
        modality_counts=(torch.full((2 * E,), -7, dtype=i32, device=dev)
                         if w.n_bias_sets == 2 else None),
        offsets=torch.full((E + 1,), -7, dtype=i32, device=dev),
        row_of=torch.full((max(1, N * k),), -7, dtype=i32, device=dev),
        token_of_row=torch.full((max(1, N * k),), -7, dtype=i32, device=dev),
        drop_mask=torch.full((max(1, N * k),), 7, dtype=torch.uint8, device=dev),
        logits=torch.full((max(1, N * E),), np.nan, dtype=torch.float64, device=dev),
        final_idx=torch.full((max(1, N * k),), -7, dtype=i32, device=dev),
        sat_count=torch.full((1,), -7, dtype=i32, device=dev),
    )


def gpu_forward(w, di, ws=None, stream=None):
    p = problem_of(w)
    out = alloc_routing(w, di.x.device)
    y = torch.full((max(1, w.N), w.d), float("nan"), dtype=torch.float32, device=di.x.device)
    if ws is None:
        ws = L.workspace(p)
    r = L.routing(**{k: v for k, v in out.items() if v is not None})
    L.moe_forward(p, L.weights(di.w_router, di.w_gate, di.w_up, di.w_down, di.ws_gate, di.ws_up,
                               di.ws_down),
                  di.x, di.logit_bias, di.sel_bias, di.modality, y, r, ws, stream=stream)
    torch.cuda.synchronize()
    return y, out


def to_np(out):
    res = {}
    for k, v in out.items():
        if v is None:
            res[k] = None
        else:
            res[k] = v.cpu().numpy()
    return res


def y_to_f64(y: torch.Tensor) -> np.ndarray:
    return y.float().cpu().numpy().astype(np.float64)


class OracleSide:
    """Float64 views of the inputs, built once per workload."""

    def __init__(self, inp: synth.Inputs):
        w = inp.w
        self.w = w
        self.inp = inp
        self.x = synth.to_f64(w, inp.x)
        self.wr = synth.to_f64(w, inp.w_router)
        self.lb = None if inp.logit_bias is None else inp.logit_bias.astype(np.float64)
        self.sb = None if inp.sel_bias is None else inp.sel_bias.astype(np.float64)
        self.mod = inp.modality
        self._route = None

    def expert(self, e):
        return tuple(None if a is None else synth.to_f64(self.w, a) for a in self.inp.expert(e))

    def shared(self, s):
        return tuple(None if a is None else synth.to_f64(self.w, a) for a in self.inp.shared(s))

    def route(self):
        if self._route is None:
            w = self.w
            self._route = O.route(self.x, self.wr, w.k, w.gating, self.lb, self.sb, self.mod,
                                  renormalize=w.renormalize)
        return self._route

    def forward(self, forced_idx, tokens=None, forced_w=None):
        w = self.w
        return O.forward(self.x, w.k, w.E, w.gating, w.activation, get_expert=self.expert,
                         n_shared=w.S, get_shared=self.shared, w_router=self.wr, clip=w.clip,
                         f=w.f, logit_bias=self.lb, sel_bias=self.sb, modality=self.mod,
                         forced_idx=forced_idx, tokens=tokens, renormalize=w.renormalize,
                         forced_w=forced_w, overflow=w.overflow if forced_w is None else "drop")


def check_route(ors: OracleSide, g: dict, report: dict) -> np.ndarray:
    """Compare routing; returns the GPU indices [N,k]."""
    w = ors.w
    N, k, E = w.N, w.k, w.E
    r = ors.route()
    gidx = g["topk_idx"][: N * k].reshape(N, k).astype(np.int64)
    gw = g["topk_w"][: N * k].reshape(N, k).astype(np.float64)
    z = g["logits"][: N * E].reshape(N, E)
    # scale: the token's RMS logit, floored at the batch RMS (the accumulation
    # error follows the size of the partial sums, which is batch-typical; with
    # E = 1 a token's own RMS is |z| and may be ~0)
    rms = np.sqrt(np.mean(r["z"] ** 2, axis=1))
    rms = np.maximum(rms, np.sqrt(np.mean(r["z"] ** 2)) if N else 0.0)
    zerr = np.max(np.abs(z - r["z"]), axis=1) / np.maximum(rms, 1e-300)
    report["logit_rel_err_max"] = float(zerr.max()) if N else 0.0
    assert report["logit_rel_err_max"] <= Z_REL_TOL, report
    bnd, order = O.near_ties(r["keys"], r["z"], k)
    report["near_tie_boundary"] = int(bnd.sum())
    report["near_tie_order"] = int((order & ~bnd).sum())
    strict = ~(bnd | order)
    mism = np.nonzero(np.any(gidx[strict] != r["idx"][strict], axis=1))[0]
    assert mism.size == 0, f"routing differs on {mism.size} tokens, e.g. {np.nonzero(strict)[0][mism[:5]]}"
    only_order = order & ~bnd
    if only_order.any():
        assert np.array_equal(np.sort(gidx[only_order], 1), np.sort(r["idx"][only_order], 1))
    # weights matched by expert (same order on strict tokens)
    okw = ~bnd
    if okw.any():
        og = r["g"][okw]
        oi = r["idx"][okw]
        gi = gidx[okw]
        gg = gw[okw]
        perm = np.argsort(gi, 1)
        operm = np.argsort(oi, 1)
        dw = np.abs(np.take_along_axis(gg, perm, 1) - np.take_along_axis(og, operm, 1))
        report["weight_abs_err_max"] = float(dw.max())
        assert report["weight_abs_err_max"] <= W_TOL, report
        if w.renormalize:
            assert float(np.max(np.abs(gw.sum(1) - 1.0))) <= 1e-6
    # every row holds k distinct experts in range
    assert gidx.min(initial=0) >= 0 and gidx.max(initial=0) < E
    assert all(len(set(row)) == k for row in gidx[: min(N, 2000)].tolist())
    return gidx


def check_dispatch(ors: OracleSide, g: dict, gidx: np.ndarray, report: dict) -> dict:
    w = ors.w
    N, k, E = w.N, w.k, w.E
    C = O.capacity(w.f, N, k, E)
    d = O.dispatch(gidx, E, C, ors.mod if w.n_bias_sets == 2 else None)
    if w.overflow == "reroute":
        # the alternates come from the oracle's keys (a near-tie among ranks
        # k+1 .. 2k would show up as a mismatch here)
        mc = d["modality_counts"]
        d = O.dispatch_reroute(gidx, O.alternates(ors.route()["keys"], k), E, C)
        d["modality_counts"] = mc
        report["rerouted"] = int(((d["final_idx"] != gidx) & (d["final_idx"] >= 0)).sum())
    final = d.get("final_idx", np.where(d["row_of"] >= 0, gidx, -1))
    assert np.array_equal(g["final_idx"][: N * k].reshape(N, k), final)
    assert np.array_equal(g["counts"], d["counts"])
    if w.n_bias_sets == 2:
        assert np.array_equal(g["modality_counts"].reshape(2, E), d["modality_counts"])
        report["modality_counts"] = d["modality_counts"].tolist()
    assert np.array_equal(g["offsets"], d["offsets"])
    A = int(d["offsets"][-1])
    assert np.array_equal(g["row_of"][: N * k].reshape(N, k), d["row_of"])
    assert np.array_equal(g["token_of_row"][:A], d["token_of_row"])
    assert np.array_equal(g["drop_mask"][: N * k].reshape(N, k), d["drop_mask"])
    # invariants
    assert int(g["counts"].sum()) == N * k
    kept = int((g["drop_mask"][: N * k] == 0).sum())
    assert kept == A and kept + int(g["drop_mask"][: N * k].sum()) == N * k
    report["kept"] = A
    report["dropped"] = N * k - A
    return d


def check_layer(ors: OracleSide, y_gpu: torch.Tensor, gidx: np.ndarray, report: dict,
                tokens=None) -> None:
    w = ors.w
    ref = ors.forward(gidx, tokens=tokens)["y"]
    yg = y_to_f64(y_gpu)
    if tokens is not None:
        yg = yg[np.asarray(tokens)]
    assert np.all(np.isfinite(yg))
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    err = np.abs(yg - ref)
    if w.dtype == "bf16":
        m = float(err.max()) / max(rms, 1e-300) if ref.size else 0.0
        report["y_err_over_rms"] = m
        assert m <= BF16_Y_TOL, report
    else:
        m = float(np.max(err / np.maximum(np.abs(ref), rms))) if ref.size else 0.0
        report["y_rel_err"] = m
        assert m <= F32_Y_TOL, report


def check_balance(ors: OracleSide, out: dict, g: dict, di, report: dict, gamma=GAMMA,
                  ws=None) -> dict:
    """moe_balance on the GPU's routing outputs against the oracle's balancing
    statistics: load bit-exact, P from the GPU's own logits within P_ABS_TOL
    (and from the oracle's logits within the logit tolerance's effect), aux
    relative AUX_REL_TOL, bias update bit-exact."""
    w = ors.w
    N, k, E = w.N, w.k, w.E
    dev = out["counts"].device
    p = problem_of(w)
    load = torch.full((E,), np.nan, dtype=torch.float64, device=dev)
    prob = torch.full((E,), np.nan, dtype=torch.float64, device=dev)
    aux = torch.full((1,), np.nan, dtype=torch.float64, device=dev)
    bias = None if di.sel_bias is None else di.sel_bias.clone()
    if ws is None:
        ws = L.workspace(p, dev)
    L.moe_balance(p, out["logits"], out["counts"], out["modality_counts"], load, prob, aux,
                  bias, gamma, ws)
    torch.cuda.synchronize()
    counts = g["counts"].astype(np.int64)
    f_ref = O.expert_load(counts, N, k)
    gl = load.cpu().numpy()
    assert np.array_equal(gl, f_ref), (gl[:8], f_ref[:8])
    z = g["logits"][: N * E].reshape(N, E)
    P_ref = O.mean_router_probs(z, w.gating)
    gp = prob.cpu().numpy()
    report["P_abs_err"] = float(np.max(np.abs(gp - P_ref))) if E else 0.0
    assert report["P_abs_err"] <= P_ABS_TOL, report
    if N:
        P_or = O.mean_router_probs(ors.route()["z"], w.gating)
        report["P_vs_oracle_logits"] = float(np.max(np.abs(gp - P_or)))
        assert report["P_vs_oracle_logits"] <= 1e-6, report
    a_ref = O.switch_aux(f_ref, gp)
    ga = float(aux.cpu().numpy()[0])
    report["aux"] = ga
    assert abs(ga - a_ref) <= AUX_REL_TOL * max(abs(a_ref), 1e-300) or (N == 0 and ga == 0.0)
    if bias is not None:
        b0 = di.sel_bias.cpu().numpy().reshape(w.n_bias_sets, E)
        nb = bias.cpu().numpy().reshape(w.n_bias_sets, E)
        if w.n_bias_sets == 1:
            ref = O.bias_update(b0[0], counts, N, k, gamma)[None, :]
        else:
            ref = O.bias_update_by_modality(b0, g["modality_counts"].reshape(2, E), k, gamma)
        assert np.array_equal(nb.view(np.uint32), ref.view(np.uint32))
        report["bias_moved"] = int((nb != b0).sum())
    return {"load": gl, "P": gp, "aux": ga, "bias": None if bias is None else bias}


def full_check(w, inp=None, di=None, tokens=None, report=None, balance=True):
    inp = inp or synth.make_inputs(w)
    di = di or sdev.upload(inp)
    report = {} if report is None else report
    y, out = gpu_forward(w, di)
    g = to_np(out)
    ors = OracleSide(inp)
    gidx = check_route(ors, g, report)
    check_dispatch(ors, g, gidx, report)
    if callable(tokens):
        # the sample may depend on the routing (e.g. the tile plan's special rows)
        tokens = tokens(g)
        report["sampled_tokens"] = len(tokens)
    check_layer(ors, y, gidx, report, tokens=tokens)
    # every fp16 intermediate of these inputs is inside fp16's range
    report["sat_count"] = int(g["sat_count"][0])
    assert report["sat_count"] == 0, report
    if balance:
        check_balance(ors, out, g, di, report)
    return report, y, g, di
