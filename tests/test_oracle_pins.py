"""Pins of the float64 oracle to facts the pages fix (printed worked examples,
closed forms, invariants, special cases), independent of the oracle's own code.

Each test names the page and section its expected values come from; the
numbers themselves live in tests/golden/*.json with their citations.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import moe_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as fh:
        return json.load(fh)


# ---------------------------------------------------------------------------
# softmax, top-k, renormalisation: printed worked examples

@pytest.mark.parametrize("ex", gold("softmax_examples.json")["examples"],
                         ids=lambda e: str(e["logits"]))
def test_softmax_printed_examples(ex):
    z = np.array([ex["logits"]])
    dec = ex["decimals"]
    p = O.softmax(z)[0]
    assert np.all(np.abs(p - np.array(ex["softmax"])) <= 0.5 * 10 ** -dec + 1e-12)
    if "exp" in ex:
        e = np.exp(z[0])
        assert np.all(np.abs(e - np.array(ex["exp"])) <= 0.5e-3 + 1e-12)
        assert abs(e.sum() - ex["exp_sum"]) <= 0.5e-3 + 1e-12
    idx = O.topk(z, 2)[0]
    assert idx.tolist() == ex["top2"]
    if "renorm" in ex:
        g = O.gate_weights(p[None, :], idx[None, :])[0]
        assert np.all(np.abs(g - np.array(ex["renorm"])) <= 0.5e-3 + 1e-12)
        # the pages divide by the sum of the *printed* (3-decimal) probabilities
        assert round(sum(round(float(v), 3) for v in p[idx]), 3) == ex["renorm_divisor"]
        assert abs(g.sum() - 1.0) < 1e-15
    if "quiz_weight_2dp" in ex:
        g = O.gate_weights(p[None, :], idx[None, :])[0]
        assert round(g[0], 2) == ex["quiz_weight_2dp"]


def test_route_through_projection_matches_printed_example():
    # x = one-hot rows, W_g = the logits as a column: z = x W_g reproduces them,
    # so the full route() path must print 0.731 / 0.269 (Основы MoE, numeric example).
    logits = np.array([2.0, 1.0, 0.5, -1.0])
    x = np.array([[1.0]])
    w_router = logits[:, None]            # [E][d] with d = 1
    r = O.route(x, w_router, 2, "softmax")
    assert r["idx"][0].tolist() == [0, 1]
    assert np.round(r["g"][0], 3).tolist() == [0.731, 0.269]


def test_k2_softmax_weight_closed_form():
    # For k = 2 the renormalised top weight equals sigmoid(z1 - z2): a closed
    # form derived from the renormalisation rule (Основы MoE, step 3).
    rng = np.random.default_rng(0)
    z = rng.normal(size=(200, 9)) * 3
    idx = O.topk(z, 2)
    g = O.gate_weights(O.softmax(z), idx)
    z1 = np.take_along_axis(z, idx, 1)
    closed = 1.0 / (1.0 + np.exp(-(z1[:, 0] - z1[:, 1])))
    assert np.max(np.abs(g[:, 0] - closed)) < 1e-14
    # sigma(0.3) and sigma(1) are the printed 0.574 and 0.731
    assert round(1 / (1 + math.exp(-0.3)), 3) == 0.574
    assert round(1 / (1 + math.exp(-1.0)), 3) == 0.731


def test_weights_sum_to_one_and_descending():
    rng = np.random.default_rng(1)
    for gating in ("softmax", "sigmoid"):
        x = rng.normal(size=(300, 12))
        w = rng.normal(size=(10, 12)) * 0.3
        r = O.route(x, w, 3, gating)
        assert np.max(np.abs(r["g"].sum(1) - 1)) < 1e-14
        ks = np.take_along_axis(r["keys"], r["idx"], 1)
        assert np.all(np.diff(ks, axis=1) <= 0)
        # each row holds k distinct experts
        assert all(len(set(row)) == 3 for row in r["idx"].tolist())


def test_tie_rule_lower_index_first():
    # Основы MoE, 'Практика': equal keys -> the lower expert index first.
    keys = np.array([[1.0, 3.0, 3.0, 2.0, 3.0],
                     [0.0, 0.0, 0.0, 0.0, 0.0]])
    assert O.topk(keys, 2).tolist() == [[1, 2], [0, 1]]
    assert O.topk(keys, 4).tolist() == [[1, 2, 4, 3], [0, 1, 2, 3]]


def test_softmax_over_chosen_equals_renormalised():
    # The fiche / lesson take softmax over the chosen logits; Основы MoE
    # renormalises the full softmax: the same in exact arithmetic.
    rng = np.random.default_rng(2)
    z = rng.normal(size=(100, 16)) * 2
    idx = O.topk(z, 4)
    a = O.softmax_over_chosen(z, idx)
    b = O.gate_weights(O.softmax(z), idx)
    assert np.max(np.abs(a - b)) < 1e-15


# ---------------------------------------------------------------------------
# selection bias and sigmoid gating: invariants

def test_sigmoid_without_bias_selects_like_softmax():
    # Both scores are increasing functions of z, so without bias they pick the
    # same experts in the same order.
    rng = np.random.default_rng(3)
    x = rng.normal(size=(500, 16))
    w = rng.normal(size=(12, 16)) * 0.4
    a = O.route(x, w, 4, "softmax")
    b = O.route(x, w, 4, "sigmoid")
    assert np.array_equal(a["idx"], b["idx"])


def test_bias_moves_selection_not_weights():
    # Le groupe d'experts, 'Étape 1': the bias decides the choice; the gate
    # weights come from the original scores.  A bias that does not change the
    # chosen set leaves the weights unchanged; a large bias forces an expert in.
    rng = np.random.default_rng(4)
    x = rng.normal(size=(200, 8))
    w = rng.normal(size=(6, 8)) * 0.5
    for gating in ("softmax", "sigmoid"):
        r0 = O.route(x, w, 2, gating)
        tiny = np.full(6, 1e-13)            # uniform shift: same order, same set
        r1 = O.route(x, w, 2, gating, sel_bias=tiny)
        assert np.array_equal(r0["idx"], r1["idx"])
        assert np.max(np.abs(r0["g"] - r1["g"])) == 0.0
        big = np.zeros(6)
        big[5] = 100.0
        r2 = O.route(x, w, 2, gating, sel_bias=big)
        assert np.all(r2["idx"][:, 0] == 5)
        s = r2["s"]
        chosen = np.take_along_axis(s, r2["idx"], 1)
        assert np.max(np.abs(r2["g"] - chosen / chosen.sum(1, keepdims=True))) < 1e-15


def test_two_equal_bias_sets_equal_one_set():
    # V4.1: each token uses its own modality's set; two identical sets must
    # route exactly like one.
    rng = np.random.default_rng(5)
    x = rng.normal(size=(300, 10))
    w = rng.normal(size=(16, 10)) * 0.3
    b = rng.uniform(-0.1, 0.1, size=16)
    mod = (rng.random(300) < 0.3).astype(np.uint8)
    one = O.route(x, w, 3, "sigmoid", sel_bias=b)
    two = O.route(x, w, 3, "sigmoid", sel_bias=np.stack([b, b]), modality=mod)
    assert np.array_equal(one["idx"], two["idx"])
    # different sets: image tokens follow set 1, text tokens set 0
    b2 = np.stack([b, -b])
    r = O.route(x, w, 3, "sigmoid", sel_bias=b2, modality=mod)
    rt = O.route(x[mod == 0], w, 3, "sigmoid", sel_bias=b)
    ri = O.route(x[mod == 1], w, 3, "sigmoid", sel_bias=-b)
    assert np.array_equal(r["idx"][mod == 0], rt["idx"])
    assert np.array_equal(r["idx"][mod == 1], ri["idx"])


# ---------------------------------------------------------------------------
# capacity and dispatch: the printed trace

def test_capacity_formula_printed_values():
    t = gold("routage_trace.json")
    assert O.capacity(t["f"], t["T"], t["k"], t["E"]) == t["C"]
    for v in t["variants"]:
        assert O.capacity(v["f"], t["T"], v["k"], t["E"]) == v["C"]
    # unlimited
    assert O.capacity(0.0, 10, 2, 4) is None
    # exact ceiling, no float rounding: 16384*2/64*1.0 = 512 exactly
    assert O.capacity(1.0, 16384, 2, 64) == 512
    # f = 0.1 is slightly above 1/10 as a binary double -> ceil goes up
    assert Fraction(0.1) > Fraction(1, 10)
    assert O.capacity(0.1, 100, 1, 1) == 11
    # a capacity-5 expert that receives 6 demands rejects exactly 1
    d = O.dispatch(np.zeros((6, 1), np.int64), 1, 5)
    assert int(d["drop_mask"].sum()) == 1 and d["drop_mask"][5, 0] == 1


def _trace_dispatch(k=2, f=1.25):
    t = gold("routage_trace.json")
    idx = np.array(t["assignments"])[:, :k]
    C = O.capacity(f, t["T"], k, t["E"])
    return t, idx, C, O.dispatch(idx, t["E"], C)


def test_trace_counts_drops_and_slot_table():
    t, idx, C, d = _trace_dispatch()
    assert d["counts"].tolist() == t["counts"]
    assert int(d["counts"].sum()) == t["T"] * t["k"]
    dropped = [[int(a), int(b)] for a, b in zip(*np.nonzero(d["drop_mask"]))]
    # t6 (0-based 5) loses its first choice, expert E1 (0-based 0)
    assert [[tok, int(idx[tok, j])] for tok, j in dropped] == t["dropped"]
    for e, toks in t["slots"].items():
        e = int(e)
        lo, hi = d["offsets"][e], d["offsets"][e + 1]
        assert d["token_of_row"][lo:hi].tolist() == toks
    used = int(d["offsets"][-1])
    assert used == t["slots_used"]
    assert t["E"] * C == t["slots_reserved"]
    util = [round(100 * (d["offsets"][e + 1] - d["offsets"][e]) / C) for e in range(t["E"])]
    assert util == t["utilisation_pct"]
    assert round(100 * (t["slots_reserved"] - used) / t["slots_reserved"]) == t["padding_pct"]
    # the row map is a bijection onto [0, A)
    rows = d["row_of"][d["row_of"] >= 0]
    assert sorted(rows.tolist()) == list(range(used))
    for (tok, j), row in np.ndenumerate(d["row_of"]):
        if row >= 0:
            assert d["token_of_row"][row] == tok


@pytest.mark.parametrize("vi", range(4))
def test_trace_variants(vi):
    t = gold("routage_trace.json")
    v = t["variants"][vi]
    _, idx, C, d = _trace_dispatch(k=v["k"], f=v["f"])
    assert C == v["C"]
    if "load" in v:
        assert d["counts"].tolist() == v["load"]
        assert int(d["drop_mask"].sum()) == v["n_dropped"]
        return
    drops = sorted(int(tok) for tok, j in zip(*np.nonzero(d["drop_mask"])) if idx[tok, j] == 0)
    assert drops == v["dropped_tokens_at_expert0"]
    assert int(d["drop_mask"].sum()) == len(v["dropped_tokens_at_expert0"])
    assert int(d["offsets"][-1]) == v["slots_used"]
    assert t["E"] * C == v["slots_reserved"]
    if "padding_pct" in v:
        assert round(100 * (v["slots_reserved"] - v["slots_used"]) / v["slots_reserved"]) == v["padding_pct"]


def test_dropped_token_keeps_unrenormalised_weight():
    # Routage trace: t6 (same logits as t1: 2.1, 1.8, 0.2, ...) loses E1 and its
    # output carries only 0.426 of the mixture, plus the shared expert.
    t = gold("routage_trace.json")
    T, E, d_model, I = 8, 4, 1, 2
    # router: x = 1 one-dimensional token; logits chosen per token through x
    # values: give every token the t1 logits (the trace assumes that for t6)
    logits = np.array([2.1, 1.8, 0.2, 0.1])
    x = np.ones((T, d_model))
    w_router = logits[:, None]
    forced = np.array(t["assignments"])
    rng = np.random.default_rng(6)
    W = {e: (rng.normal(size=(I, d_model)), rng.normal(size=(I, d_model)),
             rng.normal(size=(d_model, I))) for e in range(E)}
    SH = (rng.normal(size=(I, d_model)), rng.normal(size=(I, d_model)), rng.normal(size=(d_model, I)))
    out = O.forward(x, 2, E, "softmax", "swiglu", get_expert=lambda e: W[e], n_shared=1,
                    get_shared=lambda s: SH, w_router=w_router, f=1.25, forced_idx=forced)
    g6 = out["g"][5]
    assert round(g6[1], 3) == t["dropped_token_kept_weight"]
    assert out["row_of"][5, 0] == -1
    e2 = O.expert_ffn(x[5:6], *W[1], "swiglu")[0]
    sh = O.expert_ffn(x[5:6], *SH, "swiglu")[0]
    assert np.allclose(out["y"][5], g6[1] * e2 + sh, rtol=0, atol=1e-14)
    # and a kept token with the same choices gets the full mixture (t1)
    e1 = O.expert_ffn(x[0:1], *W[0], "swiglu")[0]
    assert np.allclose(out["y"][0], out["g"][0][0] * e1 + out["g"][0][1] * e2 + sh, atol=1e-14)


def test_dispatch_invariants_random():
    rng = np.random.default_rng(7)
    for (N, E, k, C) in [(257, 7, 3, 40), (100, 5, 5, None), (64, 16, 1, 1), (0, 4, 2, 3)]:
        idx = np.stack([rng.permutation(E)[:k] for _ in range(N)]) if N else np.zeros((0, k), np.int64)
        d = O.dispatch(idx, E, C)
        assert int(d["counts"].sum()) == N * k
        kept = np.minimum(d["counts"], C if C is not None else d["counts"].max(initial=0))
        assert d["offsets"][-1] == kept.sum()
        assert int(d["drop_mask"].sum()) + int(d["offsets"][-1]) == N * k
        rows = d["row_of"][d["row_of"] >= 0]
        assert sorted(rows.tolist()) == list(range(int(d["offsets"][-1])))
        # token-order: within one expert's slots the tokens ascend
        for e in range(E):
            seg = d["token_of_row"][d["offsets"][e]:d["offsets"][e + 1]]
            assert np.all(np.diff(seg) > 0)


def test_modality_counts():
    rng = np.random.default_rng(8)
    N, E, k = 120, 9, 3
    idx = np.stack([rng.permutation(E)[:k] for _ in range(N)])
    mod = (rng.random(N) < 0.3).astype(np.uint8)
    d = O.dispatch(idx, E, None, modality=mod)
    assert np.array_equal(d["modality_counts"].sum(0), d["counts"])
    assert int(d["modality_counts"][1].sum()) == int(mod.sum()) * k


# ---------------------------------------------------------------------------
# experts and combine: special cases that reduce to library routines

def test_silu_identities():
    a = np.linspace(-8, 8, 101)
    s = O.silu(a)
    # silu(a) - silu(-a) = a because sigmoid(a) + sigmoid(-a) = 1
    assert np.max(np.abs(s - O.silu(-a) - a)) < 1e-14
    assert O.silu(np.array([0.0]))[0] == 0.0
    assert abs(O.silu(np.array([1.0]))[0] - 1 / (1 + math.exp(-1))) < 1e-16
    assert abs(O.silu(np.array([40.0]))[0] - 40.0) < 1e-12


def test_relu_expert_positive_inputs_is_linear():
    # With non-negative x and W1 the ReLU never clips, so the expert is the
    # linear map x (W1 W2); a k-of-E mixture then equals one einsum.
    rng = np.random.default_rng(9)
    N, d, I, E, k = 40, 5, 7, 4, 2
    x = rng.random((N, d))
    W1 = rng.random((E, d, I))            # page orientation x @ W1
    W2 = rng.normal(size=(E, I, d))
    w_router = rng.normal(size=(E, d))
    out = O.forward(x, k, E, "softmax", "relu",
                    get_expert=lambda e: (None, W1[e].T, W2[e].T), w_router=w_router)
    A = np.einsum("edi,eij->edj", W1, W2)
    full = np.einsum("nd,edj->nej", x, A)                   # every expert's output
    sel = np.take_along_axis(full, out["idx"][:, :, None], 1)
    ref = np.einsum("nk,nkj->nj", out["g"], sel)
    assert np.max(np.abs(out["y"] - ref)) < 1e-12


def test_k_equals_E_is_dense_mixture():
    # Основы MoE, 'Практика': with k = N (all experts) the MoE becomes the dense
    # mixture sum_e p_e FFN_e(x) (the renormalisation divides by 1).
    rng = np.random.default_rng(10)
    N, d, I, E = 30, 6, 5, 5
    x = rng.normal(size=(N, d))
    w_router = rng.normal(size=(E, d))
    W = {e: (rng.normal(size=(I, d)), rng.normal(size=(I, d)), rng.normal(size=(d, I))) for e in range(E)}
    out = O.forward(x, E, E, "softmax", "swiglu", get_expert=lambda e: W[e], w_router=w_router)
    p = O.softmax(x @ w_router.T)
    dense = sum(p[:, e:e + 1] * O.expert_ffn(x, *W[e], "swiglu") for e in range(E))
    assert np.max(np.abs(out["y"] - dense)) < 1e-12


def test_shared_expert_added_outside_renormalisation():
    rng = np.random.default_rng(11)
    N, d, I, E, k = 25, 4, 6, 6, 2
    x = rng.normal(size=(N, d))
    w_router = rng.normal(size=(E, d))
    W = {e: (rng.normal(size=(I, d)), rng.normal(size=(I, d)), rng.normal(size=(d, I))) for e in range(E)}
    SH = (rng.normal(size=(I, d)), rng.normal(size=(I, d)), rng.normal(size=(d, I)))
    a = O.forward(x, k, E, "softmax", "swiglu", get_expert=lambda e: W[e], w_router=w_router)
    b = O.forward(x, k, E, "softmax", "swiglu", get_expert=lambda e: W[e], w_router=w_router,
                  n_shared=1, get_shared=lambda s: SH)
    assert np.max(np.abs(b["y"] - a["y"] - O.expert_ffn(x, *SH, "swiglu"))) < 1e-12
    assert np.max(np.abs(b["g"].sum(1) - 1)) < 1e-14


def test_clip_bounds_and_infinite_clip():
    rng = np.random.default_rng(12)
    d, I = 8, 16
    x = rng.normal(size=(50, d)) * 3
    wg, wu, wd = rng.normal(size=(I, d)), rng.normal(size=(I, d)), np.eye(d, I)
    plain = O.expert_ffn(x, wg, wu, wd, "swiglu", 0.0)
    assert np.array_equal(plain, O.expert_ffn(x, wg, wu, wd, "swiglu", float("inf")))
    # W_down = [I_d | 0] exposes h's first d units directly
    clipped = O.expert_ffn(x, wg, wu, wd, "swiglu", 2.0)
    assert np.max(np.abs(clipped)) <= 2.0
    h = O.silu(x @ wg.T) * (x @ wu.T)
    assert np.any(np.abs(h[:, :d]) > 2.0)
    assert np.array_equal(clipped, np.clip(h[:, :d], -2, 2))


def test_near_tie_detection():
    z = np.array([[1.0, 1.0 + 5e-7, 0.2, -3.0],
                  [1.0, 0.5, 0.2, -3.0],
                  [2.0, 1.0, 1.0 + 1e-9, -3.0]])
    bnd, order = O.near_ties(z, z, 2)
    assert bnd.tolist() == [False, False, True]
    assert order.tolist() == [True, False, False]


# ---------------------------------------------------------------------------
# parameter counts: closed forms against the printed numbers

def test_param_counts_toy():
    p = gold("param_counts.json")["toy"]
    tot, act, _ = O.layer_params(p["d"], p["I"], p["E"], p["k"], p["S"], p["activation"])
    assert (tot, act) == (p["expert_total"], p["expert_active"])


def test_param_counts_dsv3():
    p = gold("param_counts.json")["dsv3"]
    dim, H = p["dim"], p["H"]
    attn = (dim * p["q_lora"] + p["q_lora"] + p["q_lora"] * H * (p["nope"] + p["rope_d"])
            + dim * (p["kv_lora"] + p["rope_d"]) + p["kv_lora"]
            + p["kv_lora"] * H * (p["nope"] + p["v_d"]) + H * p["v_d"] * dim + 2 * dim)
    expert = O.expert_params(dim, p["moe_inter"])
    moe_layers = p["layers"] - p["dense_layers"]
    tot, act, router = O.layer_params(dim, p["moe_inter"], p["n_routed"], p["k"], p["n_shared"])
    rest = p["layers"] * attn + p["dense_layers"] * 3 * dim * p["inter"] + 2 * p["vocab"] * dim
    total = rest + moe_layers * (tot + router)
    active = rest + moe_layers * (act + router)
    assert round(attn / 1e6) == p["attn_per_layer_M"]
    assert round(expert / 1e6) == p["expert_M"]
    assert round(total / 1e9) == p["total_B"]
    assert round(active / 1e9, 1) == p["active_B"]
    assert round(100 * active / total, 1) == p["active_pct"]
    assert total == 671_026_397_184 and active == 37_552_275_456


def test_param_counts_v41():
    p = gold("param_counts.json")["v41"]
    per = O.expert_params(p["d"], p["I"])
    assert per == 35_389_440
    tot, _, _ = O.layer_params(p["d"], p["I"], p["E"], p["k"], p["S"])
    moe_total = tot * p["moe_layers"]
    assert round(100 * moe_total / (p["announced_total_G"] * 1e9), 1) == p["moe_share_pct"]
    act = (p["k"] + p["S"]) * per * p["moe_layers"]
    assert round((act / 1e9 + p["attention_active_G"] + p["head_active_G"]), 1) == p["active_total_G"]
    assert p["k"] + p["S"] == p["experts_per_token"]
    assert (p["E"] + p["S"]) // (p["k"] + p["S"]) == p["ratio"]
    assert round(100 * (p["k"] + p["S"]) / (p["E"] + p["S"]), 1) == p["active_moe_pct"]


def test_param_counts_trace_and_sparsity():
    g = gold("param_counts.json")
    t = g["trace"]
    total = (t["n_routed"] + t["n_shared"]) * t["expert_G"]
    active = (t["k"] + t["n_shared"]) * t["expert_G"]
    assert round(total) == t["total_G"] and round(active, 1) == t["active_G"]
    assert math.floor(total / active) == t["ratio_approx"]
    s = g["sparsity"]
    assert round(100 * s["active_B"] / s["total_B"], 1) == s["pct_1dp"]
    c = g["combinations"]
    n = math.comb(c["E"], c["k"])
    assert n == 409_663_695_276_000 and round(n, -14) == c["approx"]


def test_switch_top1_weight_is_the_probability():
    # Switch Transformer: k = 1 and the weight is p_i itself, not renormalised
    # (Основы MoE, paragraph on model variants).  On the printed logits the
    # top-1 expert is 0 with p = 0.609; renormalising would give exactly 1.
    logits = np.array([2.0, 1.0, 0.5, -1.0])
    x = np.array([[1.0]])
    w_router = logits[:, None]
    raw = O.route(x, w_router, 1, "softmax", renormalize=False)
    ren = O.route(x, w_router, 1, "softmax")
    assert raw["idx"][0].tolist() == [0] and round(raw["g"][0, 0], 3) == 0.609
    assert ren["g"][0, 0] == 1.0
    # raw weights of any k are the scores themselves: with k = E they sum to 1
    # for softmax, and the sigmoid ones are the sigmoid scores
    allk = O.route(x, w_router, 4, "softmax", renormalize=False)
    assert abs(allk["g"].sum() - 1.0) < 1e-15
    sig = O.route(x, w_router, 2, "sigmoid", renormalize=False)
    assert np.allclose(sig["g"][0], 1 / (1 + np.exp(-logits[[0, 1]])), rtol=0, atol=1e-15)


def test_replay_with_given_weights_and_invalid_indices():
    # forward(forced_idx, forced_w) uses the given weights as they are; an
    # index outside [0, E) goes to no expert and is marked dropped
    rng = np.random.default_rng(3)
    N, d, E, k, I = 6, 4, 5, 2, 3
    x = rng.normal(size=(N, d))
    W = {e: (rng.normal(size=(I, d)), rng.normal(size=(I, d)), rng.normal(size=(d, I)))
         for e in range(E)}
    idx = np.array([[0, 1], [2, -1], [4, 3], [1, 7], [3, 2], [0, 4]])
    gw = rng.uniform(0.1, 1.0, size=(N, k))
    out = O.forward(x, k, E, "softmax", "swiglu", get_expert=lambda e: W[e],
                    forced_idx=idx, forced_w=gw)
    assert out["drop_mask"].tolist() == [[0, 0], [0, 1], [0, 0], [0, 1], [0, 0], [0, 0]]
    assert out["counts"].tolist() == [2, 2, 2, 2, 2]
    for t in range(N):
        ref = np.zeros(d)
        for j in range(k):
            e = idx[t, j]
            if 0 <= e < E:
                ref += gw[t, j] * O.expert_ffn(x[t:t + 1], *W[e], "swiglu")[0]
        assert np.max(np.abs(out["y"][t] - ref)) < 1e-12


def test_reroute_policy_on_the_printed_trace():
    # 'Report sur E2/E3': t6, over capacity at E1 (C = 5), is processed by its
    # third-best expert instead of being dropped
    t = gold("routage_trace.json")
    rr = t["reroute"]
    idx = np.array(t["assignments"])
    E, k = t["E"], t["k"]
    C = O.capacity(t["f"], t["T"], k, E)
    alt = np.full(idx.shape, -1)
    alt[rr["token"]] = O.alternates(np.array([rr["t6_logits"]]), k)[0]
    assert alt[rr["token"], 0] == rr["third_best_expert"]
    out = O.dispatch_reroute(idx, alt, E, C)
    assert out["drop_mask"].sum() == 0
    assert out["final_idx"][rr["token"], rr["slot"]] == rr["third_best_expert"]
    # the first-round placement is the drop dispatch's, the rerouted row comes
    # after expert 2's own rows
    d = O.dispatch(idx, E, C)
    assert out["counts"].tolist() == t["counts"]
    e2 = rr["third_best_expert"]
    kept = np.diff(out["offsets"])
    assert kept.tolist() == [5, 4, 4, 3]
    assert out["row_of"][rr["token"], rr["slot"]] == out["offsets"][e2] + 3
    # slots that were kept keep their order within each expert
    for e in range(E):
        a = out["token_of_row"][out["offsets"][e]: out["offsets"][e] + np.diff(d["offsets"])[e]]
        b = d["token_of_row"][d["offsets"][e]: d["offsets"][e + 1]]
        assert a.tolist() == b.tolist()


def test_reroute_respects_capacity_and_token_order():
    # brute-force walk over a random case: every expert holds at most C rows,
    # rerouted slots take the alternates in slot order, earlier tokens first
    rng = np.random.default_rng(5)
    N, E, k = 40, 6, 2
    keys = rng.normal(size=(N, E))
    keys[:, 0] += 2.0                      # expert 0 overloaded
    idx = O.topk(keys, k)
    alt = O.alternates(keys, k)
    C = O.capacity(1.0, N, k, E)
    out = O.dispatch_reroute(idx, alt, E, C)
    assert np.all(np.diff(out["offsets"]) <= C)
    used = {}
    first = O.dispatch(idx, E, C)
    room = {e: C - int(np.diff(first["offsets"])[e]) for e in range(E)}
    for t in range(N):
        q = 0
        for j in range(k):
            if first["drop_mask"][t, j]:
                c = alt[t, q]
                q += 1
                if used.get(c, 0) < room[c]:
                    used[c] = used.get(c, 0) + 1
                    assert out["final_idx"][t, j] == c
                else:
                    assert out["final_idx"][t, j] == -1 and out["drop_mask"][t, j] == 1
            else:
                assert out["final_idx"][t, j] == idx[t, j]
    # the alternates are the next keys in order
    order = np.argsort(-keys, axis=1, kind="stable")
    assert np.array_equal(alt, order[:, k:2 * k])
    assert sum(used.values()) > 0


def test_hash_router_properties():
    # the mixer is a bijection of 64-bit words: every step is invertible (odd
    # multipliers, xor with a right shift), checked by undoing the steps
    def unmix(z):
        M = (1 << 64) - 1
        def unxorshift(y, s):
            x = y
            for _ in range(64 // s + 1):
                x = y ^ (x >> s)
            return x & M
        z = unxorshift(z, 31)
        z = (z * pow(0x94D049BB133111EB, -1, 1 << 64)) & M
        z = unxorshift(z, 27)
        z = (z * pow(0xBF58476D1CE4E5B9, -1, 1 << 64)) & M
        z = unxorshift(z, 30)
        return (z - 0x9E3779B97F4A7C15) & M
    ids = np.arange(-50, 5000, 37)
    E, k = 64, 4
    idx, g = O.hash_route(ids, E, k)
    assert np.all(g == 0.25)
    assert all(len(set(r)) == k for r in idx.tolist())
    assert np.all(idx[:, 1:] == (idx[:, :1] + np.arange(1, k)) % E)
    # loads of many ids stay near uniform (binomial bound, 6 sigma)
    big, _ = O.hash_route(np.arange(200000), E, 1)
    c = np.bincount(big.ravel(), minlength=E)
    p = 1 / E
    assert np.all(np.abs(c - 200000 * p) < 6 * np.sqrt(200000 * p * (1 - p)))
    # invertibility of the mixer, through the oracle's own expert choice
    M = (1 << 64) - 1
    for v in (0, 1, 12345, (1 << 63) - 1):
        z = (v + 0x9E3779B97F4A7C15) & M
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M
        z ^= z >> 31
        assert unmix(z) == v
        assert O.hash_route([v], E, 1)[0][0, 0] == z % E


def test_hash_router_published_outputs():
    """The mixer against the published outputs of Vigna's splitmix64 generator
    (tests/golden/splitmix64.json): from the state 0 the generator's j-th output
    mixes the state j * increment, so the oracle's hash of the token id
    (j - 1) * increment (as a signed 64-bit id) must be that output modulo E.
    Several moduli (one near 2^63) check nearly every bit of the word."""
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "splitmix64.json")))
    inc = int(g["increment"], 16)
    M = (1 << 64) - 1
    for j, out in enumerate(g["outputs"]):
        state = (int(g["state0"]) + j * inc) & M
        tid = state - (1 << 64) if state >= (1 << 63) else state   # as int64
        want = int(out, 16)
        for E in (384, 1 << 30, (1 << 63) - 25):
            idx, _ = O.hash_route(np.array([tid], np.int64), E, 1)
            assert int(idx[0, 0]) == want % E, (j, E)
