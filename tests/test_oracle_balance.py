"""Pins of the load-balancing statistics and the aux-loss-free bias update."""
import json
import os

import numpy as np

from oracle import moe_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_aux_printed_example():
    g = json.load(open(os.path.join(GOLD, "aux_example.json")))
    v = O.switch_aux(np.array(g["load"]), np.array(g["P"]))
    assert round(v, 2) == g["value"]


def test_aux_uniform_is_one_and_collapse_tends_to_n():
    for E in (4, 8, 64):
        u = np.full(E, 1.0 / E)
        assert abs(O.switch_aux(u, u) - 1.0) < 1e-14
        f = np.zeros(E)
        f[0] = 1.0
        for eps in (1e-1, 1e-3, 1e-6):
            P = np.full(E, eps / (E - 1))
            P[0] = 1 - eps
            assert abs(O.switch_aux(f, P) - E * (1 - eps)) < 1e-12


def test_expert_load_and_probs_from_routing():
    rng = np.random.default_rng(0)
    N, E, k = 500, 8, 2
    z = rng.normal(size=(N, E))
    idx = O.topk(z, k)
    counts = np.bincount(idx.ravel(), minlength=E)
    f = O.expert_load(counts, N, k)
    assert abs(f.sum() - 1) < 1e-15
    P = O.mean_router_probs(z, "softmax")
    assert abs(P.sum() - 1) < 1e-12
    # P is the batch mean of the softmax: check against a per-token loop
    ref = np.zeros(E)
    for t in range(N):
        e = np.exp(z[t] - z[t].max())
        ref += e / e.sum()
    assert np.max(np.abs(P - ref / N)) < 1e-14
    Ps = O.mean_router_probs(z, "sigmoid")
    assert abs(Ps.sum() - 1) < 1e-12


def _sigmoid_pins_hold(mean_probs) -> bool:
    """The sigmoid reading of P (each token's sigmoid scores normalised over the
    experts, then the batch mean) on logits whose values are exact fractions:
    sigmoid(0) = 1/2 and sigmoid(ln 3) = 3/4."""
    # two experts with opposite logits: sigmoid(a) + sigmoid(-a) = 1, so P_0 is
    # the batch mean of sigmoid(a) -- softmax would give sigmoid(2a) instead
    a = np.array([0.0, np.log(3.0), -np.log(3.0)])
    P = mean_probs(np.stack([a, -a], 1), "sigmoid")
    ok = np.max(np.abs(P - [(0.5 + 0.75 + 0.25) / 3, (0.5 + 0.25 + 0.75) / 3])) < 1e-15
    # per-token denominators differ (3/2 and 2): P = [17/48, 17/48, 7/24]; a
    # normalisation over the whole batch would give P_2 = 2/7 instead
    z = np.array([[0.0, 0.0, 0.0], [np.log(3.0), np.log(3.0), 0.0]])
    P = mean_probs(z, "sigmoid")
    return bool(ok and np.max(np.abs(P - [17 / 48, 17 / 48, 7 / 24])) < 1e-15)


def test_sigmoid_mean_probs_closed_forms():
    assert _sigmoid_pins_hold(O.mean_router_probs)


def test_sigmoid_mean_probs_misreadings_are_caught():
    # planted mistakes, on the CPU: a softmax for sigmoid gating, and the sigmoid
    # scores normalised over the whole batch instead of per token
    def softmax_reading(z, gating):
        return O.softmax(np.asarray(z, np.float64)).mean(axis=0)

    def batch_reading(z, gating):
        s = O.sigmoid(np.asarray(z, np.float64))
        return s.sum(axis=0) / s.sum()
    assert not _sigmoid_pins_hold(softmax_reading)
    assert not _sigmoid_pins_hold(batch_reading)


def test_bias_update_sign_rule():
    # target = N k / E = 4 here: overloaded -> -gamma, underloaded -> +gamma,
    # exactly on target -> unchanged
    b = np.array([0.5, -0.25, 0.0, 0.125], np.float32)
    counts = np.array([6, 4, 3, 3])
    nb = O.bias_update(b, counts, 8, 2, gamma=0.001)
    assert nb.dtype == np.float32
    assert nb[0] == np.float32(0.5) - np.float32(0.001)
    assert nb[1] == b[1]
    assert nb[2] == np.float32(0.0) + np.float32(0.001)
    assert nb[3] == np.float32(0.125) + np.float32(0.001)
    # equal loads leave every bias unchanged
    assert np.array_equal(O.bias_update(b, np.array([4, 4, 4, 4]), 8, 2), b)


def test_bias_update_per_modality_uses_its_own_target():
    b2 = np.zeros((2, 3), np.float32)
    mc = np.array([[4, 1, 1], [0, 3, 3]])        # text: 3 tokens, image: 3 tokens (k = 2)
    nb = O.bias_update_by_modality(b2, mc, 2, gamma=0.01)
    # text target 2: [+4 over, under, under]; image target 2: [under, over, over]
    assert np.array_equal(np.sign(nb[0]), [-1, 1, 1])
    assert np.array_equal(np.sign(nb[1]), [1, -1, -1])


def test_bias_balancing_converges_toward_uniform():
    # the lesson's step 2: with the update applied after every step, a skewed
    # router's loads move toward uniform over iterations
    rng = np.random.default_rng(1)
    N, d, E, k = 2000, 16, 8, 2
    x = rng.normal(size=(N, d))
    w = rng.normal(size=(E, d)) * 0.3
    w[0] += 0.6                              # expert 0 is favoured
    off = np.zeros(E)
    off[0] = 1.5
    b = np.zeros(E, np.float32)

    def imbalance(bias):
        r = O.route(x, w, k, "softmax", logit_bias=off, sel_bias=bias)
        c = np.bincount(r["idx"].ravel(), minlength=E)
        return c, c.max() / (N * k / E)

    c0, start = imbalance(b)
    for _ in range(300):
        c, _ = imbalance(b)
        b = O.bias_update(b, c, N, k, gamma=0.01)
    _, end = imbalance(b)
    assert start > 1.5 and end < start * 0.7
