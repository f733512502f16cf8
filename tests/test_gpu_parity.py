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


def test_split_tile_plan_all_tokens():
    """Every token of a layer whose per-expert row counts take every branch of
    the prefill grouped GEMM's tile plan (more than 128 groups averaging more
    than 128 rows: 256-row tiles, the remainders past a group's last full tile
    -- at most 128 rows and more than 128 --, groups smaller than one tile and
    an empty group) against the oracle: the shape class of the DeepSeek- and
    V4.1-shaped prefill layers, small enough for the oracle."""
    import parity
    w = synth.get("ds-split-s")
    G = w.E + w.S
    assert w.N > 64 and G >= 128 and (w.N * w.k + w.N * w.S) // G >= 128
    rep, y, g, _ = parity.full_check(w)
    m = np.diff(g["offsets"].astype(np.int64))
    rem = m % 256
    classes = {"empty": int((m == 0).sum()), "two_or_more_full_tiles": int((m >= 512).sum()),
               "rem_le_128": int(((m > 256) & (rem > 0) & (rem <= 128)).sum()),
               "rem_gt_128": int(((m > 256) & (rem > 128)).sum()),
               "below_128": int(((m > 0) & (m <= 128)).sum()),
               "between_128_256": int(((m > 128) & (m < 256)).sum())}
    _say(f"[parity] ds-split-s row classes {classes} {rep}")
    assert all(v > 0 for v in classes.values()), classes


def test_clamped_bf16_forward_all_tokens():
    """The bf16 forward with the SwiGLU clamp active on a large share of the
    hidden elements (clip 0.06 on the V4.1-shaped small layer), every token
    against the oracle."""
    import parity
    from oracle import moe_oracle as O
    w = synth.get("v41-clip-s")
    inp = synth.make_inputs(w)
    # share of the shared expert's hidden elements the clamp changes
    x = synth.to_f64(w, inp.x)
    wg, wu, _ = (synth.to_f64(w, a) for a in inp.shared(0))
    frac = float(np.mean(np.abs(O.silu(x @ wg.T) * (x @ wu.T)) > w.clip))
    assert frac > 0.1, frac
    rep, *_ = parity.full_check(w, inp=inp)
    _say(f"[parity] v41-clip-s clamped share {frac:.3f} {rep}")


def _scaled_x_inputs(w, s):
    """The workload's inputs with x multiplied by 2^s (exact in bf16), and the
    oracle's largest |h| and |expert output row| over every routed and shared
    expert on all tokens."""
    from oracle import moe_oracle as O
    inp = synth.make_inputs(w)
    inp.x = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(inp.x) * np.float32(2.0 ** s))
    x = synth.to_f64(w, inp.x)
    hmax = ymax = 0.0
    for arrs in [inp.expert(e) for e in range(w.E)] + [inp.shared(j) for j in range(w.S)]:
        wg, wu, wd = (synth.to_f64(w, a) for a in arrs)
        h = O.silu(x @ wg.T) * (x @ wu.T)
        hmax = max(hmax, float(np.abs(h).max()))
        ymax = max(ymax, float(np.abs(h @ wd.T).max()))
    return inp, hmax, ymax


def test_fp16_range_large_but_in_range():
    """x scaled by 2^7: hidden values up to about 2e4, still inside fp16's
    range -- the layer matches the oracle and reports no saturation."""
    import parity
    w = synth.derive(synth.get("mix-s"), name="mix-s-x128")
    inp, hmax, ymax = _scaled_x_inputs(w, 7)
    assert 4000 < hmax < 65504 / 1.5 and ymax < 65504 / 1.5, (hmax, ymax)
    rep, *_ = parity.full_check(w, inp=inp, balance=False)
    _say(f"[range] in range: max|h| {hmax:.0f} max|row| {ymax:.0f} {rep}")


def test_fp16_range_overflow_is_reported():
    """x scaled by 2^8: some |h| exceed 65504, so the fp16 intermediates
    saturate; the forward must say so through routing_out->sat_count, with at
    least as many saturated values as the oracle's hidden values beyond the
    range (the expert rows computed from them may add more)."""
    import parity
    from oracle import moe_oracle as O
    w = synth.derive(synth.get("mix-s"), name="mix-s-x256")
    inp, hmax, ymax = _scaled_x_inputs(w, 8)
    assert hmax > 65504 * 1.01, hmax
    di = sdev.upload(inp)
    y, out = parity.gpu_forward(w, di)
    g = parity.to_np(out)
    sat = int(g["sat_count"][0])
    # the oracle's hidden values beyond the range, on the GPU's routing
    x = synth.to_f64(w, inp.x)
    idx = g["topk_idx"].reshape(w.N, w.k)
    n_lo = n_hi = 0
    for e in range(w.E):
        rows = np.nonzero((idx == e).any(axis=1))[0]
        wg, wu, _ = (synth.to_f64(w, a) for a in inp.expert(e))
        h = np.abs(O.silu(x[rows] @ wg.T) * (x[rows] @ wu.T))
        n_lo += int((h > 65504 * (1 + 1e-4)).sum())
        n_hi += int((h > 65504 * (1 - 1e-4)).sum())
    for j in range(w.S):
        wg, wu, _ = (synth.to_f64(w, a) for a in inp.shared(j))
        h = np.abs(O.silu(x @ wg.T) * (x @ wu.T))
        n_lo += int((h > 65504 * (1 + 1e-4)).sum())
        n_hi += int((h > 65504 * (1 - 1e-4)).sum())
    rows_total = (w.N * w.k + w.N * w.S)
    _say(f"[range] overflow: max|h| {hmax:.0f}, GPU count {sat}, oracle h beyond {n_lo}")
    assert n_lo > 0
    assert n_lo <= sat <= n_hi + rows_total * w.d


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
    # batches of at most 64 tokens route and dispatch in one launch
    "small-batch-two-bias-sets": dict(base="v41-s", N=40),
    "small-batch-drops": dict(base="cap-s", N=48, f=0.5),
    "small-batch-64": dict(base="ds-s", N=64),
    "small-batch-raw-weights": dict(base="mixd-s", N=30, renormalize=False),
    # short reductions on the direct-to-LDS tiles (groups average >= 128 rows):
    # one k-slice in each pass (gate/up K = d = 64; down K = I = 40, ragged, with
    # 40 of a tile's 128 h columns), two slices (d = 128; I = 96, ragged), and
    # one slice on the split plan's 128-row remainder tiles
    "short-k-one-slice": dict(base="mix-s", d=64, I=40),
    "short-k-two-slices": dict(base="mix-s", d=128, I=96),
    "short-k-split-plan": dict(base="ds-split-s", d=64, I=40),
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
