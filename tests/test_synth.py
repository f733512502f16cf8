"""The seeded input generators: determinism, shapes and the stated recipe."""
import numpy as np

import synth


def test_bf16_round_to_nearest_even():
    f = np.array([1.0, 1.00390625, 1.01171875, -2.5, 3.0e-3], np.float32)
    bits = synth.f32_to_bf16_bits(f)
    back = synth.bf16_bits_to_f32(bits)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa (1.0) wins;
    # 1 + 3*2^-8 ties between 1+2^-7 and 1+2^-6: even is 1 + 2^-6
    assert back.tolist()[:4] == [1.0, 1.0, 1.015625, -2.5]
    assert abs(back[4] - 3.0e-3) <= 3.0e-3 * 2 ** -8


def test_deterministic_and_per_expert():
    w = synth.get("cap-s")
    a = synth.make_inputs(w)
    b = synth.make_inputs(w)
    assert np.array_equal(a.x, b.x) and np.array_equal(a.w_router, b.w_router)
    ea, eb = a.expert(3), b.expert(3)
    assert all(np.array_equal(u, v) for u, v in zip(ea, eb))
    assert not np.array_equal(a.expert(3)[0], a.expert(4)[0])
    assert a.x.dtype == np.uint16 and a.x.shape == (w.N, w.d)
    wg, wu, wd = ea
    assert wg.shape == (w.I, w.d) and wu.shape == (w.I, w.d) and wd.shape == (w.d, w.I)
    xs = synth.to_f64(w, a.x)
    assert abs(xs.std() - 1.0) < 0.05
    assert abs(synth.to_f64(w, wg).std() - 0.02) < 0.002


def test_modality_layout():
    w = synth.get("v41")
    m = synth.modality_flags(w)
    assert m.shape == (16384,) and m.dtype == np.uint8
    assert int(m.sum()) == 8 * 614
    # one contiguous image block per 2048-token segment
    for s in range(8):
        seg = m[s * 2048:(s + 1) * 2048]
        edges = np.flatnonzero(np.diff(np.concatenate([[0], seg, [0]])))
        assert len(edges) == 2 and edges[1] - edges[0] == 614


def test_decode_uses_separate_token_stream_same_weights():
    p, d = synth.get("mixd-s"), synth.get("mix-s")
    ip, idd = synth.make_inputs(p), synth.make_inputs(d)
    assert np.array_equal(ip.w_router, idd.w_router)
    assert not np.array_equal(ip.x[:5], idd.x[:5])


def test_toy_draw_order():
    # default_rng(42) draws W1, W2, router, tokens in that order
    w = synth.get("toy")
    inp = synth.make_inputs(w)
    rng = np.random.default_rng(42)
    W1 = rng.normal(0, 0.1, (8, 64, 256))
    rng.normal(0, 0.1, (8, 256, 64))
    R = rng.normal(0, 0.1, (64, 8))
    X = rng.normal(0, 1, (1000, 64))
    assert np.array_equal(inp.x, X.astype(np.float32))
    assert np.array_equal(inp.w_router, R.T.astype(np.float32))
    assert np.array_equal(inp.expert(2)[1], W1[2].T.astype(np.float32))


def test_zipf_offset():
    off = synth.logit_offset(synth.get("cap"))
    assert off.dtype == np.float32 and off.shape == (64,)
    assert off[0] == 1.0 and np.all(np.diff(off) < 0)
