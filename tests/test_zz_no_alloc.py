"""The allocation-free entry point (moe_forward_noalloc) against moe_forward
with a caller workspace: the same kernels on the same inputs, so every output
-- y and each routing array -- must be identical, bit for bit.  Two calls in a
row on the same GPU scratch, the second with a smaller batch (the scratch
keeps the first call's contents), then the first again."""
import numpy as np
import pytest
import torch

import synth
from synth import device as sdev

pytestmark = pytest.mark.gpu


def _run(w, di, noalloc):
    import parity
    from mixture_experts_layer_16_amd import _lib as L
    p = parity.problem_of(w)
    out = parity.alloc_routing(w, di.x.device)
    y = torch.full((max(1, w.N), w.d), float("nan"), dtype=torch.float32, device=di.x.device)
    r = L.routing(**{k: v for k, v in out.items() if v is not None})
    wts = L.weights(di.w_router, di.w_gate, di.w_up, di.w_down, di.ws_gate, di.ws_up, di.ws_down)
    if noalloc:
        L.moe_forward_noalloc(p, wts, di.x, di.logit_bias, di.sel_bias, di.modality, y, r)
    else:
        L.moe_forward(p, wts, di.x, di.logit_bias, di.sel_bias, di.modality, y, r,
                      L.workspace(p))
    torch.cuda.synchronize()
    return y.cpu().numpy(), parity.to_np(out)


def _same(a, b, w):
    ya, ra = a
    yb, rb = b
    assert np.array_equal(ya.view(np.uint32), yb.view(np.uint32))
    for k in ra:
        if ra[k] is None:
            continue
        n = {"logits": w.N * w.E, "counts": w.E, "offsets": w.E + 1,
             "modality_counts": 2 * w.E, "sat_count": 1}.get(k, w.N * w.k)
        assert np.array_equal(ra[k].reshape(-1)[:n].view(np.uint8),
                              rb[k].reshape(-1)[:n].view(np.uint8)), k


@pytest.mark.parametrize("base", ["v41-s", "mixd-s", "cap-s"])
def test_noalloc_equals_forward_two_calls(base):
    from mixture_experts_layer_16_amd import _lib as L
    import parity
    w1 = synth.get(base)
    w2 = synth.derive(w1, name=w1.name + "-small", N=max(1, w1.N // 7))
    assert L.moe_workspace_size(parity.problem_of(w1)) <= L.NOALLOC_SCRATCH_BYTES
    d1 = sdev.upload(synth.make_inputs(w1))
    d2 = sdev.upload(synth.make_inputs(w2))
    print(f"[noalloc] {base}: N={w1.N} then N={w2.N}", flush=True)
    first = _run(w1, d1, True)
    second = _run(w2, d2, True)
    _same(first, _run(w1, d1, False), w1)
    _same(second, _run(w2, d2, False), w2)
    _same(_run(w1, d1, True), first, w1)


def test_noalloc_rejects_problems_beyond_its_scratch():
    from mixture_experts_layer_16_amd import _lib as L
    import parity
    w = synth.derive(synth.get("v41"), name="v41-2048", N=2048)
    p = parity.problem_of(w)
    assert L.moe_workspace_size(p) > L.NOALLOC_SCRATCH_BYTES
    t = torch.zeros(8, dtype=torch.float32, device="cuda")
    wts = L.weights(t, t, t, t, t, t, t)
    st = L.moe_forward_noalloc(p, wts, t, None, t, torch.zeros(8, dtype=torch.uint8,
                                                              device="cuda"), t, raw=True)
    assert st == -6 and "64 MiB" in L.moe_status_string(st)
