"""GPU parity at the full workload sizes, in the configuration bench.py times.

Routing (indices, weights, logits) and dispatch (counts, per-modality counts,
offsets, row and token maps, drops) are compared for every token; the layer
output is compared on a sample of tokens spread over the batch, which the
float64 oracle evaluates one by one (routing and capacity are still decided
over the whole batch)."""
import numpy as np
import pytest

import synth
from synth import device as sdev

pytestmark = pytest.mark.gpu

FULL = ["cap", "mix-D", "ds-D", "mix-P", "ds-P", "v41"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_parity(name):
    import parity
    w = synth.get(name)
    print(f"[full] {name}: generating inputs", flush=True)
    inp = synth.make_inputs(w, materialize=True)
    di = sdev.upload(inp)
    n_sample = min(w.N, 48)
    tokens = np.unique(np.linspace(0, w.N - 1, n_sample).astype(np.int64))
    print(f"[full] {name}: running the layer and the oracle on {len(tokens)} sampled tokens",
          flush=True)
    rep, y, g, _ = parity.full_check(w, inp=inp, di=di, tokens=tokens)
    print(f"[full] {name}: {dict((k, v) for k, v in rep.items() if k != 'modality_counts')}",
          flush=True)
    if w.n_bias_sets == 2:
        mc = np.array(rep["modality_counts"])
        assert mc.shape == (2, w.E)
        assert int(mc[1].sum()) == int(inp.modality.sum()) * w.k
    if w.f > 0:
        assert rep["dropped"] > 0          # the capacity workload really drops
    del di
