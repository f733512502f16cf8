"""GPU parity at the full workload sizes, in the configuration bench.py times.

Routing (indices, weights, logits) and dispatch (counts, per-modality counts,
offsets, row and token maps, drops) are compared for every token; the layer
output is compared on a sample of tokens, half spread over the batch and half
on the rows of each expert's last partial GEMM tile (the remainder plan's tiles
on the many-expert layers), which the float64 oracle evaluates one by one
(routing and capacity are still decided over the whole batch)."""
import numpy as np
import pytest

import synth
from synth import device as sdev

pytestmark = pytest.mark.gpu

FULL = ["cap", "mix-D", "ds-D", "mix-P", "ds-P", "v41"]
BM = 256   # rows per tile of the prefill grouped GEMMs


def sample_tokens(w, n=96):
    """Token sample for the output check, chosen from the GPU's routing: half
    spread evenly over the batch, half on the rows the grouped GEMMs' tile plan
    treats apart -- the last partial tile of each expert (the remainder plan's
    128-row tiles on the many-expert layers, a partly filled 256-row tile
    otherwise), experts with fewer rows than one tile, and the last row of the
    busiest expert."""
    def pick(g):
        N, k, E = w.N, w.k, w.E
        if N <= n:
            return np.arange(N, dtype=np.int64)
        spread = np.linspace(0, N - 1, n // 2).astype(np.int64)
        off = g["offsets"][: E + 1].astype(np.int64)
        tor = g["token_of_row"][: N * k].astype(np.int64)
        cnt = np.diff(off)
        rows = []
        for e in np.argsort(-cnt, kind="stable"):
            c = int(cnt[e])
            if c % BM:                                  # a partial last tile
                rows += [off[e] + (c // BM) * BM, off[e] + c - 1]
        rows.append(off[int(np.argmax(cnt))] + int(cnt.max()) - 1)
        rows = np.asarray(rows, np.int64)
        step = max(1, len(rows) // (n // 2))
        special = tor[rows[::step][: n // 2]]
        return np.unique(np.concatenate([spread, special[special >= 0]]))
    return pick


@pytest.mark.parametrize("name", FULL)
def test_full_size_parity(name):
    import parity
    w = synth.get(name)
    print(f"[full] {name}: generating inputs", flush=True)
    inp = synth.make_inputs(w, materialize=True)
    di = sdev.upload(inp)
    print(f"[full] {name}: running the layer and the oracle on about 96 sampled tokens "
          f"(half of them on the tile plan's partial tiles)", flush=True)
    rep, y, g, _ = parity.full_check(w, inp=inp, di=di, tokens=sample_tokens(w))
    print(f"[full] {name}: {dict((k, v) for k, v in rep.items() if k != 'modality_counts')}",
          flush=True)
    if w.n_bias_sets == 2:
        mc = np.array(rep["modality_counts"])
        assert mc.shape == (2, w.E)
        assert int(mc[1].sum()) == int(inp.modality.sum()) * w.k
    if w.f > 0:
        assert rep["dropped"] > 0          # the capacity workload really drops
    del di
