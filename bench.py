#!/usr/bin/env python3
"""Benchmark of the MoE-layer forward pass on one MI355X.

A step is one whole layer (router, top-k, dispatch, routed + shared experts,
combine) over one batch of seeded synthetic tokens already resident in HBM.
The default workload is the largest one-GPU layer, the DeepSeek-V4.1-Flash-
shaped multimodal layer (N=16384, d=5120, 384 routed + 1 shared SwiGLU experts
of inner size 2304 clipped at 10, top-6, sigmoid router with one selection-bias
set per modality, 30% image tokens in contiguous blocks).

Prints one JSON line: tokens/s, ms per step, the roofline entry of the
dominant kernel (timed with HIP events on the library's stream over the timed
region), the per-modality expert load histograms, the GPU clock sampled during
the timed steps, and the float64 CPU oracle timed on a bounded sample on this
host.  Progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_MFMA_TFLOPS = 2500.0    # MI355X dense bf16 / fp16 matrix peak
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def algorithmic(w, A, touched, dtype_bytes=2):
    """Algorithmic work of one layer step: (flops, bytes, gate_up_flops,
    gate_up_bytes).  Flops: router 2NdE + per kept assignment 6dI (SwiGLU) or
    4dI (ReLU) + the same per token for each shared expert.  Bytes: the weights
    of every touched expert and the shared experts, the router matrix, x read
    once and y (fp32) written once."""
    m = 3 if w.activation == "swiglu" else 2
    rows = A + w.N * w.S
    flops = 2 * w.N * w.d * w.E + 2 * m * w.d * w.I * rows
    wbytes = m * w.d * w.I * dtype_bytes
    nbytes = ((touched + w.S) * wbytes + w.d * w.E * dtype_bytes + w.N * w.d * dtype_bytes
              + w.N * w.d * 4)
    gu_mats = m - 1
    gu_flops = 2 * gu_mats * w.d * w.I * rows
    # gate/up launch: its weights (touched + shared), the gathered x rows, h (fp16) written
    gu_bytes = ((touched + w.S) * gu_mats * w.d * w.I * dtype_bytes + rows * w.d * dtype_bytes
                + rows * w.I * 2)
    return flops, nbytes, gu_flops, gu_bytes


def cpu_model() -> str:
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.lower().startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def _blas_info():
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        threads = max((i.get("num_threads", 1) for i in info), default=1)
        blas = ",".join(sorted({f"{i.get('internal_api')}" for i in info}))
    except Exception:  # pragma: no cover
        threads, blas = len(os.sched_getaffinity(0)), "unknown"
    return threads, blas


def cpu_baseline(w, inp, budget_s=15.0, reps=1, single_thread=False):
    """Time the float64 oracle (as it is) on a bounded sample of the workload
    and scale it to the whole layer:
      * routing + dispatch of the whole batch (timed as they are);
      * routed experts: a seeded sample of the touched experts runs through the
        oracle's forward (the routing restricted to them: the others' slots
        become 'no expert', so the oracle skips them), with each sampled
        expert's bf16 -> float64 weight upcast timed apart; FFN time is scaled
        by kept rows, upcast time by touched experts;
      * shared experts: their upcast, and the oracle on a prefix of the tokens
        (scaled by N / prefix).
    Data generation is outside every timed region.  reps > 1 keeps the best of
    that many measurements; single_thread adds the same estimate with one BLAS
    thread.  Memory: one sampled expert's float64 weights at a time."""
    import numpy as np
    from oracle import moe_oracle as O
    import synth
    threads, blas = _blas_info()
    x = synth.to_f64(w, inp.x)
    wr = synth.to_f64(w, inp.w_router)
    lb = None if inp.logit_bias is None else inp.logit_bias.astype(np.float64)
    sb = None if inp.sel_bias is None else inp.sel_bias.astype(np.float64)
    C = O.capacity(w.f, w.N, w.k, w.E)

    def route_once():
        t0 = time.perf_counter()
        r = O.route(x, wr, w.k, w.gating, lb, sb, inp.modality)
        disp = O.dispatch(r["idx"], w.E, C, inp.modality)
        return time.perf_counter() - t0, r, disp

    t_route, r, disp = route_once()
    rows = np.diff(disp["offsets"]).astype(np.int64)
    touched = np.nonzero(rows)[0]
    by_rows = touched[np.argsort(rows[touched], kind="stable")]
    A = int(rows.sum())

    def timed_get(enc, acc):
        def get(e):
            t = time.perf_counter()
            arrs = tuple(None if a is None else synth.to_f64(w, a) for a in enc[e])
            acc[0] += time.perf_counter() - t
            return arrs
        return get

    def run(idx, get, n_shared=0, get_shared=None, tokens=None):
        t0 = time.perf_counter()
        O.forward(x, w.k, w.E, w.gating, w.activation, get_expert=get, n_shared=n_shared,
                  get_shared=get_shared, clip=w.clip, f=w.f, modality=inp.modality,
                  forced_idx=idx, forced_w=r["g"], tokens=tokens)
        return time.perf_counter() - t0

    none = np.full((w.N, w.k), -1, np.int64)

    def measure(n_exp, n_tok, t_route=t_route):
        """One estimate of the whole layer's oracle time: n_exp routed experts
        spread evenly over the touched experts ordered by kept rows (so the
        sample's rows mirror the layer's), their time scaled by touched /
        n_exp; the shared experts on the first n_tok tokens, scaled by N /
        n_tok.  The oracle's per-call work that does not depend on the experts
        (dispatch, the loop over all E experts' masks) is timed apart, once."""
        sel = np.unique(np.linspace(0, len(by_rows) - 1, n_exp).round().astype(np.int64))
        sample = np.sort(by_rows[sel])
        enc = {int(e): inp.expert(int(e)) for e in sample}        # generated, untimed
        up = [0.0]
        t_fixed = run(none, timed_get({}, [0.0]))
        t_s = run(np.where(np.isin(r["idx"], sample), r["idx"], -1), timed_get(enc, up))
        scale = len(touched) / len(sample)
        res = {"route_s": t_route, "fixed_s": t_fixed,
               "routed_upcast_s": up[0] * scale,
               "routed_ffn_s": max(t_s - t_fixed - up[0], 0.0) * scale,
               "shared_upcast_s": 0.0, "shared_ffn_s": 0.0,
               "sample_s": t_s, "sampled_experts": int(len(sample)),
               "sampled_rows": int(rows[sample].sum()), "shared_tokens": 0}
        if w.S:
            senc = [inp.shared(j) for j in range(w.S)]
            sup = [0.0]
            toks = np.arange(n_tok)
            t_f = run(none, timed_get({}, [0.0]), tokens=toks)
            t_sh = run(none, timed_get({}, [0.0]), n_shared=w.S,
                       get_shared=timed_get(dict(enumerate(senc)), sup), tokens=toks)
            res["shared_upcast_s"] = sup[0]
            res["shared_ffn_s"] = max(t_sh - t_f - sup[0], 0.0) * w.N / n_tok
            res["shared_tokens"] = int(n_tok)
            res["sample_s"] += t_sh
        res["upcast_s"] = res["routed_upcast_s"] + res["shared_upcast_s"]
        res["experts_s"] = res["routed_ffn_s"] + res["shared_ffn_s"]
        res["total_s"] = t_route + t_fixed + res["upcast_s"] + res["experts_s"]
        return res

    # size the sample from a small probe: about half the budget on routed
    # experts, a third on the shared experts' token prefix
    probe = measure(min(2, len(touched)), min(w.N, 128))
    per_exp = (probe["routed_upcast_s"] + probe["routed_ffn_s"]) / max(len(touched), 1)
    n_exp = int(min(len(touched), max(2, 0.5 * budget_s / max(per_exp, 1e-6))))
    n_tok = 0
    if w.S:
        per_tok = probe["shared_ffn_s"] / w.N
        n_tok = int(min(w.N, max(128, budget_s / 3 / max(per_tok, 1e-9))))
    best = None
    for _ in range(max(1, reps)):
        est = measure(n_exp, n_tok)
        if best is None or est["total_s"] < best["total_s"]:
            best = est
    out = {"value": w.N / best["total_s"], "unit": "tokens/s", "cores": int(threads),
           "kind": "oracle", "cpu_model": cpu_model(), "blas": blas,
           "host_cpu_count": len(os.sched_getaffinity(0)), "best_of": max(1, reps),
           "route_s": best["route_s"], "upcast_s": best["upcast_s"],
           "experts_s": best["experts_s"], "fixed_s": best["fixed_s"],
           "layer_s": best["total_s"], "sample_s": best["sample_s"],
           "sample": (f"float64 NumPy oracle: routing + dispatch of all {w.N} tokens timed "
                      f"({best['route_s']:.2f} s); routed experts: {best['sampled_experts']} of "
                      f"the {len(touched)} touched experts, spread over their row counts "
                      f"({best['sampled_rows']} of {A} kept rows), through the oracle's forward, "
                      f"their time scaled by touched / sampled experts, with the bf16->float64 "
                      f"weight upcasts shown apart ({best['upcast_s']:.2f} s for the layer)"
                      + (f"; shared expert on the first {best['shared_tokens']} tokens, scaled "
                         f"by N" if w.S else "")
                      + f"; value = N / estimated layer time ({best['total_s']:.2f} s; "
                      f"{best['sample_s']:.1f} s measured on the sample)")}
    if single_thread:
        try:
            from threadpoolctl import threadpool_limits
            with threadpool_limits(limits=1):
                t1, _, _ = route_once()
                st = measure(max(2, n_exp // 16), max(128, n_tok // 16) if w.S else 0, t1)
            out["single_thread"] = {"value": w.N / st["total_s"], "layer_s": st["total_s"],
                                    "upcast_s": st["upcast_s"],
                                    "sampled_experts": st["sampled_experts"]}
        except Exception as e:  # pragma: no cover
            out["single_thread"] = {"error": str(e)}
    return out


def cpu_baseline_backward(w, inp, budget_s=15.0):
    """Time the float64 oracle's backward (as it is) on a bounded sample: the
    batch of the first n tokens (same weights and layer), n sized to the
    budget.  Returns the dict for the JSON line."""
    import numpy as np
    from oracle import moe_oracle as O
    import synth
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        threads = max((i.get("num_threads", 1) for i in info), default=1)
        blas = ",".join(sorted({f"{i.get('internal_api')}" for i in info}))
    except Exception:  # pragma: no cover
        threads, blas = len(os.sched_getaffinity(0)), "unknown"
    x = synth.to_f64(w, inp.x)
    wr = synth.to_f64(w, inp.w_router)
    dy = synth.upstream_grad(w).astype(np.float64)
    lb = None if inp.logit_bias is None else inp.logit_bias.astype(np.float64)
    sb = None if inp.sel_bias is None else inp.sel_bias.astype(np.float64)
    cache = {}

    def get(e, shared=False):
        key = (shared, e)
        if key not in cache:
            arrs = inp.shared(e) if shared else inp.expert(e)
            cache[key] = tuple(None if a is None else synth.to_f64(w, a) for a in arrs)
        return cache[key]

    for e in range(w.E):
        get(e)
    for s in range(w.S):
        get(s, True)

    def run(n):
        mod = None if inp.modality is None else inp.modality[:n]
        t = time.perf_counter()
        O.backward(x[:n], w.k, w.E, w.gating, w.activation, get_expert=get, n_shared=w.S,
                   get_shared=lambda s: get(s, True), w_router=wr, clip=w.clip, f=w.f,
                   logit_bias=lb, sel_bias=sb, modality=mod, dy=dy[:n],
                   renormalize=w.renormalize, overflow=w.overflow)
        return time.perf_counter() - t

    n2 = min(w.N, 64)
    t = run(n2)
    # grow the sample until it takes about the budget (the first runs include
    # one-time costs, so one extrapolation step can fall short)
    while n2 < w.N and t < 0.5 * budget_s:
        n2 = int(min(w.N, max(2 * n2, n2 * budget_s / max(t, 1e-6))))
        t = run(n2)
    return {"value": n2 / t, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": (f"float64 NumPy oracle ({blas} BLAS): backward of the batch of the first "
                       f"{n2} tokens ({t:.2f} s; same weights, layer options and capacity "
                       f"factor); value = {n2} / time"),
            "host_cpu_count": len(os.sched_getaffinity(0))}


class ClockSampler:
    """Samples the GPU's graphics clock on a host thread while the timed steps
    run: the current level of the driver's sclk table (sysfs pp_dpm_sclk, the
    entry marked '*', in MHz).  Reports mean, min and max, or why it could not
    (then mhz_mean is null)."""

    def __init__(self, period_s=0.005):
        import glob
        import threading
        self.period = period_s
        self.samples = []
        self.error = None
        self._stop = threading.Event()
        self._thread = None
        self.path = None
        try:
            paths = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
            if not paths:
                raise RuntimeError("no pp_dpm_sclk in sysfs")
            self.path = paths[0]
            if len(paths) > 1:
                # the GPU torch runs on, by PCI bus number
                import torch
                pr = torch.cuda.get_device_properties(torch.cuda.current_device())
                bus = getattr(pr, "pci_bus_id", None)
                for q in paths:
                    addr = os.path.basename(os.path.realpath(os.path.dirname(q)))
                    if bus is not None and int(addr.split(":")[1], 16) == bus:
                        self.path = q
            self.read()
        except Exception as e:
            self.error = f"{type(e).__name__}: {e}"

    def read(self):
        for ln in open(self.path).read().splitlines():
            if ln.rstrip().endswith("*"):
                return float(ln.split(":", 1)[1].strip().split("M")[0])
        raise RuntimeError("no current level marked")

    def _run(self):
        while not self._stop.is_set():
            try:
                self.samples.append(self.read())
            except Exception as e:  # pragma: no cover
                self.error = f"{type(e).__name__}: {e}"
                return
            time.sleep(self.period)

    def start(self):
        if self.error is None:
            import threading
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()

    def stop(self):
        if self._thread is not None:
            self._stop.set()
            self._thread.join()
        if self.error is not None or not self.samples:
            return {"mhz_mean": None, "note": self.error or "no samples"}
        import numpy as np
        a = np.asarray(self.samples)
        return {"mhz_mean": float(a.mean()), "mhz_min": float(a.min()), "mhz_max": float(a.max()),
                "samples": int(a.size),
                "source": f"{self.path} (current sclk level), sampled every "
                          f"{self.period * 1e3:.0f} ms during the timed steps"}


def modality_loads(w, counts, mcounts, modality):
    """Per-modality expert load histograms: demand per expert for text and image
    tokens, and each expert's share of the modality's assignments."""
    import numpy as np
    n_img = int(np.asarray(modality).sum())
    res = {}
    for m, name in enumerate(("text", "image")):
        c = np.asarray(mcounts[m], np.int64)
        tot = int(c.sum())
        share = c / tot if tot else np.zeros_like(c, dtype=np.float64)
        res[name] = {"tokens": (w.N - n_img) if m == 0 else n_img, "assignments": tot,
                     "counts": c.tolist(), "load_share": [round(float(v), 6) for v in share],
                     "max_over_mean": float(c.max() * w.E / tot) if tot else 0.0,
                     "idle_experts": int((c == 0).sum())}
    res["all"] = {"counts": np.asarray(counts, np.int64).tolist()}
    return res


def roofline_entry(flops, nbytes, ms, traffic):
    """The roofline entry of a launch with the given algorithmic flops and
    bytes: bound by HBM when its flops per byte are below the ridge (peak
    flops / peak bandwidth, 312.5 flop/B), else by the matrix cores."""
    ridge = PEAK_MFMA_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    intensity = flops / max(nbytes, 1)
    if intensity < ridge:
        ach = nbytes / (ms * 1e-3) / 1e9
        return {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": ach / PEAK_HBM_GBS, "traffic": traffic, "algorithmic_per_launch": nbytes,
                "flop_per_byte": intensity}
    ach = flops / (ms * 1e-3) / 1e12
    return {"bound": "mfma", "achieved": ach, "peak": PEAK_MFMA_TFLOPS, "unit": "TFLOP/s",
            "frac": ach / PEAK_MFMA_TFLOPS, "traffic": traffic, "algorithmic_per_launch": flops,
            "flop_per_byte": intensity}


def code_hash(path: str) -> str:
    """sha256 of a source file with its comments and white space removed: a
    counter summary stays matched to the code it measured across edits of the
    comments, and to no other code."""
    s = open(path, encoding="utf-8").read()
    s = re.sub(r"/\*.*?\*/", " ", s, flags=re.S)
    s = re.sub(r"//[^\n]*", " ", s)
    return hashlib.sha256("".join(s.split()).encode()).hexdigest()


def pmc_traffic(kernel: str, workload: str, src_hash: str):
    """HBM traffic of one launch from a committed rocprofv3 counter summary, if
    it was taken on the current kernel code (code_hash); else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_pmc.json")
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
    except Exception:
        return None
    if d.get("code_sha256") != src_hash:
        return None
    return d.get("hbm_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1,
                    help="GPUs (one only: the layer runs on one GPU; more exits with a message)")
    ap.add_argument("--steps", type=int, default=100, help="timed steps")
    ap.add_argument("--warmup", type=int, default=10, help="untimed steps before them")
    ap.add_argument("--workload", default="v41",
                    help="v41 (default), cap, mix-P, ds-P, mix-D, ds-D, toy, or a small member "
                         "of a family (cap-s, mix-s, ds-s, v41-s, ...)")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip timing the float64 oracle on the host")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of host time the oracle sample is sized for")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward pass (moe_backward on the forward's routing and "
                         "saved pre-activations) instead of the forward")
    ap.add_argument("--dw-bf16", action="store_true",
                    help="with --backward: weight gradients written as bf16 instead of float32")
    ap.add_argument("--recompute", action="store_true",
                    help="with --backward: the forward saves no pre-activations, the backward "
                         "recomputes them")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after the run, copy 256 MiB device-to-device once: a kernel of known "
                         "traffic to scale rocprofv3's FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs the MoE layer on exactly one GPU; multi-GPU runs (expert or "
              "token sharding over xGMI) are not built. Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import synth
    from synth import device as sdev
    from mixture_experts_layer_16_amd import _lib as L

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    w = synth.get(args.workload)
    log(f"workload {w.name}: N={w.N} d={w.d} E={w.E}+{w.S} k={w.k} I={w.I} f={w.f}")
    t = time.perf_counter()
    inp = synth.make_inputs(w)
    di = sdev.upload(inp)
    log(f"inputs generated and uploaded in {time.perf_counter() - t:.1f} s")

    p = L.problem(w.N, w.d, w.E, w.k, w.I, S=w.S, gating=w.gating, activation=w.activation,
                  dtype=w.dtype, n_bias_sets=w.n_bias_sets, act_clip=w.clip,
                  capacity_factor=w.f)
    if args.backward:
        return bench_backward(args, w, inp, di, p)
    ws = L.workspace(p)
    y = torch.empty((w.N, w.d), dtype=torch.float32, device="cuda")
    offsets = torch.empty(w.E + 1, dtype=torch.int32, device="cuda")
    counts = torch.empty(w.E, dtype=torch.int32, device="cuda")
    mcounts = (torch.empty(2 * w.E, dtype=torch.int32, device="cuda")
               if w.n_bias_sets == 2 else None)
    sat = torch.zeros(1, dtype=torch.int32, device="cuda")
    rout = L.routing(offsets=offsets, counts=counts, modality_counts=mcounts, sat_count=sat)
    wts = L.weights(di.w_router, di.w_gate, di.w_up, di.w_down, di.ws_gate, di.ws_up, di.ws_down)
    stream = torch.cuda.current_stream()

    def step(profile=None):
        L.moe_forward(p, wts, di.x, di.logit_bias, di.sel_bias, di.modality, y, rout, ws,
                      stream=stream, profile=profile)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps done")

    # timed region: K steps; the gate/up GEMM (dominant kernel) is bracketed by
    # HIP events recorded on the same stream by the library
    K = args.steps
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(K)]
    for a, b in evs:
        a.record(stream)
        b.record(stream)
    profs = [L.profile({("gate_up", 0): a, ("gate_up", 1): b}) for a, b in evs]
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    clock = ClockSampler()
    clock.start()
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(K):
        step(profs[i])
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    clk = clock.stop()
    ms_step = wall * 1e3 / K
    ms_step_ev = e0.elapsed_time(e1) / K
    gu_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    log(f"timed {K} steps: {ms_step:.4f} ms/step wall, {ms_step_ev:.4f} ms/step events, "
        f"gate/up {gu_ms:.4f} ms")

    # per-stage breakdown (separate, untimed-for-value pass)
    stage_ev = {(s, j): torch.cuda.Event(enable_timing=True) for s in L.STAGES for j in (0, 1)}
    for ev in stage_ev.values():
        ev.record(stream)
    torch.cuda.synchronize()
    sprof = L.profile(stage_ev)
    reps = 10
    acc = {s: 0.0 for s in L.STAGES}
    for _ in range(reps):
        step(sprof)
        torch.cuda.synchronize()
        for s in L.STAGES:
            acc[s] += stage_ev[(s, 0)].elapsed_time(stage_ev[(s, 1)]) / reps
    log("stages ms: " + ", ".join(f"{s}={v:.4f}" for s, v in acc.items()))

    off = offsets.cpu().numpy()
    A = int(off[-1])
    touched = int(np.count_nonzero(np.diff(off)))
    n_sat = int(sat.cpu().item())
    if n_sat:
        log(f"WARNING: {n_sat} fp16 intermediates saturated")
    loads = None
    if mcounts is not None:
        loads = modality_loads(w, counts.cpu().numpy(),
                               mcounts.cpu().numpy().reshape(2, w.E), inp.modality)
        log("per-modality load: " + ", ".join(
            f"{m}: {loads[m]['assignments']} assignments, max/mean {loads[m]['max_over_mean']:.2f}"
            f", {loads[m]['idle_experts']} idle" for m in ("text", "image")))
    flops, nbytes, gu_flops, gu_bytes = algorithmic(w, A, touched,
                                                    dtype_bytes=2 if w.dtype == "bf16" else 4)
    tokens_s = w.N / (ms_step * 1e-3)
    layer_tflops = flops / (ms_step * 1e-3) / 1e12
    layer_gbs = nbytes / (ms_step * 1e-3) / 1e9
    src_hash = code_hash(os.path.join(ROOT, "mixture_experts_layer_16_amd", "csrc", "gemm.hip"))
    # the gate/up grouped GEMM (ffn_gemm_dl<GATEUP, 256, 8> for prefill,
    # ffn_gemm_bf16<GATEUP, 32, ...> for decode batches)
    kname = "ffn_gemm_gate_up"
    traffic = pmc_traffic(kname, w.name, src_hash)
    roof = roofline_entry(gu_flops, gu_bytes, gu_ms, traffic)
    roof["kernel"] = kname
    roof["ms_per_launch"] = gu_ms

    if args.calibrate_copy:
        a = torch.ones(64 * 1024 * 1024, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        log("calibration copy of 256 MiB done")

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the float64 CPU oracle on a bounded sample ...")
        small = w.N <= 64 or w.name in ("cap", "toy") or w.name.endswith("-s")
        cpu = cpu_baseline(w, inp, args.cpu_budget, reps=3 if small else 1,
                           single_thread=small)
        log(f"cpu oracle {cpu['value']:.1f} tokens/s on {cpu['cores']} threads")

    out = {
        "metric": "MoE-layer tokens/s at 1 GPU",
        "value": tokens_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded; random-init weights of the stated shapes)",
        "config": {"workload": w.name, "N": w.N, "d": w.d, "E": w.E, "S": w.S, "k": w.k,
                   "I": w.I, "capacity_factor": w.f, "gating": w.gating,
                   "activation": w.activation, "clip": w.clip,
                   "n_bias_sets": w.n_bias_sets, "image_frac": w.image_frac,
                   "kept_assignments": A, "touched_experts": touched},
        "layer": {"tflops": layer_tflops, "mfma_frac": layer_tflops / PEAK_MFMA_TFLOPS,
                  "gbs": layer_gbs, "hbm_frac": layer_gbs / PEAK_HBM_GBS,
                  "algorithmic_flops": flops, "algorithmic_bytes": nbytes,
                  "ms_per_step_events": ms_step_ev, "fp16_saturated": n_sat},
        "stages_ms": acc,
        "roofline": roof,
        "gpu_clock": clk,
        "modality_load": loads,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def bench_backward(args, w, inp, di, p):
    """The backward pass: forward once for the routing (and, unless
    --recompute, the saved pre-activations), then K timed calls of
    moe_backward (all gradients: x, every expert, shared experts, router,
    logit offset).  Dominant stage: the three weight-gradient grouped GEMMs."""
    import numpy as np
    import torch
    import synth
    from mixture_experts_layer_16_amd import _lib as L

    dev = "cuda"
    N, d, E, k, I, S = w.N, w.d, w.E, w.k, w.I, w.S
    i32, f32 = torch.int32, torch.float32
    rt_t = dict(topk_idx=torch.empty(N * k, dtype=i32, device=dev),
                topk_w=torch.empty(N * k, dtype=f32, device=dev),
                offsets=torch.empty(E + 1, dtype=i32, device=dev),
                row_of=torch.empty(N * k, dtype=i32, device=dev),
                token_of_row=torch.empty(N * k, dtype=i32, device=dev),
                logits=torch.empty(N * E, dtype=torch.float64, device=dev))
    swiglu = w.activation == "swiglu"
    if not args.recompute:
        # the training forward keeps x W_gate^T and x W_up^T (fp16) for the backward
        rt_t["act_u"] = torch.empty((N * (k + S), I), dtype=torch.float16, device=dev)
        if swiglu:
            rt_t["act_a"] = torch.empty((N * (k + S), I), dtype=torch.float16, device=dev)
    wts = L.weights(di.w_router, di.w_gate, di.w_up, di.w_down, di.ws_gate, di.ws_up, di.ws_down)
    rt = L.routing(**rt_t)
    ws = L.workspace(p)
    y = torch.empty((N, d), dtype=f32, device=dev)
    L.moe_forward(p, wts, di.x, di.logit_bias, di.sel_bias, di.modality, y, rt, ws)
    torch.cuda.synchronize()
    del ws, y
    wt = torch.bfloat16 if args.dw_bf16 else f32
    g = dict(dx=torch.empty((N, d), dtype=f32, device=dev),
             dw_router=torch.empty((E, d), dtype=wt, device=dev),
             dw_up=torch.empty((E, I, d), dtype=wt, device=dev),
             dw_down=torch.empty((E, d, I), dtype=wt, device=dev),
             d_logit_bias=torch.empty(E, dtype=f32, device=dev))
    if swiglu:
        g["dw_gate"] = torch.empty((E, I, d), dtype=wt, device=dev)
    if S:
        g["dws_up"] = torch.empty((S, I, d), dtype=wt, device=dev)
        g["dws_down"] = torch.empty((S, d, I), dtype=wt, device=dev)
        if swiglu:
            g["dws_gate"] = torch.empty((S, I, d), dtype=wt, device=dev)
    dy = torch.from_numpy(synth.upstream_grad(w)).to(dev)
    bws = L.backward_workspace(p)
    gr = L.grads(dw_bf16=args.dw_bf16, **g)
    stream = torch.cuda.current_stream()
    log(f"backward: workspace {bws.numel() / 2**30:.2f} GiB, gradients "
        f"{sum(t.numel() * t.element_size() for t in g.values()) / 2**30:.2f} GiB")

    def step(prof=None):
        L.moe_backward_ex(p, wts, di.x, rt, dy, gr, prof, bws, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(K)]
    for a, b in evs:
        a.record(stream)
        b.record(stream)
    profs = [L.profile({("wgrad", 0): a, ("wgrad", 1): b}, L.BSTAGES) for a, b in evs]
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(K):
        step(profs[i])
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / K
    ms_step_ev = e0.elapsed_time(e1) / K
    wg_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    log(f"timed {K} backward steps: {ms_step:.4f} ms/step wall, {ms_step_ev:.4f} ms/step "
        f"events, weight gradients {wg_ms:.4f} ms")
    stage_ev = {(s_, j): torch.cuda.Event(enable_timing=True) for s_ in L.BSTAGES for j in (0, 1)}
    for ev in stage_ev.values():
        ev.record(stream)
    torch.cuda.synchronize()
    sprof = L.profile(stage_ev, L.BSTAGES)
    acc = {s_: 0.0 for s_ in L.BSTAGES}
    reps = 5
    for _ in range(reps):
        step(sprof)
        torch.cuda.synchronize()
        for s_ in L.BSTAGES:
            acc[s_] += stage_ev[(s_, 0)].elapsed_time(stage_ev[(s_, 1)]) / reps
    log("backward stages ms: " + ", ".join(f"{s_}={v:.4f}" for s_, v in acc.items()))

    off = rt_t["offsets"].cpu().numpy()
    A = int(off[-1])
    rows = A + N * S
    m = 3 if swiglu else 2
    # chain-rule flops: dh 2dI, weight gradients 2dI each, dx 2dI per matrix
    # with a reduction over I (gate, up); router dW and dx 2NdE each.  The
    # recomputation of a and u (m-1 products) is counted apart.
    flops = (1 + m + (m - 1)) * 2 * d * I * rows + 4 * N * d * E
    flops_recompute = (m - 1) * 2 * d * I * rows
    # the weight-gradient stage: m launches of 2·d·I flop per row; each writes
    # every expert's and shared expert's float32 dW and reads its two operands
    # (bf16 rows) once
    per_launch = 2 * d * I * rows
    per_launch_bytes = (E + S) * d * I * (2 if args.dw_bf16 else 4) + rows * (d + I) * 2
    kname = "bwd_gemm_wgrad"
    roof = roofline_entry(per_launch, per_launch_bytes, wg_ms / m,
                          pmc_traffic(kname, w.name, code_hash(
                              os.path.join(ROOT, "mixture_experts_layer_16_amd", "csrc",
                                           "backward.hip"))))
    roof.update({"kernel": kname, "launches_per_step": m, "ms_per_launch": wg_ms / m})
    if args.calibrate_copy:
        a = torch.ones(64 * 1024 * 1024, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        log("calibration copy of 256 MiB done")
    cpu = None
    if not args.no_cpu_baseline:
        log("timing the float64 CPU oracle's backward on a bounded sample ...")
        cpu = cpu_baseline_backward(w, inp, args.cpu_budget)
        log(f"cpu oracle backward {cpu['value']:.1f} tokens/s on {cpu['cores']} threads")
    out = {
        "metric": "MoE-layer backward tokens/s at 1 GPU",
        "value": N / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; random-init weights of the stated shapes; dy ~ N(0, 1))",
        "config": {"workload": w.name, "pass": "backward",
                   "activations": "recomputed" if args.recompute else "saved by the forward",
                   "weight_gradients": "bf16" if args.dw_bf16 else "float32",
                   "N": N, "d": d, "E": E, "S": S,
                   "k": k, "I": I, "capacity_factor": w.f, "gating": w.gating,
                   "activation": w.activation, "kept_assignments": A},
        "layer": {"tflops": flops / (ms_step * 1e-3) / 1e12,
                  "mfma_frac": flops / (ms_step * 1e-3) / 1e12 / PEAK_MFMA_TFLOPS,
                  "algorithmic_flops": flops, "recompute_flops": flops_recompute,
                  "ms_per_step_events": ms_step_ev},
        "stages_ms": acc,
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
