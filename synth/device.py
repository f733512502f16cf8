"""Upload synthetic inputs to the GPU as torch tensors (device memory only;
no arithmetic of the layer).  bf16 data keeps its exact bits."""
from __future__ import annotations

import concurrent.futures as cf
import os
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from . import Inputs, Workload


def _t(arr: np.ndarray, device) -> torch.Tensor:
    if arr.dtype == np.uint16:
        return torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(arr)).to(device)


def act_dtype(w: Workload):
    return torch.bfloat16 if w.dtype == "bf16" else torch.float32


@dataclass
class DeviceInputs:
    w: Workload
    x: torch.Tensor
    w_router: torch.Tensor
    logit_bias: Optional[torch.Tensor]
    sel_bias: Optional[torch.Tensor]
    modality: Optional[torch.Tensor]
    w_gate: Optional[torch.Tensor]
    w_up: torch.Tensor
    w_down: torch.Tensor
    ws_gate: Optional[torch.Tensor]
    ws_up: Optional[torch.Tensor]
    ws_down: Optional[torch.Tensor]


def _stack_upload(inp: Inputs, shared: bool, device, threads: int):
    """Allocate [n][..] device tensors and fill them expert by expert, drawing
    each expert on a host thread (the host never holds all experts at once)."""
    w = inp.w
    n = w.S if shared else w.E
    if n == 0:
        return None, None, None
    dt = act_dtype(w)
    gate = torch.empty((n, w.I, w.d), dtype=dt, device=device) if w.activation == "swiglu" else None
    up = torch.empty((n, w.I, w.d), dtype=dt, device=device)
    down = torch.empty((n, w.d, w.I), dtype=dt, device=device)
    get = inp.shared if shared else inp.expert

    def work(e):
        return e, get(e)

    with cf.ThreadPoolExecutor(threads) as ex:
        for e, (g, u, dn) in ex.map(work, range(n)):
            if gate is not None:
                gate[e].copy_(_t(g, "cpu"))
            up[e].copy_(_t(u, "cpu"))
            down[e].copy_(_t(dn, "cpu"))
    return gate, up, down


def upload(inp: Inputs, device="cuda", threads: Optional[int] = None) -> DeviceInputs:
    threads = threads or min(16, os.cpu_count() or 1)
    w = inp.w
    g, u, dn = _stack_upload(inp, False, device, threads)
    sg, su, sd = _stack_upload(inp, True, device, threads)
    return DeviceInputs(
        w=w, x=_t(inp.x, device), w_router=_t(inp.w_router, device),
        logit_bias=None if inp.logit_bias is None else _t(inp.logit_bias, device),
        sel_bias=None if inp.sel_bias is None else _t(inp.sel_bias, device),
        modality=None if inp.modality is None else _t(inp.modality, device),
        w_gate=g, w_up=u, w_down=dn, ws_gate=sg, ws_up=su, ws_down=sd)
