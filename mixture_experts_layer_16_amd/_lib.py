"""ctypes binding of ``libmoe.so`` (the C ABI declared in include/moe.h).

Argument marshalling only: every step of the layer runs in the HIP kernels of
the library.  Tensors are torch device tensors (PyTorch provides the device
memory and the stream); they are passed as raw pointers.  There is no fallback:
if the library is missing, importing this module raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch  # noqa: F401  -- load torch's HIP runtime first so the library shares it

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe.so")

MOE_SOFTMAX, MOE_SIGMOID = 0, 1
MOE_OVERFLOW_DROP, MOE_OVERFLOW_REROUTE = 0, 1
MOE_SWIGLU, MOE_RELU = 0, 1
MOE_BF16, MOE_F32 = 0, 1
STATUS = {0: "MOE_OK", -1: "MOE_ERR_NULL", -2: "MOE_ERR_INVALID", -3: "MOE_ERR_UNSUPPORTED",
          -4: "MOE_ERR_WORKSPACE", -5: "MOE_ERR_HIP", -6: "MOE_ERR_TOO_LARGE"}
NOALLOC_SCRATCH_BYTES = 64 << 20   # MOE_NOALLOC_SCRATCH_BYTES

# every function include/moe.h declares
EXPORTS = ("moe_workspace_size", "moe_capacity", "moe_param_counts", "moe_route",
           "moe_permute", "moe_expert_ffn", "moe_combine", "moe_forward", "moe_forward_ex",
           "moe_balance", "moe_forward_routed", "moe_route_hash", "moe_backward_workspace_size",
           "moe_backward", "moe_backward_ex", "moe_status_string", "moe_version",
           "moe_forward_noalloc")
STAGES = ("route", "permute", "plan", "gate_up", "down", "combine")
BSTAGES = ("prep", "recompute", "dh", "rows", "wgrad", "dx")


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} ({msg})")
        self.status = status


class Problem(ctypes.Structure):
    _fields_ = [("n_tokens", ctypes.c_int64), ("d_model", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("d_expert", ctypes.c_int32), ("n_shared", ctypes.c_int32),
                ("gating", ctypes.c_int32), ("activation", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("n_bias_sets", ctypes.c_int32),
                ("renormalize", ctypes.c_int32), ("act_clip", ctypes.c_float),
                ("capacity_factor", ctypes.c_double), ("overflow", ctypes.c_int32)]


class Weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("w_router", "w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down")]


class Routing(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("topk_idx", "topk_w", "counts", "modality_counts", "offsets", "row_of",
                 "token_of_row", "drop_mask", "logits", "final_idx", "act_a", "act_u",
                 "sat_count")]


class Grads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("dx", "dw_router", "dw_gate", "dw_up", "dw_down", "dws_gate", "dws_up",
                 "dws_down", "d_logit_bias", "dz", "dg")] + [("dw_bf16", ctypes.c_int32)]


class Profile(ctypes.Structure):
    _fields_ = [("ev", ctypes.c_void_p * (2 * len(STAGES)))]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m "
                          "mixture_experts_layer_16_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    P, V = ctypes.POINTER(Problem), ctypes.c_void_p
    i64p = ctypes.POINTER(ctypes.c_int64)
    sig = {
        "moe_workspace_size": [P, ctypes.POINTER(ctypes.c_size_t)],
        "moe_capacity": [P, i64p],
        "moe_param_counts": [P, i64p, i64p, i64p],
        "moe_route": [P, V, V, V, V, V, V, V, V, V, ctypes.c_size_t, V],
        "moe_permute": [P, V, V, V, V, V, V, V, V, V, ctypes.c_size_t, V],
        "moe_expert_ffn": [P, V, V, V, V, V, V, V, V, ctypes.c_size_t, V],
        "moe_combine": [P, V, V, V, V, V, V],
        "moe_forward": [P, ctypes.POINTER(Weights), V, V, V, V, V, ctypes.POINTER(Routing), V,
                        ctypes.c_size_t, V],
        "moe_forward_ex": [P, ctypes.POINTER(Weights), V, V, V, V, V, ctypes.POINTER(Routing),
                           ctypes.POINTER(Profile), V, ctypes.c_size_t, V],
        "moe_balance": [P, V, V, V, V, V, V, V, ctypes.c_float, V, ctypes.c_size_t, V],
        "moe_forward_noalloc": [P, ctypes.POINTER(Weights), V, V, V, V, V,
                                ctypes.POINTER(Routing), V],
        "moe_forward_routed": [P, ctypes.POINTER(Weights), V, V, V, V, V,
                               ctypes.POINTER(Routing), V, ctypes.c_size_t, V],
        "moe_route_hash": [P, V, V, V, V],
        "moe_backward_workspace_size": [P, ctypes.POINTER(ctypes.c_size_t)],
        "moe_backward": [P, ctypes.POINTER(Weights), V, ctypes.POINTER(Routing), V,
                         ctypes.POINTER(Grads), V, ctypes.c_size_t, V],
        "moe_backward_ex": [P, ctypes.POINTER(Weights), V, ctypes.POINTER(Routing), V,
                            ctypes.POINTER(Grads), ctypes.POINTER(Profile), V, ctypes.c_size_t,
                            V],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    lib.moe_status_string.argtypes = [ctypes.c_int]
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_version.argtypes = []
    lib.moe_version.restype = ctypes.c_char_p
    return lib


LIB = _load()


def _check(fn: str, st: int) -> None:
    if st != 0:
        raise MoeError(fn, st, LIB.moe_status_string(st).decode())


def ptr(t) -> Optional[int]:
    """Raw address of a tensor (None -> NULL)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def problem(N, d, E, k, I, S=0, gating=MOE_SOFTMAX, activation=MOE_SWIGLU, dtype=MOE_BF16,
            n_bias_sets=0, act_clip=0.0, capacity_factor=0.0, renormalize=1,
            overflow=0) -> Problem:
    if isinstance(gating, str):
        gating = {"softmax": MOE_SOFTMAX, "sigmoid": MOE_SIGMOID}[gating]
    if isinstance(activation, str):
        activation = {"swiglu": MOE_SWIGLU, "relu": MOE_RELU}[activation]
    if isinstance(dtype, str):
        dtype = {"bf16": MOE_BF16, "f32": MOE_F32}[dtype]
    if isinstance(overflow, str):
        overflow = {"drop": MOE_OVERFLOW_DROP, "reroute": MOE_OVERFLOW_REROUTE}[overflow]
    return Problem(int(N), int(d), int(E), int(k), int(I), int(S), int(gating), int(activation),
                   int(dtype), int(n_bias_sets), int(renormalize), float(act_clip),
                   float(capacity_factor), int(overflow))


# ---------------------------------------------------------------------------
# host queries

def moe_workspace_size(p: Problem) -> int:
    out = ctypes.c_size_t(0)
    _check("moe_workspace_size", LIB.moe_workspace_size(ctypes.byref(p), ctypes.byref(out)))
    return out.value


def moe_capacity(p: Problem) -> int:
    out = ctypes.c_int64(0)
    _check("moe_capacity", LIB.moe_capacity(ctypes.byref(p), ctypes.byref(out)))
    return out.value


def moe_param_counts(p: Problem):
    a, b, c = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    _check("moe_param_counts", LIB.moe_param_counts(ctypes.byref(p), ctypes.byref(a),
                                                    ctypes.byref(b), ctypes.byref(c)))
    return a.value, b.value, c.value


def moe_backward_workspace_size(p: Problem) -> int:
    out = ctypes.c_size_t(0)
    _check("moe_backward_workspace_size",
           LIB.moe_backward_workspace_size(ctypes.byref(p), ctypes.byref(out)))
    return out.value


def moe_status_string(status: int) -> str:
    return LIB.moe_status_string(int(status)).decode()


def moe_version() -> str:
    return LIB.moe_version().decode()


# ---------------------------------------------------------------------------
# device entry points (torch tensors in, results written into given tensors)

def workspace(p: Problem, device="cuda") -> torch.Tensor:
    """A device byte buffer of moe_workspace_size(p) bytes (allocated by torch)."""
    return torch.empty(max(1, moe_workspace_size(p)), dtype=torch.uint8, device=device)


def moe_route(p, x, w_router, logit_bias, sel_bias, modality, topk_idx, topk_w, logits=None,
              ws=None, stream=None, raw=False):
    st = LIB.moe_route(ctypes.byref(p), ptr(x), ptr(w_router), ptr(logit_bias), ptr(sel_bias),
                       ptr(modality), ptr(topk_idx), ptr(topk_w), ptr(logits), ptr(ws),
                       ws.numel() if ws is not None and not isinstance(ws, int) else 0,
                       _stream(stream))
    if raw:
        return st
    _check("moe_route", st)


def moe_permute(p, topk_idx, modality, counts, modality_counts, offsets, row_of, token_of_row,
                drop_mask, ws, stream=None, raw=False):
    st = LIB.moe_permute(ctypes.byref(p), ptr(topk_idx), ptr(modality), ptr(counts),
                         ptr(modality_counts), ptr(offsets), ptr(row_of), ptr(token_of_row),
                         ptr(drop_mask), ptr(ws),
                         ws.numel() if ws is not None and not isinstance(ws, int) else 0,
                         _stream(stream))
    if raw:
        return st
    _check("moe_permute", st)


def moe_expert_ffn(p, x, token_of_row, offsets, w_gate, w_up, w_down, y_rows, ws, stream=None,
                   raw=False):
    st = LIB.moe_expert_ffn(ctypes.byref(p), ptr(x), ptr(token_of_row), ptr(offsets),
                            ptr(w_gate), ptr(w_up), ptr(w_down), ptr(y_rows), ptr(ws),
                            ws.numel() if ws is not None and not isinstance(ws, int) else 0,
                            _stream(stream))
    if raw:
        return st
    _check("moe_expert_ffn", st)


def moe_combine(p, y_rows, row_of, topk_w, y_shared, y, stream=None, raw=False):
    st = LIB.moe_combine(ctypes.byref(p), ptr(y_rows), ptr(row_of), ptr(topk_w), ptr(y_shared),
                         ptr(y), _stream(stream))
    if raw:
        return st
    _check("moe_combine", st)


def moe_balance(p, logits, counts, modality_counts, load, mean_prob, aux, sel_bias, gamma,
                ws=None, stream=None, raw=False):
    st = LIB.moe_balance(ctypes.byref(p), ptr(logits), ptr(counts), ptr(modality_counts),
                         ptr(load), ptr(mean_prob), ptr(aux), ptr(sel_bias), float(gamma),
                         ptr(ws), ws.numel() if ws is not None and not isinstance(ws, int) else 0,
                         _stream(stream))
    if raw:
        return st
    _check("moe_balance", st)


def moe_forward_routed(p, w: "Weights", x, topk_idx, topk_w, modality, y, routing_out=None,
                       ws=None, stream=None, raw=False):
    st = LIB.moe_forward_routed(ctypes.byref(p), ctypes.byref(w), ptr(x), ptr(topk_idx),
                                ptr(topk_w), ptr(modality), ptr(y),
                                ctypes.byref(routing_out) if routing_out is not None else None,
                                ptr(ws),
                                ws.numel() if ws is not None and not isinstance(ws, int) else 0,
                                _stream(stream))
    if raw:
        return st
    _check("moe_forward_routed", st)


def moe_route_hash(p, token_ids, topk_idx, topk_w, stream=None, raw=False):
    st = LIB.moe_route_hash(ctypes.byref(p), ptr(token_ids), ptr(topk_idx), ptr(topk_w),
                            _stream(stream))
    if raw:
        return st
    _check("moe_route_hash", st)


def backward_workspace(p: Problem, device="cuda") -> torch.Tensor:
    """A device byte buffer of moe_backward_workspace_size(p) bytes."""
    return torch.empty(max(1, moe_backward_workspace_size(p)), dtype=torch.uint8, device=device)


def moe_backward(p, w: "Weights", x, routing_in: "Routing", dy, grads_out: "Grads", ws=None,
                 stream=None, raw=False):
    st = LIB.moe_backward(ctypes.byref(p), ctypes.byref(w), ptr(x),
                          ctypes.byref(routing_in) if routing_in is not None else None, ptr(dy),
                          ctypes.byref(grads_out) if grads_out is not None else None, ptr(ws),
                          ws.numel() if ws is not None and not isinstance(ws, int) else 0,
                          _stream(stream))
    if raw:
        return st
    _check("moe_backward", st)


def moe_backward_ex(p, w: "Weights", x, routing_in: "Routing", dy, grads_out: "Grads",
                    prof=None, ws=None, stream=None, raw=False):
    st = LIB.moe_backward_ex(ctypes.byref(p), ctypes.byref(w), ptr(x),
                             ctypes.byref(routing_in) if routing_in is not None else None,
                             ptr(dy), ctypes.byref(grads_out) if grads_out is not None else None,
                             ctypes.byref(prof) if prof is not None else None, ptr(ws),
                             ws.numel() if ws is not None and not isinstance(ws, int) else 0,
                             _stream(stream))
    if raw:
        return st
    _check("moe_backward_ex", st)


def grads(dw_bf16=False, **tensors) -> Grads:
    return Grads(**{k: ptr(v) for k, v in tensors.items()}, dw_bf16=int(dw_bf16))


def weights(w_router, w_gate, w_up, w_down, ws_gate=None, ws_up=None, ws_down=None) -> Weights:
    return Weights(ptr(w_router), ptr(w_gate), ptr(w_up), ptr(w_down), ptr(ws_gate),
                   ptr(ws_up), ptr(ws_down))


def routing(**tensors) -> Routing:
    return Routing(**{k: ptr(v) for k, v in tensors.items()})


def moe_forward(p, w: Weights, x, logit_bias, sel_bias, modality, y, routing_out=None, ws=None,
                stream=None, raw=False, profile: "Profile" = None):
    rout = ctypes.byref(routing_out) if routing_out is not None else None
    nb = ws.numel() if ws is not None and not isinstance(ws, int) else 0
    if profile is None:
        st = LIB.moe_forward(ctypes.byref(p), ctypes.byref(w), ptr(x), ptr(logit_bias),
                             ptr(sel_bias), ptr(modality), ptr(y), rout, ptr(ws), nb,
                             _stream(stream))
    else:
        st = LIB.moe_forward_ex(ctypes.byref(p), ctypes.byref(w), ptr(x), ptr(logit_bias),
                                ptr(sel_bias), ptr(modality), ptr(y), rout,
                                ctypes.byref(profile), ptr(ws), nb, _stream(stream))
    if raw:
        return st
    _check("moe_forward", st)


def moe_forward_noalloc(p, w: Weights, x, logit_bias, sel_bias, modality, y, routing_out=None,
                        stream=None, raw=False):
    """moe_forward on the library's fixed per-GPU scratch (no workspace)."""
    rout = ctypes.byref(routing_out) if routing_out is not None else None
    st = LIB.moe_forward_noalloc(ctypes.byref(p), ctypes.byref(w), ptr(x), ptr(logit_bias),
                                 ptr(sel_bias), ptr(modality), ptr(y), rout, _stream(stream))
    if raw:
        return st
    _check("moe_forward_noalloc", st)


def profile(events: dict, stages=STAGES) -> Profile:
    """Profile struct from {(stage_name, 0|1): torch.cuda.Event} (0 = before,
    1 = after); stages = STAGES (forward) or BSTAGES (backward).  Each event
    must already exist (record it once first)."""
    pr = Profile()
    for (name, which), ev in events.items():
        pr.ev[2 * stages.index(name) + which] = ev.cuda_event
    return pr
