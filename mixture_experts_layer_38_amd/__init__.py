"""MI355X (gfx950) MoE layer forward pass: Python binding of libmoe.so.

The functions below carry the names of the C ABI in include/moe.h and do
argument marshalling only: every step of the layer runs in the HIP kernels of
libmoe.so.  Tensors are torch tensors on the GPU (torch supplies device memory
and the stream); optional arguments may be None.  The binding raises MoEError
for any non-OK status, and raises at import of the library when libmoe.so has
not been built (there is no fallback path).
"""
from __future__ import annotations

import ctypes
import os

from .configs import CONFIGS, MoEConfig

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe.so")

MOE_DTYPE_F32, MOE_DTYPE_BF16 = 0, 1
MOE_FLAG_BIAS_SELECT_ONLY, MOE_FLAG_COMBINE_MEAN = 1, 2

KERNEL_IDS = {
    "router": 0, "dispatch_count": 1, "dispatch_scan": 2, "dispatch_scatter": 3,
    "dispatch_gather": 4, "ffn_gate_up": 5, "ffn_down": 6, "combine": 7, "aux_loss": 8,
    "bias_update": 9, "ffn_plan": 10, "router_losses": 11, "ffn": 12,
}


class MoEError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib().moe_status_string(status).decode() if status >= 0 else "?"
        super().__init__(f"{where}: status {status} ({msg})")


class MoEProblem(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("d_model", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("d_ff", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("capacity", ctypes.c_int32), ("flags", ctypes.c_uint32)]


class MoEDebugOut(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "logits", "probs", "prob_sum", "topk_ids", "topk_w", "counts", "kept", "offsets",
        "assign_row", "row_assign", "z_loss", "aux_topk")]


_LIB = None


def _lib():
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m mixture_experts_layer_38_amd.build` (no fallback exists)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz, i32, f32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_float
    P = ctypes.POINTER(MoEProblem)
    sigs = {
        "moe_route_workspace_size": [P, ctypes.POINTER(sz)],
        "moe_dispatch_workspace_size": [P, ctypes.POINTER(sz)],
        "moe_expert_ffn_workspace_size": [P, ctypes.POINTER(sz)],
        "moe_workspace_size": [P, ctypes.POINTER(sz)],
        "moe_router_losses_workspace_size": [P, ctypes.POINTER(sz)],
        "moe_combine_concat_workspace_size": [P, ctypes.POINTER(sz)],
        "moe_forward_chunked_workspace_size": [P, ctypes.c_int32, ctypes.POINTER(sz)],
        "moe_forward_chunked": [P, ctypes.c_int32, vp, vp, vp, vp, vp, vp, vp,
                                ctypes.POINTER(MoEDebugOut), vp, sz, vp],
        "moe_router_losses": [P, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "moe_combine_concat": [P, vp, vp, vp, vp, vp, sz, vp],
        "moe_route": [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "moe_dispatch": [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "moe_expert_ffn": [P, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "moe_combine": [P, vp, vp, vp, vp, vp],
        "moe_forward": [P, vp, vp, vp, vp, vp, vp, vp, ctypes.POINTER(MoEDebugOut), vp, sz, vp],
        "moe_forward_noalloc": [P, vp, vp, vp, vp, vp, vp, vp, ctypes.POINTER(MoEDebugOut), vp],
        "moe_aux_loss": [P, vp, vp, vp, vp],
        "moe_bias_update": [P, vp, f32, vp, vp],
        "moe_set_kernel_timer": [i32, vp, vp, i32, ctypes.POINTER(i32)],
    }
    for name, args in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.moe_status_string.argtypes = [ctypes.c_int]
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_version.restype = ctypes.c_char_p
    lib.moe_kernel_name.argtypes = [ctypes.c_int]
    lib.moe_kernel_name.restype = ctypes.c_char_p
    _LIB = lib
    return lib


def load():
    """Load libmoe.so (raises when it is missing)."""
    return _lib()


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check(status: int, where: str):
    if status != 0:
        raise MoEError(status, where)


def problem(T: int, d_model: int, n_experts: int, top_k: int, d_ff: int, dtype: str = "bf16",
            capacity: int = -1, flags: int = 0) -> MoEProblem:
    code = {"f32": MOE_DTYPE_F32, "bf16": MOE_DTYPE_BF16}[dtype]
    return MoEProblem(T, d_model, n_experts, top_k, d_ff, code, capacity, flags)


def problem_of(cfg: MoEConfig, T: int | None = None) -> MoEProblem:
    return problem(cfg.T if T is None else T, cfg.d, cfg.E, cfg.K, cfg.F, cfg.dtype, cfg.capacity)


def _size(fn, p: MoEProblem) -> int:
    out = ctypes.c_size_t(0)
    _check(fn(ctypes.byref(p), ctypes.byref(out)), fn.__name__)
    return out.value


def moe_workspace_size(p: MoEProblem) -> int:
    return _size(_lib().moe_workspace_size, p)


def moe_route_workspace_size(p: MoEProblem) -> int:
    return _size(_lib().moe_route_workspace_size, p)


def moe_dispatch_workspace_size(p: MoEProblem) -> int:
    return _size(_lib().moe_dispatch_workspace_size, p)


def moe_expert_ffn_workspace_size(p: MoEProblem) -> int:
    return _size(_lib().moe_expert_ffn_workspace_size, p)


def moe_router_losses_workspace_size(p: MoEProblem) -> int:
    return _size(_lib().moe_router_losses_workspace_size, p)


def moe_route(p, x, w_router, logit_bias, logits, probs, prob_sum, topk_ids, topk_w,
              ws=None, stream=None):
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(_lib().moe_route(ctypes.byref(p), _ptr(x), _ptr(w_router), _ptr(logit_bias),
                            _ptr(logits), _ptr(probs), _ptr(prob_sum), _ptr(topk_ids),
                            _ptr(topk_w), _ptr(ws), ws_bytes, _stream(stream)), "moe_route")


def moe_dispatch(p, topk_ids, x, counts, kept, offsets, assign_row, row_assign, x_perm, ws,
                 stream=None):
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(_lib().moe_dispatch(ctypes.byref(p), _ptr(topk_ids), _ptr(x), _ptr(counts), _ptr(kept),
                               _ptr(offsets), _ptr(assign_row), _ptr(row_assign), _ptr(x_perm),
                               _ptr(ws), ws_bytes, _stream(stream)), "moe_dispatch")


def moe_expert_ffn(p, x_perm, offsets, w1, w3, w2, act, h, ws, stream=None):
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(_lib().moe_expert_ffn(ctypes.byref(p), _ptr(x_perm), _ptr(offsets), _ptr(w1), _ptr(w3),
                                 _ptr(w2), _ptr(act), _ptr(h), _ptr(ws), ws_bytes,
                                 _stream(stream)), "moe_expert_ffn")


def moe_combine(p, h, assign_row, topk_w, y, stream=None):
    _check(_lib().moe_combine(ctypes.byref(p), _ptr(h), _ptr(assign_row), _ptr(topk_w), _ptr(y),
                              _stream(stream)), "moe_combine")


def moe_forward(p, x, w_router, w1, w3, w2, logit_bias, y, ws, dbg: dict | None = None,
                stream=None):
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    d = None
    if dbg:
        d = MoEDebugOut(**{k: _ptr(v) for k, v in dbg.items()})
    _check(_lib().moe_forward(ctypes.byref(p), _ptr(x), _ptr(w_router), _ptr(w1), _ptr(w3),
                              _ptr(w2), _ptr(logit_bias), _ptr(y),
                              ctypes.byref(d) if d is not None else None, _ptr(ws), ws_bytes,
                              _stream(stream)), "moe_forward")


MOE_NOALLOC_WS_BYTES = 32 << 20


def moe_forward_noalloc(p, x, w_router, w1, w3, w2, logit_bias, y, dbg: dict | None = None, stream=None):
    """The layer on the library's static per-GPU workspace (no allocation)."""
    d = None
    if dbg:
        d = MoEDebugOut(**{k: _ptr(v) for k, v in dbg.items()})
    _check(_lib().moe_forward_noalloc(ctypes.byref(p), _ptr(x), _ptr(w_router), _ptr(w1), _ptr(w3),
                                      _ptr(w2), _ptr(logit_bias), _ptr(y),
                                      ctypes.byref(d) if d is not None else None, _stream(stream)),
           "moe_forward_noalloc")


def moe_forward_chunked_workspace_size(p: MoEProblem, chunk_tokens: int) -> int:
    out = ctypes.c_size_t(0)
    _check(_lib().moe_forward_chunked_workspace_size(ctypes.byref(p), chunk_tokens, ctypes.byref(out)),
           "moe_forward_chunked_workspace_size")
    return out.value


def moe_forward_chunked(p, chunk_tokens: int, x, w_router, w1, w3, w2, logit_bias, y, ws,
                        dbg: dict | None = None, stream=None):
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    d = None
    if dbg:
        d = MoEDebugOut(**{k: _ptr(v) for k, v in dbg.items()})
    _check(_lib().moe_forward_chunked(ctypes.byref(p), chunk_tokens, _ptr(x), _ptr(w_router), _ptr(w1),
                                      _ptr(w3), _ptr(w2), _ptr(logit_bias), _ptr(y),
                                      ctypes.byref(d) if d is not None else None, _ptr(ws), ws_bytes,
                                      _stream(stream)), "moe_forward_chunked")


def moe_aux_loss(p, counts, prob_sum, aux, stream=None):
    _check(_lib().moe_aux_loss(ctypes.byref(p), _ptr(counts), _ptr(prob_sum), _ptr(aux),
                               _stream(stream)), "moe_aux_loss")


def moe_combine_concat_workspace_size(p: MoEProblem) -> int:
    return _size(_lib().moe_combine_concat_workspace_size, p)


def moe_combine_concat(p, h, assign_row, w_cat, y, ws, stream=None):
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(_lib().moe_combine_concat(ctypes.byref(p), _ptr(h), _ptr(assign_row), _ptr(w_cat), _ptr(y),
                                     _ptr(ws), ws_bytes, _stream(stream)), "moe_combine_concat")


def moe_router_losses(p, logits, logit_bias, topk_ids, counts, z_loss, aux_topk, ws, stream=None):
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(_lib().moe_router_losses(ctypes.byref(p), _ptr(logits), _ptr(logit_bias), _ptr(topk_ids),
                                    _ptr(counts), _ptr(z_loss), _ptr(aux_topk), _ptr(ws), ws_bytes,
                                    _stream(stream)), "moe_router_losses")


def moe_bias_update(p, counts, alpha: float, bias, stream=None):
    _check(_lib().moe_bias_update(ctypes.byref(p), _ptr(counts), ctypes.c_float(alpha), _ptr(bias),
                                  _stream(stream)), "moe_bias_update")


def moe_set_kernel_timer(kernel: str | int, start_events, stop_events):
    """Bracket the next len(start_events) launches of `kernel` with the given
    torch.cuda.Event pairs (recorded on the kernel's own stream)."""
    kid = KERNEL_IDS[kernel] if isinstance(kernel, str) else kernel
    n = len(start_events)
    if n == 0:
        _check(_lib().moe_set_kernel_timer(kid, None, None, 0, None), "moe_set_kernel_timer")
        return None
    arr_t = ctypes.c_void_p * n
    starts = arr_t(*[e.cuda_event for e in start_events])
    stops = arr_t(*[e.cuda_event for e in stop_events])
    _check(_lib().moe_set_kernel_timer(kid, starts, stops, n, None), "moe_set_kernel_timer")
    return (starts, stops)  # caller keeps these alive while the hook is set


def moe_kernel_timer_count(kernel: str | int) -> int:
    kid = KERNEL_IDS[kernel] if isinstance(kernel, str) else kernel
    out = ctypes.c_int(0)
    _check(_lib().moe_set_kernel_timer(kid, None, None, -1, ctypes.byref(out)), "moe_set_kernel_timer")
    return out.value


__all__ = [
    "CONFIGS", "MoEConfig", "MoEError", "MoEProblem", "MoEDebugOut", "load", "problem", "problem_of",
    "moe_workspace_size", "moe_route_workspace_size", "moe_dispatch_workspace_size",
    "moe_expert_ffn_workspace_size", "moe_route", "moe_dispatch", "moe_expert_ffn", "moe_combine",
    "moe_forward", "moe_forward_chunked", "moe_forward_chunked_workspace_size", "moe_aux_loss", "moe_bias_update", "moe_router_losses",
    "moe_combine_concat", "moe_combine_concat_workspace_size",
    "moe_router_losses_workspace_size", "moe_set_kernel_timer",
    "moe_kernel_timer_count",
]
