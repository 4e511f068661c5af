"""ctypes binding of ``libmoe_mi355x.so`` (the C ABI in include/moe.h).

Argument marshalling only: torch supplies device memory and the stream; every
step of the layer runs in the library's HIP kernels.  There is no fallback: if
the library is missing or fails to load, importing the binding raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

from . import workloads as W

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_mi355x.so")

MOE_OK = 0
MOE_NOALLOC_SCRATCH_BYTES = 64 << 20  # the per-device scratch of moe_forward_noalloc
STATUS_NAMES = {0: "MOE_OK", 1: "MOE_ERR_INVALID_ARGUMENT", 2: "MOE_ERR_UNSUPPORTED",
                3: "MOE_ERR_WORKSPACE_TOO_SMALL", 4: "MOE_ERR_HIP"}

# every symbol include/moe.h declares
EXPORTED = ["moe_status_string", "moe_last_error", "moe_version", "moe_workspace_bytes",
            "moe_permuted_rows", "moe_route", "moe_permute", "moe_expert_ffn", "moe_combine",
            "moe_forward", "moe_forward_noalloc", "moe_router_stats", "moe_bias_update", "moe_profile_enable",
            "moe_profile_read"]


class MoEError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}: {detail}")
        self.status = status


class moe_config(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("d", ctypes.c_int32), ("E", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("F", ctypes.c_int32), ("n_shared", ctypes.c_int32),
                ("score", ctypes.c_int32), ("renormalize", ctypes.c_int32), ("tau", ctypes.c_float),
                ("bias_mode", ctypes.c_int32), ("capacity_factor", ctypes.c_float),
                ("act_dtype", ctypes.c_int32), ("w_dtype", ctypes.c_int32),
                ("out_dtype", ctypes.c_int32), ("reroute_depth", ctypes.c_int32),
                ("n_groups", ctypes.c_int32), ("topk_groups", ctypes.c_int32)]


class moe_expert_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ["w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down",
                 "sh_gate", "sh_up", "sh_down", "sh_s_gate", "sh_s_up", "sh_s_down"]]


class moe_routing_out(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ["logits", "topk_idx", "topk_w", "dest_row"]]


class moe_kernel_time(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 48), ("launches", ctypes.c_int32),
                ("total_ms", ctypes.c_double)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m mixture_experts_sparse_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    cfgp = ctypes.POINTER(moe_config)
    sigs = {
        "moe_status_string": ([ctypes.c_int], ctypes.c_char_p),
        "moe_last_error": ([], ctypes.c_char_p),
        "moe_version": ([], ctypes.c_int32),
        "moe_workspace_bytes": ([cfgp, ctypes.POINTER(ctypes.c_size_t)], ctypes.c_int),
        "moe_permuted_rows": ([cfgp, ctypes.POINTER(ctypes.c_int64)], ctypes.c_int),
        "moe_route": ([cfgp, P, P, P, P, P, P, P, P, ctypes.c_size_t, P], ctypes.c_int),
        "moe_permute": ([cfgp, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P], ctypes.c_int),
        "moe_expert_ffn": ([cfgp, P, P, P, ctypes.POINTER(moe_expert_weights), P, P, P,
                            ctypes.c_size_t, P], ctypes.c_int),
        "moe_combine": ([cfgp, P, P, P, P, P, P], ctypes.c_int),
        "moe_forward": ([cfgp, P, P, P, P, ctypes.POINTER(moe_expert_weights), P, P,
                         ctypes.POINTER(moe_routing_out), P, ctypes.c_size_t, P], ctypes.c_int),
        "moe_forward_noalloc": ([cfgp, P, P, P, P, ctypes.POINTER(moe_expert_weights), P, P,
                                 ctypes.POINTER(moe_routing_out), P], ctypes.c_int),
        "moe_router_stats": ([cfgp, P, P, P, P, P, P, P, ctypes.c_size_t, P], ctypes.c_int),
        "moe_bias_update": ([cfgp, P, P, ctypes.c_float, ctypes.c_float, P], ctypes.c_int),
        "moe_profile_enable": ([ctypes.c_int32], ctypes.c_int),
        "moe_profile_read": ([ctypes.POINTER(moe_kernel_time), ctypes.c_int32,
                              ctypes.POINTER(ctypes.c_int32)], ctypes.c_int),
    }
    for name, (args, res) in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


_LIB = _load()


def lib() -> ctypes.CDLL:
    return _LIB


def _check(status: int, where: str):
    if status != MOE_OK:
        detail = _LIB.moe_last_error().decode(errors="replace")
        raise MoEError(status, where, detail)


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to the MoE library must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


# ------------------------------------------------------------------ config helpers
def make_config(shape: W.MoEShape, out_dtype: Optional[int] = None) -> moe_config:
    return moe_config(shape.T, shape.d, shape.E, shape.k, shape.F, shape.n_shared, shape.score,
                      shape.renormalize, shape.tau, shape.bias_mode, shape.capacity_factor,
                      shape.act_dtype, shape.w_dtype,
                      shape.out_dtype if out_dtype is None else out_dtype, shape.reroute_depth,
                      shape.n_groups, shape.topk_groups)


def workspace_bytes(cfg: moe_config) -> int:
    n = ctypes.c_size_t(0)
    _check(_LIB.moe_workspace_bytes(ctypes.byref(cfg), ctypes.byref(n)), "moe_workspace_bytes")
    return n.value


def permuted_rows(cfg: moe_config) -> int:
    n = ctypes.c_int64(0)
    _check(_LIB.moe_permuted_rows(ctypes.byref(cfg), ctypes.byref(n)), "moe_permuted_rows")
    return n.value


def alloc_workspace(cfg: moe_config, device="cuda") -> torch.Tensor:
    """uint8 device buffer of moe_workspace_bytes(cfg) (torch allocations are 512-byte aligned)."""
    return torch.empty(max(workspace_bytes(cfg), 256), dtype=torch.uint8, device=device)


def expert_weights(inp: W.MoEInputs) -> moe_expert_weights:
    return moe_expert_weights(*[None if t is None else t.data_ptr() for t in (
        inp.w_gate, inp.w_up, inp.w_down, inp.s_gate, inp.s_up, inp.s_down,
        inp.sh_gate, inp.sh_up, inp.sh_down, inp.sh_s_gate, inp.sh_s_up, inp.sh_s_down)])


# ------------------------------------------------------------------ entry points
def moe_route(cfg, x, w_router, bias, gumbel_u, logits, topk_idx, topk_w, ws, stream=None):
    _check(_LIB.moe_route(ctypes.byref(cfg), _ptr(x), _ptr(w_router), _ptr(bias), _ptr(gumbel_u),
                          _ptr(logits), _ptr(topk_idx), _ptr(topk_w), _ptr(ws),
                          ws.numel() if ws is not None else 0, _stream(stream)), "moe_route")


def moe_permute(cfg, x, topk_idx, counts, offsets, dest_row, src_token, n_dropped, x_perm, ws,
                stream=None):
    _check(_LIB.moe_permute(ctypes.byref(cfg), _ptr(x), _ptr(topk_idx), _ptr(counts), _ptr(offsets),
                            _ptr(dest_row), _ptr(src_token), _ptr(n_dropped), _ptr(x_perm),
                            _ptr(ws), ws.numel() if ws is not None else 0, _stream(stream)),
           "moe_permute")


def moe_expert_ffn(cfg, x, x_perm, offsets, weights: moe_expert_weights, y_perm, y_shared, ws,
                   stream=None):
    _check(_LIB.moe_expert_ffn(ctypes.byref(cfg), _ptr(x), _ptr(x_perm), _ptr(offsets),
                               ctypes.byref(weights), _ptr(y_perm), _ptr(y_shared), _ptr(ws),
                               ws.numel() if ws is not None else 0, _stream(stream)),
           "moe_expert_ffn")


def moe_combine(cfg, y_perm, y_shared, dest_row, topk_w, out, stream=None):
    _check(_LIB.moe_combine(ctypes.byref(cfg), _ptr(y_perm), _ptr(y_shared), _ptr(dest_row),
                            _ptr(topk_w), _ptr(out), _stream(stream)), "moe_combine")


def moe_forward(cfg, x, w_router, bias, gumbel_u, weights: moe_expert_weights, out, stats, ws,
                routing: Optional[dict] = None, stream=None):
    r = None
    if routing:
        r = moe_routing_out(*[None if routing.get(k) is None else routing[k].data_ptr()
                              for k in ("logits", "topk_idx", "topk_w", "dest_row")])
    _check(_LIB.moe_forward(ctypes.byref(cfg), _ptr(x), _ptr(w_router), _ptr(bias), _ptr(gumbel_u),
                            ctypes.byref(weights), _ptr(out), _ptr(stats),
                            ctypes.byref(r) if r is not None else None, _ptr(ws),
                            ws.numel() if ws is not None else 0, _stream(stream)), "moe_forward")


def moe_forward_noalloc(cfg, x, w_router, bias, gumbel_u, weights: moe_expert_weights, out, stats,
                        routing: Optional[dict] = None, stream=None):
    """moe_forward with the library's per-device scratch instead of a workspace."""
    r = None
    if routing:
        r = moe_routing_out(*[None if routing.get(k) is None else routing[k].data_ptr()
                              for k in ("logits", "topk_idx", "topk_w", "dest_row")])
    _check(_LIB.moe_forward_noalloc(ctypes.byref(cfg), _ptr(x), _ptr(w_router), _ptr(bias), _ptr(gumbel_u),
                                    ctypes.byref(weights), _ptr(out), _ptr(stats),
                                    ctypes.byref(r) if r is not None else None, _stream(stream)),
           "moe_forward_noalloc")


def moe_router_stats(cfg, logits, bias, gumbel_u, counts, prob_mean, aux, ws, stream=None):
    _check(_LIB.moe_router_stats(ctypes.byref(cfg), _ptr(logits), _ptr(bias), _ptr(gumbel_u), _ptr(counts),
                                 _ptr(prob_mean), _ptr(aux), _ptr(ws), ws.numel() if ws is not None else 0,
                                 _stream(stream)), "moe_router_stats")


def moe_bias_update(cfg, counts, bias, decay: float = 0.99, rate: float = 0.01, stream=None):
    _check(_LIB.moe_bias_update(ctypes.byref(cfg), _ptr(counts), _ptr(bias), ctypes.c_float(decay),
                                ctypes.c_float(rate), _stream(stream)), "moe_bias_update")


def moe_profile_enable(on: bool):
    _check(_LIB.moe_profile_enable(1 if on else 0), "moe_profile_enable")


def moe_profile_read() -> dict:
    """{kernel name: (launches, total ms)} since the last read (synchronises its events)."""
    buf = (moe_kernel_time * 64)()
    n = ctypes.c_int32(0)
    _check(_LIB.moe_profile_read(buf, 64, ctypes.byref(n)), "moe_profile_read")
    return {buf[i].name.decode(): (buf[i].launches, buf[i].total_ms) for i in range(min(n.value, 64))}
