"""Python binding of the MI355X routed mixture-of-experts layer.

Argument marshalling only: every function here has the name of a C entry point
of ``include/moe_gemv.h`` and passes its arguments through to
``libmoe_gemv.so`` (built by :mod:`mixture_experts_gemv_amd.build`).  Device
buffers are PyTorch tensors (or raw integer device addresses); PyTorch is used
for device memory and streams only.  There is no fallback: if the library is
missing, importing a function raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_gemv.so")

MOE_OK, MOE_ERR_INVALID, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_F32, MOE_BF16, MOE_Q8_0, MOE_MXFP4 = 0, 1, 2, 3
MOE_TOPK_SOFTMAX, MOE_SOFTMAX_ALL_NORENORM, MOE_SIGMOID_NORM = 0, 1, 2
MOE_BIAS_NONE, MOE_BIAS_LOGIT, MOE_BIAS_SELECT_ONLY = 0, 1, 2
MOE_PATH_AUTO, MOE_PATH_GEMV, MOE_PATH_MFMA = 0, 1, 2
MOE_LOGITS_IN = 1

_STATUS = {0: "MOE_OK", 1: "MOE_ERR_INVALID", 2: "MOE_ERR_UNSUPPORTED",
           3: "MOE_ERR_WORKSPACE", 4: "MOE_ERR_HIP"}


class MoeError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status
        self.message = message


class moe_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "hidden", "num_experts", "top_k", "expert_inter", "shared_inter", "max_tokens",
        "select", "bias_mode")] + [("swiglu_limit", ctypes.c_float), ("rms_eps", ctypes.c_float)] + [
        (n, ctypes.c_int32) for n in ("x_dtype", "router_dtype", "expert_dtype", "shared_dtype", "path")]


_WEIGHT_FIELDS = ("router", "bias", "gate", "up", "down", "gate_scale", "up_scale", "down_scale",
                  "shared_gate", "shared_up", "shared_down", "shared_gate_scale",
                  "shared_up_scale", "shared_down_scale", "router_scale", "router_x_scale")


class moe_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in _WEIGHT_FIELDS]


_lib = None


def lib() -> ctypes.CDLL:
    """Load ``libmoe_gemv.so``; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing; build it with "
                              "`python -m mixture_experts_gemv_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        L.moe_plan_create.argtypes = [ctypes.POINTER(moe_config), ctypes.POINTER(P)]
        L.moe_plan_create.restype = I32
        L.moe_plan_destroy.argtypes = [P]
        L.moe_plan_destroy.restype = None
        L.moe_workspace_bytes.argtypes = [P, I32]
        L.moe_workspace_bytes.restype = SZ
        L.moe_last_error.argtypes = []
        L.moe_last_error.restype = ctypes.c_char_p
        W = ctypes.POINTER(moe_weights)
        L.moe_route.argtypes = [P, P, W, I32, P, I32, P, P, P, SZ, P]
        L.moe_permute.argtypes = [P, P, I32, P, P, P, P, P, SZ, P]
        L.moe_expert_ffn.argtypes = [P, P, W, I32, P, P, P, P, SZ, P]
        L.moe_combine.argtypes = [P, P, W, I32, P, P, P, P, P, P, P, SZ, P]
        L.moe_forward.argtypes = [P, P, W, I32, P, P, P, P, P, SZ, P]
        L.moe_forward_fused.argtypes = [P, P, P, P, W, I32, P, P, P, P, P, SZ, P]
        L.moe_forward_noalloc.argtypes = [P, P, W, I32, P, P, P, P, P]
        L.moe_forward_timed.argtypes = [P, P, W, I32, P, P, P, P, P, SZ, P,
                                        ctypes.POINTER(P), I32, P, ctypes.POINTER(I32)]
        L.moe_q8_0_split.argtypes = [P, ctypes.c_int64, I32, P, P, P]
        L.moe_mxfp4_split.argtypes = [P, ctypes.c_int64, I32, P, P, P]
        L.moe_forward_path.argtypes = [P, I32]
        L.moe_forward_path.restype = I32
        for f in ("moe_route", "moe_permute", "moe_expert_ffn", "moe_combine", "moe_forward", "moe_forward_fused",
                  "moe_forward_noalloc",
                  "moe_forward_timed", "moe_q8_0_split", "moe_mxfp4_split"):
            getattr(L, f).restype = I32
        _lib = L
    return _lib


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("device buffers must be GPU tensors")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int) -> None:
    if status != MOE_OK:
        raise MoeError(status, lib().moe_last_error().decode())


def _nbytes(ws) -> int:
    return ws.numel() * ws.element_size() if ws is not None and not isinstance(ws, int) else 0


class Plan:
    """Owns a ``moe_plan*``."""

    def __init__(self, handle: int, cfg: moe_config):
        self.handle = handle
        self.cfg = cfg

    def __del__(self):
        if self.handle and _lib is not None:
            _lib.moe_plan_destroy(self.handle)
            self.handle = None


def make_weights(**tensors) -> moe_weights:
    """Build a ``moe_weights`` struct from tensors (unknown names raise)."""
    bad = set(tensors) - set(_WEIGHT_FIELDS)
    if bad:
        raise KeyError(f"unknown weight fields {sorted(bad)}")
    return moe_weights(*[_ptr(tensors.get(n)) for n in _WEIGHT_FIELDS])


def moe_plan_create(hidden, num_experts, top_k, expert_inter, shared_inter=0, max_tokens=1,
                    select=MOE_TOPK_SOFTMAX, bias_mode=MOE_BIAS_NONE, swiglu_limit=0.0,
                    rms_eps=0.0, x_dtype=MOE_BF16, router_dtype=MOE_BF16,
                    expert_dtype=MOE_BF16, shared_dtype=MOE_BF16, path=MOE_PATH_AUTO) -> Plan:
    cfg = moe_config(hidden, num_experts, top_k, expert_inter, shared_inter, max_tokens, select,
                     bias_mode, swiglu_limit, rms_eps, x_dtype, router_dtype, expert_dtype,
                     shared_dtype, path)
    h = ctypes.c_void_p()
    _check(lib().moe_plan_create(ctypes.byref(cfg), ctypes.byref(h)))
    return Plan(h.value, cfg)


def moe_plan_destroy(plan: Plan) -> None:
    if plan.handle:
        lib().moe_plan_destroy(plan.handle)
        plan.handle = None


def moe_workspace_bytes(plan: Plan, M: int) -> int:
    return int(lib().moe_workspace_bytes(plan.handle, M))


def moe_last_error() -> str:
    return lib().moe_last_error().decode()


def moe_route(plan, x, weights, M, logits, flags, ids, w, ws, stream=None):
    _check(lib().moe_route(plan.handle, _ptr(x), ctypes.byref(weights), M, _ptr(logits), flags,
                           _ptr(ids), _ptr(w), _ptr(ws), _nbytes(ws), _stream(stream)))


def moe_permute(plan, ids, M, counts, offsets, sorted_routes, route_pos, ws, stream=None):
    _check(lib().moe_permute(plan.handle, _ptr(ids), M, _ptr(counts), _ptr(offsets),
                             _ptr(sorted_routes), _ptr(route_pos), _ptr(ws), _nbytes(ws),
                             _stream(stream)))


def moe_expert_ffn(plan, x, weights, M, offsets, sorted_routes, act, ws, stream=None):
    _check(lib().moe_expert_ffn(plan.handle, _ptr(x), ctypes.byref(weights), M, _ptr(offsets),
                                _ptr(sorted_routes), _ptr(act), _ptr(ws), _nbytes(ws),
                                _stream(stream)))


def moe_combine(plan, act, weights, M, offsets, sorted_routes, route_pos, w, seed, y, ws,
                stream=None):
    _check(lib().moe_combine(plan.handle, _ptr(act), ctypes.byref(weights), M, _ptr(offsets),
                             _ptr(sorted_routes), _ptr(route_pos), _ptr(w), _ptr(seed), _ptr(y),
                             _ptr(ws), _nbytes(ws), _stream(stream)))


def moe_forward(plan, x, weights, M, y, ids_out, w_out, counts_out, ws, stream=None):
    _check(lib().moe_forward(plan.handle, _ptr(x), ctypes.byref(weights), M, _ptr(y),
                             _ptr(ids_out), _ptr(w_out), _ptr(counts_out), _ptr(ws), _nbytes(ws),
                             _stream(stream)))


def moe_forward_noalloc(plan, x, weights, M, y, ids_out, w_out, counts_out, stream=None):
    _check(lib().moe_forward_noalloc(plan.handle, _ptr(x), ctypes.byref(weights), M, _ptr(y),
                                     _ptr(ids_out), _ptr(w_out), _ptr(counts_out), _stream(stream)))


def moe_forward_fused(plan, x, norm_weight, residual, weights, M, y, ids_out, w_out, counts_out, ws,
                      stream=None):
    _check(lib().moe_forward_fused(plan.handle, _ptr(x), _ptr(norm_weight), _ptr(residual),
                                   ctypes.byref(weights), M, _ptr(y), _ptr(ids_out), _ptr(w_out),
                                   _ptr(counts_out), _ptr(ws), _nbytes(ws), _stream(stream)))


MOE_STAGE_NAMES = ("rms", "router", "topk", "permute", "gateup", "down", "combine")
MOE_RUN_NAMES = ("single", "gemv", "mfma")


def moe_forward_path(plan, M) -> int:
    """moe_run value (0 single, 1 gemv, 2 mfma) of an M-token moe_forward."""
    r = lib().moe_forward_path(plan.handle, M)
    if r < 0:
        raise MoeError(1, lib().moe_last_error().decode())
    return r


def moe_forward_timed(plan, x, weights, M, y, ids_out, w_out, counts_out, ws, events,
                      stream=None):
    """``events``: sequence of hipEvent_t handles (ints).  Returns the stage ids."""
    n = len(events)
    ev = (ctypes.c_void_p * n)(*events)
    stages = (ctypes.c_int32 * n)()
    n_st = ctypes.c_int32(0)
    _check(lib().moe_forward_timed(plan.handle, _ptr(x), ctypes.byref(weights), M, _ptr(y),
                                   _ptr(ids_out), _ptr(w_out), _ptr(counts_out), _ptr(ws),
                                   _nbytes(ws), _stream(stream), ev, n,
                                   ctypes.cast(stages, ctypes.c_void_p), ctypes.byref(n_st)))
    return [int(stages[i]) for i in range(n_st.value)]


def moe_q8_0_split(blocks, rows, cols, qs, scales, stream=None):
    _check(lib().moe_q8_0_split(_ptr(blocks), rows, cols, _ptr(qs), _ptr(scales),
                                _stream(stream)))


def moe_mxfp4_split(blocks, rows, cols, codes, scales, stream=None):
    _check(lib().moe_mxfp4_split(_ptr(blocks), rows, cols, _ptr(codes), _ptr(scales),
                                 _stream(stream)))
