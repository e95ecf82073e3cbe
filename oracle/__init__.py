"""CPU oracle of the routed mixture-of-experts layer -- TEST INFRASTRUCTURE ONLY.

Thin ctypes wrapper over ``moe_oracle.c`` (plain fp64 C).  Only ``tests/``,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import
this package; the product library never loads it and has no fallback to it.

Inputs are the host byte arrays drawn by :mod:`synth`; outputs are fp64 (or
int32 for indices and counts).
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "libmoe_oracle.so")

# Names of the deliberate mistakes the C file can switch on (for pin-strength tests).
MUTANTS = {
    1: "topk-softmax divides by the all-expert sum",
    2: "SiLU applied to up instead of gate",
    3: "logit bias ignored by the top-k",
    4: "ties go to the higher expert id",
    5: "clamp applied to the gate only",
    6: "down projection read transposed",
    7: "softmax-over-all mode renormalises",
    8: "shared expert dropped",
    9: "RMS pre-norm uses the sum, not the mean",
    10: "permutation not stable",
    11: "Q8_0 reads the next block's scale",
    12: "SiLU sign flipped",
    13: "combine ignores the routing weights",
    14: "selection-only bias leaks into the softmax",
    15: "gate clamped from above only",
    16: "pre-norm applied to the router input only",
    17: "sigmoid mode adds the correction bias to the logit",
    18: "sigmoid mode leaves the weights unnormalised",
    19: "MXFP4 element 2j read from the high nibble",
    20: "MXFP4 scale exponent bias 128",
    21: "MXFP4 exponent field 0 given an implicit one",
    22: "MXFP4 reads the next block's scale",
    23: "norm weight applied to the router input only",
    24: "residual stream not added",
    25: "router input scale ignored",
    26: "router input scale applied to the experts too",
}


class _Layer(ctypes.Structure):
    _fields_ = [
        ("hidden", ctypes.c_int), ("num_experts", ctypes.c_int), ("top_k", ctypes.c_int),
        ("expert_inter", ctypes.c_int), ("shared_inter", ctypes.c_int),
        ("select", ctypes.c_int), ("bias_mode", ctypes.c_int),
        ("swiglu_limit", ctypes.c_double), ("rms_eps", ctypes.c_double),
        ("x_fmt", ctypes.c_int), ("router_fmt", ctypes.c_int),
        ("expert_fmt", ctypes.c_int), ("shared_fmt", ctypes.c_int),
    ]


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O2, OpenMP) into ``oracle/libmoe_oracle.so``."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                        "-Wall", "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        L.orc_forward.argtypes = [ctypes.POINTER(_Layer), ctypes.c_int] + [P] * 16
        L.orc_forward_fused.argtypes = [ctypes.POINTER(_Layer), ctypes.c_int] + [P] * 19
        L.orc_forward.restype = ctypes.c_int
        L.orc_select.argtypes = [ctypes.POINTER(_Layer), ctypes.c_int, P, P, P, P, P]
        L.orc_route.argtypes = [ctypes.POINTER(_Layer), ctypes.c_int] + [P] * 8
        L.orc_route.restype = ctypes.c_int
        L.orc_permute.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P, P, P, P]
        L.orc_element.argtypes = [P, ctypes.c_int, ctypes.c_longlong, ctypes.c_longlong,
                                  ctypes.c_longlong]
        L.orc_element.restype = ctypes.c_double
        L.orc_down.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, P, ctypes.c_int, P, P]
        L.orc_set_mutant.argtypes = [ctypes.c_int]
        L.orc_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def layer_struct(spec) -> _Layer:
    return _Layer(spec.hidden, spec.num_experts, spec.top_k, spec.expert_inter,
                  spec.shared_inter, spec.select, spec.bias_mode, float(spec.swiglu_limit),
                  float(spec.rms_eps), spec.x_dtype, spec.router_dtype, spec.expert_dtype,
                  spec.shared_dtype)


def forward(spec, layer: Dict[str, Optional[np.ndarray]], x: np.ndarray,
            forced_ids: Optional[np.ndarray] = None, want_act: bool = False,
            norm_w: Optional[np.ndarray] = None,
            residual: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """Run the whole layer on ``x [M][H]``; returns logits, ids, w, counts, y (and act).

    ``norm_w`` (``[H]`` in the x storage format) weights the RMS pre-norm
    (needs ``spec.rms_eps > 0``); ``residual`` (``[M][H]`` fp32) is added to y.
    ``layer["router_x_scale"]`` (bf16 bits ``[H]``, optional) scales the
    router's input element by element."""
    M = x.shape[0]
    E, k, H, I = spec.num_experts, spec.top_k, spec.hidden, spec.expert_inter
    out = {
        "logits": np.zeros((M, E), np.float64),
        "ids": np.zeros((M, k), np.int32),
        "w": np.zeros((M, k), np.float64),
        "counts": np.zeros(E, np.int32),
        "y": np.zeros((M, H), np.float64),
    }
    act = np.zeros((M * k, I), np.float64) if want_act else None
    fids = None if forced_ids is None else np.ascontiguousarray(forced_ids, np.int32)
    bias = layer.get("bias")
    bias = None if bias is None else np.ascontiguousarray(bias, np.float32)
    st = layer_struct(spec)
    nw = None if norm_w is None else np.ascontiguousarray(norm_w)
    res = None if residual is None else np.ascontiguousarray(residual, np.float32)
    rxs = layer.get("router_x_scale")
    rxs = None if rxs is None else np.ascontiguousarray(rxs, np.uint16)
    rc = lib().orc_forward_fused(
        ctypes.byref(st), M, _ptr(np.ascontiguousarray(x)), _ptr(nw), _ptr(res),
        _ptr(layer["router"]), _ptr(rxs), _ptr(bias),
        _ptr(layer["gate"]), _ptr(layer["up"]), _ptr(layer["down"]),
        _ptr(layer.get("shared_gate")), _ptr(layer.get("shared_up")),
        _ptr(layer.get("shared_down")), _ptr(fids), _ptr(out["logits"]), _ptr(out["ids"]),
        _ptr(out["w"]), _ptr(out["counts"]), _ptr(act), _ptr(out["y"]))
    if rc != 0:
        raise ValueError("oracle refused the layer shape")
    if want_act:
        out["act"] = act
    return out


def route(spec, layer: Dict[str, Optional[np.ndarray]], x: np.ndarray,
          norm_w: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """The routing half of :func:`forward` for every token of ``x [M][H]``:
    logits, ids and w, as ``forward`` computes them (no expert work)."""
    M = x.shape[0]
    E, k = spec.num_experts, spec.top_k
    out = {"logits": np.zeros((M, E), np.float64), "ids": np.zeros((M, k), np.int32),
           "w": np.zeros((M, k), np.float64)}
    bias = layer.get("bias")
    bias = None if bias is None else np.ascontiguousarray(bias, np.float32)
    nw = None if norm_w is None else np.ascontiguousarray(norm_w)
    rxs = layer.get("router_x_scale")
    rxs = None if rxs is None else np.ascontiguousarray(rxs, np.uint16)
    st = layer_struct(spec)
    rc = lib().orc_route(ctypes.byref(st), M, _ptr(np.ascontiguousarray(x)), _ptr(nw),
                         _ptr(layer["router"]), _ptr(rxs), _ptr(bias), _ptr(out["logits"]),
                         _ptr(out["ids"]), _ptr(out["w"]))
    if rc != 0:
        raise ValueError("oracle refused the layer shape")
    return out


def select(spec, logits: np.ndarray, bias: Optional[np.ndarray] = None,
           forced_ids: Optional[np.ndarray] = None):
    """Bias, top-k and weights from given logits ``[M][E]`` (converted exactly to fp64)."""
    logits = np.ascontiguousarray(logits, np.float64)
    M = logits.shape[0]
    ids = np.zeros((M, spec.top_k), np.int32)
    w = np.zeros((M, spec.top_k), np.float64)
    b = None if bias is None else np.ascontiguousarray(bias, np.float32)
    f = None if forced_ids is None else np.ascontiguousarray(forced_ids, np.int32)
    st = layer_struct(spec)
    lib().orc_select(ctypes.byref(st), M, _ptr(logits), _ptr(b), _ptr(f), _ptr(ids), _ptr(w))
    return ids, w


def permute(E: int, ids: np.ndarray):
    """Counting sort of the routes by expert: counts, offsets, sorted_routes, route_pos."""
    ids = np.ascontiguousarray(ids, np.int32)
    M, k = ids.shape
    counts = np.zeros(E, np.int32)
    offsets = np.zeros(E + 1, np.int32)
    sr = np.zeros(M * k, np.int32)
    rp = np.zeros(M * k, np.int32)
    lib().orc_permute(E, M, k, _ptr(ids), _ptr(counts), _ptr(offsets), _ptr(sr), _ptr(rp))
    return counts, offsets, sr, rp


def down(spec, layer: Dict[str, Optional[np.ndarray]], e: int, act_row: np.ndarray) -> np.ndarray:
    """Expert ``e``'s down projection of one act row ``[I]`` (fp64): ``[H]``."""
    out = np.zeros(spec.hidden, np.float64)
    a = np.ascontiguousarray(act_row, np.float64)
    lib().orc_down(spec.hidden, spec.expert_inter, spec.expert_dtype, _ptr(layer["down"]), int(e), _ptr(a),
                   _ptr(out))
    return out


def element(buf: np.ndarray, fmt: int, r: int, cols: int, c: int) -> float:
    return lib().orc_element(_ptr(np.ascontiguousarray(buf)), fmt, r, cols, c)


def set_mutant(m: int) -> None:
    lib().orc_set_mutant(int(m))


def threads() -> int:
    return int(lib().orc_threads())
