"""Seeded synthetic inputs for the routed mixture-of-experts layer.

This module is shared by the CPU oracle's tests and the HIP path's tests and
bench. It only draws random numbers and stores them in the byte formats the
layer reads (fp32, bf16, Q8_0 and MXFP4 blocks); it holds none of the
layer's arithmetic.

Byte formats produced here:

* bf16 tensors are ``uint16`` arrays of bf16 bit patterns, drawn in fp32 and
  rounded to nearest-even.
* Q8_0 tensors are ``uint8`` arrays of 34-byte blocks, one block per 32
  consecutive elements along the reduction dimension: a little-endian fp16
  scale ``d`` followed by 32 int8 values ``q`` (value = d * q).  This is the
  GGUF block the turbospark-runtime pages name for their Q8_0 MoE kernels
  (``src/families/deepseek2/state.rs``, ``RealDeepseek2State::build``, the
  kernel-contract check that the dots walk whole 32-element blocks).
* MXFP4 tensors are ``uint8`` arrays of 17-byte blocks, one block per 32
  consecutive elements along the reduction dimension: the E8M0 scale byte,
  then 16 bytes of 4-bit E2M1 codes, byte j holding element 2j in its low
  nibble and element 2j+1 in its high nibble (OCP Microscaling v1.0 element
  and scale formats; the block layout is a reading, the pages name the format
  for gpt-oss's routed experts without giving bytes).
* Layer tensors are row-major with the reduction dimension contiguous:
  router ``[E][H]``, gate and up ``[E][I][H]``, down ``[E][H][I]``, shared
  gate and up ``[Is][H]``, shared down ``[H][Is]``.

Seeding: each workload has an integer seed; ``numpy.random.SeedSequence(seed)``
is spawned into named child streams in the fixed order of ``STREAMS``.  Expert
tensors spawn one grandchild stream per expert so that large layers can be drawn
on several threads and still come out identical.
"""

from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import math
import os
from typing import Dict, Optional

import numpy as np

F32, BF16, Q8_0, MXFP4 = 0, 1, 2, 3
TOPK_SOFTMAX, SOFTMAX_ALL_NORENORM, SIGMOID_NORM = 0, 1, 2
BIAS_NONE, BIAS_LOGIT, BIAS_SELECT_ONLY = 0, 1, 2

STREAMS = ("x", "router", "bias", "gate", "up", "down", "shared_gate",
           "shared_up", "shared_down", "zipf_perm", "q8_scale", "router_x_scale")

Q8_BLOCK = 32
Q8_BYTES = 34
MX_BLOCK = 32
MX_BYTES = 17


@dataclasses.dataclass(frozen=True)
class LayerSpec:
    """Shape, modes and value distributions of one synthetic MoE layer."""
    name: str
    hidden: int
    num_experts: int
    top_k: int
    expert_inter: int
    shared_inter: int = 0
    select: int = TOPK_SOFTMAX
    bias_mode: int = BIAS_NONE
    bias_kind: str = "none"        # "none" | "normal" | "zipf"
    bias_std: float = 0.1
    zipf_s: float = 1.1
    swiglu_limit: float = 0.0
    rms_eps: float = 0.0
    x_dtype: int = BF16
    router_dtype: int = BF16
    expert_dtype: int = BF16
    shared_dtype: int = BF16
    weight_std: float = 0.02
    q8_scale_lo: float = 1e-4
    q8_scale_hi: float = 1e-3
    mx_exp_lo: int = 118           # MXFP4 scale byte ~ U{lo..hi}: 2^-9 .. 2^-5
    mx_exp_hi: int = 122
    router_x_scale: str = "none"   # "none" | "uniform": bf16 [H] ~ U[0.5, 1.5], the router's input scale
    seed: int = 1000
    token_counts: tuple = (1,)

    def replace(self, **kw) -> "LayerSpec":
        return dataclasses.replace(self, **kw)


# The workloads: a tiny fp32 layer and layers shaped like public MoE models
# (no trained weights; every value is drawn here).
SPECS: Dict[str, LayerSpec] = {
    "tiny": LayerSpec(
        name="tiny", hidden=256, num_experts=8, top_k=2, expert_inter=512,
        x_dtype=F32, router_dtype=F32, expert_dtype=F32, shared_dtype=F32,
        seed=1001, token_counts=(4,)),
    "gpt-oss-20b": LayerSpec(
        name="gpt-oss-20b", hidden=2880, num_experts=32, top_k=4,
        expert_inter=2880, bias_mode=BIAS_LOGIT, bias_kind="normal",
        bias_std=0.1, swiglu_limit=7.0, expert_dtype=Q8_0, seed=1002,
        token_counts=(1, 16)),
    "deepseek-v2-lite": LayerSpec(
        name="deepseek-v2-lite", hidden=2048, num_experts=64, top_k=6,
        expert_inter=1408, shared_inter=2816, select=SOFTMAX_ALL_NORENORM,
        seed=1003, token_counts=(1, 16)),
    "mixtral-8x7b": LayerSpec(
        name="mixtral-8x7b", hidden=4096, num_experts=8, top_k=2,
        expert_inter=14336, seed=1004, token_counts=(1, 16, 512)),
    "qwen3-30b-a3b": LayerSpec(
        name="qwen3-30b-a3b", hidden=2048, num_experts=128, top_k=8,
        expert_inter=768, bias_mode=BIAS_LOGIT, bias_kind="zipf",
        rms_eps=1e-6, seed=1005, token_counts=(2048,)),
    # the dense lead layer of the DeepSeek-V2-Lite shape (layer 0: one dense
    # SwiGLU 10944 wide), run as the one-expert, top-1 case of the same path
    "deepseek-v2-lite-dense": LayerSpec(
        name="deepseek-v2-lite-dense", hidden=2048, num_experts=1, top_k=1,
        expert_inter=10944, seed=1006, token_counts=(1, 16, 512)),
    # sigmoid scoring with a selection-only correction bias and an fp32 router,
    # as the pages' MiniMax branch requires; the shape (not on the pages) is
    # chosen at the ABI's 256-expert limit
    "sigmoid-e256": LayerSpec(
        name="sigmoid-e256", hidden=3072, num_experts=256, top_k=8,
        expert_inter=1536, select=SIGMOID_NORM, bias_mode=BIAS_SELECT_ONLY,
        bias_kind="normal", bias_std=0.05, router_dtype=F32, seed=1007,
        token_counts=(1, 16)),
    # the gpt-oss-20B shape with an INT8 router: Q8_0 router rows and a
    # per-element bf16 scale of the router's input, the router form of the
    # pages' INT8 router kernels (the scale drawn U[0.5, 1.5] rather than the
    # pages' identically-one, so that it matters)
    "gpt-oss-20b-int8-router": LayerSpec(
        name="gpt-oss-20b-int8-router", hidden=2880, num_experts=32, top_k=4,
        expert_inter=2880, bias_mode=BIAS_LOGIT, bias_kind="normal",
        bias_std=0.1, swiglu_limit=7.0, expert_dtype=Q8_0, router_dtype=Q8_0,
        router_x_scale="uniform", seed=1009, token_counts=(1, 16, 64)),
    # the gpt-oss-20B shape with its routed experts in MXFP4, the format the
    # pages name for gpt-oss's routed pair (scale bytes 2^-9..2^-5 give weights
    # of about the Q8_0 layer's magnitude)
    "gpt-oss-20b-mxfp4": LayerSpec(
        name="gpt-oss-20b-mxfp4", hidden=2880, num_experts=32, top_k=4,
        expert_inter=2880, bias_mode=BIAS_LOGIT, bias_kind="normal",
        bias_std=0.1, swiglu_limit=7.0, expert_dtype=MXFP4, seed=1008,
        token_counts=(1, 16)),
}

_NTHREADS = max(1, min(16, len(os.sched_getaffinity(0))))


def _children(seed: int) -> Dict[str, np.random.SeedSequence]:
    kids = np.random.SeedSequence(seed).spawn(len(STREAMS))
    return dict(zip(STREAMS, kids))


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); return the bits."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    return ((b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1)))
            >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def q8_row_bytes(cols: int) -> int:
    return cols // Q8_BLOCK * Q8_BYTES


def q8_pack(q: np.ndarray, d_f16: np.ndarray) -> np.ndarray:
    """Pack int8 values ``q [rows][cols]`` and fp16 scales ``d [rows][cols/32]``
    into 34-byte blocks ``[rows][cols/32*34]`` (uint8)."""
    rows, cols = q.shape
    nb = cols // Q8_BLOCK
    out = np.empty((rows, nb, Q8_BYTES), dtype=np.uint8)
    out[:, :, 0:2] = np.ascontiguousarray(d_f16, dtype=np.float16).view(
        np.uint8).reshape(rows, nb, 2)
    out[:, :, 2:] = q.astype(np.int8).view(np.uint8).reshape(rows, nb, Q8_BLOCK)
    return out.reshape(rows, nb * Q8_BYTES)


def q8_unpack(blocks: np.ndarray, cols: int):
    """Split 34-byte blocks back into ``(q int8 [rows][cols], d fp16 [rows][cols/32])``."""
    rows = blocks.shape[0]
    nb = cols // Q8_BLOCK
    b = np.ascontiguousarray(blocks).reshape(rows, nb, Q8_BYTES)
    d = np.ascontiguousarray(b[:, :, 0:2]).view(np.float16).reshape(rows, nb)
    q = np.ascontiguousarray(b[:, :, 2:]).view(np.int8).reshape(rows, cols)
    return q, d


def mx_row_bytes(cols: int) -> int:
    return cols // MX_BLOCK * MX_BYTES


def mx_pack(codes: np.ndarray, e8: np.ndarray) -> np.ndarray:
    """Pack 4-bit codes ``[rows][cols]`` (values 0..15) and E8M0 scale bytes
    ``[rows][cols/32]`` into 17-byte blocks ``[rows][cols/32*17]`` (uint8)."""
    rows, cols = codes.shape
    nb = cols // MX_BLOCK
    c = np.asarray(codes, dtype=np.uint8).reshape(rows, nb, MX_BLOCK // 2, 2)
    out = np.empty((rows, nb, MX_BYTES), dtype=np.uint8)
    out[:, :, 0] = np.asarray(e8, dtype=np.uint8).reshape(rows, nb)
    out[:, :, 1:] = (c[..., 0] & np.uint8(15)) | ((c[..., 1] & np.uint8(15)) << np.uint8(4))
    return out.reshape(rows, nb * MX_BYTES)


def mx_unpack(blocks: np.ndarray, cols: int):
    """Split 17-byte blocks back into ``(codes uint8 [rows][cols], e8 uint8 [rows][cols/32])``."""
    rows = blocks.shape[0]
    nb = cols // MX_BLOCK
    b = np.ascontiguousarray(blocks).reshape(rows, nb, MX_BYTES)
    e8 = np.ascontiguousarray(b[:, :, 0])
    q = b[:, :, 1:]
    codes = np.stack([q & np.uint8(15), q >> np.uint8(4)], axis=-1).reshape(rows, cols)
    return codes, e8


def _draw_matrix(ss: np.random.SeedSequence, rows: int, cols: int, dtype: int,
                 std: float, scale_ss: Optional[np.random.SeedSequence],
                 lo: float, hi: float, mx_exp=(118, 122)) -> np.ndarray:
    rng = np.random.default_rng(ss)
    if dtype == MXFP4:
        if cols % MX_BLOCK:
            raise ValueError("MXFP4 rows must hold whole 32-element blocks")
        codes = rng.integers(0, 16, size=(rows, cols), dtype=np.uint8)
        e8 = np.random.default_rng(scale_ss).integers(mx_exp[0], mx_exp[1] + 1,
                                                       size=(rows, cols // MX_BLOCK), dtype=np.uint8)
        return mx_pack(codes, e8)
    if dtype == Q8_0:
        if cols % Q8_BLOCK:
            raise ValueError("Q8_0 rows must hold whole 32-element blocks")
        q = rng.integers(-127, 128, size=(rows, cols), dtype=np.int8)
        srng = np.random.default_rng(scale_ss)
        d = srng.uniform(lo, hi, size=(rows, cols // Q8_BLOCK)).astype(np.float16)
        return q8_pack(q, d)
    w = rng.standard_normal((rows, cols), dtype=np.float32)
    w *= np.float32(std)
    if dtype == BF16:
        return bf16_bits(w)
    if dtype == F32:
        return w
    raise ValueError(f"unknown dtype {dtype}")


def _draw_experts(ss: np.random.SeedSequence, scale_ss: np.random.SeedSequence,
                  n: int, rows: int, cols: int, dtype: int, std: float,
                  lo: float, hi: float, mx_exp=(118, 122)) -> np.ndarray:
    kids = ss.spawn(n)
    skids = scale_ss.spawn(n)
    first = _draw_matrix(kids[0], rows, cols, dtype, std, skids[0], lo, hi, mx_exp)
    out = np.empty((n,) + first.shape, dtype=first.dtype)
    out[0] = first

    def one(e):
        out[e] = _draw_matrix(kids[e], rows, cols, dtype, std, skids[e], lo, hi, mx_exp)

    if n > 1:
        with _cf.ThreadPoolExecutor(max_workers=_NTHREADS) as ex:
            list(ex.map(one, range(1, n)))
    return out


def make_layer(spec: LayerSpec) -> Dict[str, Optional[np.ndarray]]:
    """Draw one layer's weights (host arrays in storage format)."""
    H, E, I, Is = spec.hidden, spec.num_experts, spec.expert_inter, spec.shared_inter
    ch = _children(spec.seed)
    # Each scale-bearing tensor takes its own grandchild of the q8_scale stream.
    sc = dict(zip(("gate", "up", "down", "shared_gate", "shared_up", "shared_down", "router"),
                  ch["q8_scale"].spawn(7)))
    std, lo, hi = spec.weight_std, spec.q8_scale_lo, spec.q8_scale_hi
    mx = (spec.mx_exp_lo, spec.mx_exp_hi)
    layer: Dict[str, Optional[np.ndarray]] = {}
    layer["router"] = _draw_matrix(ch["router"], E, H, spec.router_dtype, std, sc["router"], lo, hi)
    if spec.router_x_scale == "uniform":
        rs = np.random.default_rng(ch["router_x_scale"]).uniform(0.5, 1.5, H).astype(np.float32)
        layer["router_x_scale"] = bf16_bits(rs)
    else:
        layer["router_x_scale"] = None
    if spec.bias_kind == "normal":
        b = np.random.default_rng(ch["bias"]).standard_normal(E, dtype=np.float32)
        b *= np.float32(spec.bias_std)
        layer["bias"] = bf16_to_f32(bf16_bits(b))        # bf16-representable fp32
    elif spec.bias_kind == "zipf":
        # Expert e gets popularity rank 1 + perm[e]; its logit offset is
        # -s*ln(rank), so exp(offset) falls off as rank**-s (a Zipf law).
        perm = np.random.default_rng(ch["zipf_perm"]).permutation(E)
        rank = (1 + perm).astype(np.float64)
        layer["bias"] = (-spec.zipf_s * np.log(rank)).astype(np.float32)
    else:
        layer["bias"] = None
    layer["gate"] = _draw_experts(ch["gate"], sc["gate"], E, I, H, spec.expert_dtype, std, lo, hi, mx)
    layer["up"] = _draw_experts(ch["up"], sc["up"], E, I, H, spec.expert_dtype, std, lo, hi, mx)
    layer["down"] = _draw_experts(ch["down"], sc["down"], E, H, I, spec.expert_dtype, std, lo, hi, mx)
    if Is > 0:
        layer["shared_gate"] = _draw_matrix(ch["shared_gate"], Is, H, spec.shared_dtype, std, sc["shared_gate"], lo, hi, mx)
        layer["shared_up"] = _draw_matrix(ch["shared_up"], Is, H, spec.shared_dtype, std, sc["shared_up"], lo, hi, mx)
        layer["shared_down"] = _draw_matrix(ch["shared_down"], H, Is, spec.shared_dtype, std, sc["shared_down"], lo, hi, mx)
    else:
        layer["shared_gate"] = layer["shared_up"] = layer["shared_down"] = None
    return layer


def make_tokens(spec: LayerSpec, M: int, batch: int = 0) -> np.ndarray:
    """Draw ``M`` token rows ``x ~ N(0,1)`` for token batch ``batch``."""
    base = _children(spec.seed)["x"]
    ss = np.random.SeedSequence(base.entropy, spawn_key=base.spawn_key + (M, batch))
    x = np.random.default_rng(ss).standard_normal((M, spec.hidden), dtype=np.float32)
    if spec.x_dtype == BF16:
        return bf16_bits(x)
    if spec.x_dtype == F32:
        return x
    raise ValueError("x must be fp32 or bf16")


def small_spec(name: str = "small", **kw) -> LayerSpec:
    """A reduced layer for fast tests; keyword arguments override fields."""
    base = LayerSpec(name=name, hidden=64, num_experts=6, top_k=2, expert_inter=96,
                     seed=4242)
    return base.replace(**kw)


def expert_bytes_per_weight(dtype: int) -> float:
    return {F32: 4.0, BF16: 2.0, Q8_0: Q8_BYTES / Q8_BLOCK, MXFP4: MX_BYTES / MX_BLOCK}[dtype]


def storage_nbytes(dtype: int, rows: int, cols: int) -> int:
    return int(math.ceil(rows * cols * expert_bytes_per_weight(dtype)))
