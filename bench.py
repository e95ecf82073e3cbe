"""Throughput of the routed MoE layer on one MI355X, against the HBM and MFMA roofs.

One JSON line, with three measured points of the metric (tokens/s at
M = 1 / 16 / 2048):

* ``value``: a gpt-oss-20B-shaped MoE layer (hidden 2880, 32 experts, expert
  width 2880, top-4, logit bias, SwiGLU clamp 7, Q8_0 experts, bf16 x)
  decoding M = 1 token per call;
* ``points``: the same layer at M = 16, and a Qwen3-30B-A3B-shaped layer
  (hidden 2048, 128 experts, width 768, top-8, Zipf(1.1) logit skew, RMS
  pre-norm, bf16 experts) prefilling M = 2048 tokens per call.

One step = one moe_forward call (router, top-k, permutation, gate/up +
SwiGLU, down + combine) on inputs already resident in HBM.  Each point
captures K steps in one HIP graph and replays it in loops of at least 20 ms;
the point's time is the median of at least five loops (>= 100 ms in all).

Layer copies are rotated so that the 256 MB MALL cannot hold the touched
weights across calls; copy 0 comes from the seeded host generator, the others
are drawn on the device with the same distributions (the Zipf skew too, from
a permutation of their own).

`roofline` is for each point's dominant kernel (gate/up), timed with HIP
events recorded by the kernel's own dispatch on the layer's stream;
`cpu_baseline` times the fp64 CPU oracle, over all host cores, on a bounded
sample of the headline workload.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE layer tokens/s at M=1/16/2048 + % of HBM / MFMA roofline"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFS = 2500.0
# gate/up + SwiGLU kernel of each moe_forward path (the layer's dominant kernel)
GATEUP_KERNEL = {"single": "k_gateup_m1", "gemv": "k_gateup_rows", "mfma": "k_gemm_lds<0"}


def gateup_kernel(spec, M: int, path: str) -> str:
    """Name of the gate/up kernel the library runs for this layer and M (it
    labels the roofline object and picks the traffic record).  On the gemv
    path the library streams (touched expert, row) pairs with the whole batch
    in LDS when x is bf16, the weights are bf16, Q8_0 or MXFP4 (the shared
    expert's alike), a row is at most 4 chunks a lane (2 for MXFP4) and the
    batch fits 150 KB of LDS; otherwise it runs the per-row kernel."""
    if path != "gemv":
        return GATEUP_KERNEL[path]
    H, k = spec.hidden, spec.top_k
    n = {0: 4, 1: 8, 2: 16, 3: 32}[spec.expert_dtype]
    cpl = (H // n + 63) // 64
    lds = M * H * 2 + M * k * 4 + M * 4 + (2 * 256 + 2) * 4
    stream = (spec.x_dtype == 1 and spec.expert_dtype != 0
              and (spec.shared_inter == 0 or spec.shared_dtype == spec.expert_dtype)
              and spec.num_experts <= 256 and lds <= 150 * 1024
              and cpl <= (2 if spec.expert_dtype == 3 else 4))
    return "k_gateup_stream" if stream else "k_gateup_rows"


# ------------------------------------------------------------------ workload
def bytes_per_weight(dtype: int) -> float:
    return {0: 4.0, 1: 2.0, 2: 34.0 / 32.0, 3: 17.0 / 32.0}[dtype]


def algorithmic_bytes(spec, M: int, counts: np.ndarray, fused: bool = False) -> dict:
    """Bytes the layer must move per call (weights of touched experts once).

    `gateup_kernel` is what the gate/up kernel itself must move: the touched
    experts' gate and up rows, x and act."""
    H, E, I, Is = spec.hidden, spec.num_experts, spec.expert_inter, spec.shared_inter
    T = int((counts > 0).sum())
    bpw = bytes_per_weight(spec.expert_dtype)
    bpx = 4 if spec.x_dtype == 0 else 2
    R = M * spec.top_k
    gate_up = T * 2 * H * I * bpw + (2 * H * Is * bytes_per_weight(spec.shared_dtype) if Is else 0)
    down = T * H * I * bpw + (H * Is * bytes_per_weight(spec.shared_dtype) if Is else 0)
    router = (H * E * bytes_per_weight(spec.router_dtype) + (4 * E if spec.bias_mode else 0)
              + (2 * H if spec.router_x_scale != "none" else 0))
    layer = gate_up + down + router + M * H * bpx + 4 * M * H
    if fused:  # the residual read, and the norm weight
        layer += 4 * M * H + (H * bpx if spec.rms_eps > 0 else 0)
    gk = gate_up + M * H * bpx + 4 * (R * I + M * Is)
    return {"layer": layer, "gateup_kernel": gk, "touched": T}


def algorithmic_flops(spec, M: int) -> float:
    H, E, I, Is, k = spec.hidden, spec.num_experts, spec.expert_inter, spec.shared_inter, spec.top_k
    return M * k * 6 * H * I + 2 * M * H * E + M * 6 * H * Is


def device_copy(spec, dev, rng_seed: int):
    """Random layer tensors with the host generator's distributions (timing only)."""
    import torch
    g = torch.Generator(device=dev)
    g.manual_seed(rng_seed)
    H, E, I, Is = spec.hidden, spec.num_experts, spec.expert_inter, spec.shared_inter

    def mat(rows, cols, dtype):
        if dtype == 2:
            q = torch.randint(-127, 128, (rows * cols,), generator=g, device=dev, dtype=torch.int8)
            d = torch.empty(rows * cols // 32, device=dev, dtype=torch.float32)
            d.uniform_(spec.q8_scale_lo, spec.q8_scale_hi, generator=g)
            return q, d.half().view(torch.int16)
        if dtype == 3:  # MXFP4: code bytes (two E2M1 codes each) and E8M0 scale bytes
            c = torch.randint(0, 256, (rows * cols // 2,), generator=g, device=dev, dtype=torch.uint8)
            e = torch.randint(spec.mx_exp_lo, spec.mx_exp_hi + 1, (rows * cols // 32,), generator=g,
                              device=dev, dtype=torch.uint8)
            return c, e
        t = torch.empty(rows * cols, device=dev, dtype=torch.float32).normal_(0.0, spec.weight_std, generator=g)
        return (t.bfloat16() if dtype == 1 else t), None

    out = {}
    out["router"], rsc = mat(E, H, spec.router_dtype)
    if rsc is not None:
        out["router_scale"] = rsc
    if spec.router_x_scale == "uniform":
        out["router_x_scale"] = torch.empty(H, device=dev).uniform_(0.5, 1.5, generator=g).bfloat16()
    if spec.bias_kind == "zipf":
        # the host generator's skew with a permutation of this copy's own:
        # expert e gets rank 1 + perm[e] and the logit offset -s * ln(rank)
        perm = torch.randperm(E, generator=g, device=dev)
        out["bias"] = (-spec.zipf_s * torch.log((1 + perm).double())).float()
    elif spec.bias_kind == "normal":
        out["bias"] = (torch.empty(E, device=dev).normal_(0.0, spec.bias_std, generator=g)
                       .bfloat16().float())
    for name, rows, cols in (("gate", E * I, H), ("up", E * I, H), ("down", E * H, I)):
        t, s = mat(rows, cols, spec.expert_dtype)
        out[name] = t
        if s is not None:
            out[name + "_scale"] = s
    if Is:
        for name, rows, cols in (("shared_gate", Is, H), ("shared_up", Is, H), ("shared_down", H, Is)):
            t, s = mat(rows, cols, spec.shared_dtype)
            out[name] = t
            if s is not None:
                out[name + "_scale"] = s
    return out


def layer_bytes(spec) -> float:
    H, E, I, Is = spec.hidden, spec.num_experts, spec.expert_inter, spec.shared_inter
    return 3 * E * H * I * bytes_per_weight(spec.expert_dtype) + 3 * H * Is * bytes_per_weight(spec.shared_dtype)


def cpu_baseline(spec, host_layer, M: int, budget_s: float) -> dict:
    """Time the fp64 CPU oracle on successive M-token calls until ~budget_s."""
    import oracle
    import synth
    calls = 0
    t0 = time.perf_counter()
    while True:
        x = synth.make_tokens(spec, M, batch=100 + calls)
        oracle.forward(spec, host_layer, x)
        calls += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    threads = oracle.threads()
    how = ("tokens in parallel" if M >= threads else
           "each expert's output rows in parallel (fewer tokens than threads)")
    return {"value": calls * M / el, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{calls} calls of M={M} token(s) of the same layer ({el:.1f} s), "
                      f"OpenMP over {threads} host threads, {how}"}


def time_graph(step, K: int, stream: int, ev, min_loop_ms: float = 20.0, min_loops: int = 5):
    """Capture K steps in one HIP graph; replay it in loops of >= min_loop_ms.

    Returns (median ms per step over the loops, details)."""
    import torch
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            for i in range(K):
                step(i)
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    g.replay()                      # warm replay
    torch.cuda.synchronize()
    ev.record(0, stream)
    g.replay()
    ev.record(1, stream)
    torch.cuda.synchronize()
    one = ev.elapsed_ms(0, 1)
    reps = max(1, math.ceil(min_loop_ms / max(one, 1e-3)))
    loops = []
    while len(loops) < min_loops or sum(loops) * reps * K < 100.0:
        ev.record(0, stream)
        for _ in range(reps):
            g.replay()
        ev.record(1, stream)
        torch.cuda.synchronize()
        loops.append(ev.elapsed_ms(0, 1) / (reps * K))
    del g
    return float(np.median(loops)), {"loops": len(loops), "replays_per_loop": reps, "graph_steps": K,
                                     "timed_ms": float(sum(loops) * reps * K),
                                     "spread": [float(min(loops)), float(max(loops))]}


_HOST: dict = {}   # the last workload's host layer (points of one workload share it)


def measure_point(spec, M: int, args, want_cpu: bool) -> dict:
    """Time one (workload, M) point; returns its JSON object."""
    import torch
    import synth
    import mixture_experts_gemv_amd as m
    from mixture_experts_gemv_amd import profiling
    from mixture_experts_gemv_amd.events import HipEvents
    from mixture_experts_gemv_amd.layer import MoeLayer

    dev = torch.device("cuda:0")
    t_setup = time.perf_counter()
    if spec.name not in _HOST:
        _HOST.clear()
        _HOST[spec.name] = synth.make_layer(spec)
    host = _HOST[spec.name]
    kw = dict(hidden=spec.hidden, num_experts=spec.num_experts, top_k=spec.top_k,
              expert_inter=spec.expert_inter, shared_inter=spec.shared_inter, select=spec.select,
              bias_mode=spec.bias_mode, swiglu_limit=spec.swiglu_limit, rms_eps=spec.rms_eps,
              x_dtype=spec.x_dtype, router_dtype=spec.router_dtype, expert_dtype=spec.expert_dtype,
              shared_dtype=spec.shared_dtype, max_tokens=M, device=dev,
              path={"auto": m.MOE_PATH_AUTO, "gemv": m.MOE_PATH_GEMV, "mfma": m.MOE_PATH_MFMA}[args.path])
    base = MoeLayer(**kw).load(host["router"], host["bias"], host["gate"], host["up"], host["down"],
                               host.get("shared_gate"), host.get("shared_up"), host.get("shared_down"),
                               host.get("router_x_scale"))
    # estimate touched bytes with a realised call, then size the rotation
    x0 = base.x_tensor(synth.make_tokens(spec, M, batch=0))
    cnt = torch.empty(spec.num_experts, dtype=torch.int32, device=dev)
    base.forward(x0, counts=cnt)
    touched = algorithmic_bytes(spec, M, cnt.cpu().numpy())["layer"]
    L = args.layers or max(2, math.ceil(2 ** 30 / touched) + 1)
    copies = [base]
    for c in range(1, L):
        copies.append(MoeLayer(**kw).load_tensors(device_copy(spec, dev, 7919 * c)))
    P = 64 if M == 1 else (8 if M <= 16 else 2)
    xs = [base.x_tensor(synth.make_tokens(spec, M, batch=b)) for b in range(P)]
    ws = base.workspace(M)
    y = torch.empty(M, spec.hidden, dtype=torch.float32, device=dev)
    K, W = args.steps, args.warmup
    counts = [torch.empty(spec.num_experts, dtype=torch.int32, device=dev) for _ in range(K)]
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_setup

    norm_w = None
    if args.fused and spec.rms_eps > 0:
        gw = torch.Generator(device=dev)
        gw.manual_seed(4099)
        nw = torch.empty(spec.hidden, device=dev).uniform_(0.25, 2.0, generator=gw)
        norm_w = nw.bfloat16() if spec.x_dtype == 1 else nw
    y.zero_()

    def step(i, cnt_out=None):
        lay = copies[i % L]
        if args.fused:
            m.moe_forward_fused(lay.plan, xs[i % P], norm_w, y, lay.weights, M, y, None, None, cnt_out, ws)
        else:
            m.moe_forward(lay.plan, xs[i % P], lay.weights, M, y, None, None, cnt_out, ws)

    # realised expert counts of exactly the timed calls (untimed pre-pass)
    for i in range(K):
        step(i, counts[i])
    torch.cuda.synchronize()
    run = m.moe_forward_path(base.plan, M)
    cnts = [c.cpu().numpy() for c in counts]
    ab = [algorithmic_bytes(spec, M, c, args.fused) for c in cnts]
    layer_bytes_avg = float(np.mean([a["layer"] for a in ab]))
    gateup_bytes_avg = float(np.mean([a["gateup_kernel"] for a in ab]))
    touched_avg = float(np.mean([a["touched"] for a in ab]))
    max_load = float(np.mean([c.max() for c in cnts]))

    ev = HipEvents(2)
    stream = torch.cuda.current_stream().cuda_stream
    # ---- eager launches (one loop of K steps; informational)
    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    ev.record(0, stream)
    for i in range(K):
        step(i)
    ev.record(1, stream)
    torch.cuda.synchronize()
    eager_ms = ev.elapsed_ms(0, 1)

    # ---- the timed region: K steps in one HIP graph, median of replay loops
    graph_timing = None
    if not args.no_graph:
        ms_per_step, graph_timing = time_graph(step, K, stream, ev)
    else:
        ms_per_step = eager_ms / K

    # ---- per kernel: start/end events recorded by each kernel's own dispatch
    n_ev = 16
    kev = HipEvents(n_ev * K)
    stages = None
    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    for i in range(K):
        lay = copies[i % L]
        stages = m.moe_forward_timed(lay.plan, xs[i % P], lay.weights, M, y, None, None, None, ws,
                                     kev.ev[i * n_ev:(i + 1) * n_ev])
    torch.cuda.synchronize()
    per_stage = {}
    for j, sid in enumerate(stages):
        d = [kev.elapsed_ms(i * n_ev + 2 * j, i * n_ev + 2 * j + 1) for i in range(K)]
        per_stage[m.MOE_STAGE_NAMES[sid]] = float(np.mean(d)) * 1e3  # us
    timed_total_us = float(np.mean([kev.elapsed_ms(i * n_ev, i * n_ev + 2 * len(stages) - 1)
                                    for i in range(K)])) * 1e3
    kev.close()
    ev.close()

    kernel = gateup_kernel(spec, M, m.MOE_RUN_NAMES[run])
    tag = f"{spec.name}_M{M}" + ("_fused" if args.fused else "")
    trec = profiling.load_traffic(os.path.join(ROOT, "profiles"), kernel, tag)
    flops = algorithmic_flops(spec, M)
    gateup_us = per_stage.get("gateup")
    gateup_flops = M * spec.top_k * 4 * spec.hidden * spec.expert_inter + M * 4 * spec.hidden * spec.shared_inter
    achieved = gateup_bytes_avg / (gateup_us * 1e-6) / 1e9
    layer_gbs = layer_bytes_avg / (ms_per_step * 1e-3) / 1e9
    point = {
        "workload": (f"{spec.name}-shaped dense SwiGLU layer (one expert, top-1), M={M} tokens per call"
                     if spec.num_experts == 1 else
                     f"{spec.name}-shaped routed MoE layer, M={M} tokens per call"),
        "tokens_per_call": M,
        "tokens_per_s": M / (ms_per_step * 1e-3),
        "ms_per_call": ms_per_step,
        "config": {
            "hidden": spec.hidden, "num_experts": spec.num_experts, "top_k": spec.top_k,
            "expert_inter": spec.expert_inter, "shared_inter": spec.shared_inter,
            "expert_weights": {0: "f32", 1: "bf16", 2: "q8_0", 3: "mxfp4"}[spec.expert_dtype],
            "router_bias": spec.bias_kind if spec.bias_mode else "none",
            "rms_prenorm": spec.rms_eps > 0,
            "layer_copies": L, "token_batches": P,
            "touched_experts_avg": touched_avg, "max_expert_routes_avg": max_load,
            "path": m.MOE_RUN_NAMES[run],
            "call": ("moe_forward_fused (norm weight %s, residual in place); per-kernel times from "
                     "the unfused moe_forward_timed" % ("on" if norm_w is not None else "off")
                     if args.fused else "moe_forward"),
        },
        "timing": dict(graph_timing, method="hip_graph_replay_median") if graph_timing
        else {"method": "eager", "steps": K},
        "eager": {"tokens_per_s": M * K / (eager_ms * 1e-3), "ms_per_call": eager_ms / K},
        "roofline": {
            "bound": "hbm", "kernel": kernel, "path": m.MOE_RUN_NAMES[run],
            "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": trec["traffic_bytes"] if trec else None,
            "traffic_source": os.path.basename(trec["_file"]) if trec else None,
            "bytes_per_launch": gateup_bytes_avg, "us_per_launch": gateup_us,
            "mfma_frac": gateup_flops / (gateup_us * 1e-6) / (MFMA_BF16_PEAK_TFS * 1e12),
        },
        "layer": {
            "algorithmic_bytes": layer_bytes_avg, "algorithmic_flops": flops,
            "achieved_GBs": layer_gbs, "hbm_frac": layer_gbs / HBM_PEAK_GBS,
            "mfma_frac": flops / (ms_per_step * 1e-3) / (MFMA_BF16_PEAK_TFS * 1e12),
            "kernel_us": per_stage, "timed_sum_us": timed_total_us,
        },
        "setup_s": setup_s,
    }
    if want_cpu:
        point["cpu_baseline"] = cpu_baseline(spec, host, M, args.cpu_seconds)
    del copies, base, xs, ws, host
    torch.cuda.empty_cache()
    return point


DEFAULT_POINTS = (("gpt-oss-20b", 1), ("gpt-oss-20b", 16), ("qwen3-30b-a3b", 2048))


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20, help="K: steps captured in each point's graph")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None,
                    help="measure this workload only (default: the three points of the metric)")
    ap.add_argument("--tokens", type=int, default=None, help="M per call (with --workload; default: its first)")
    ap.add_argument("--layers", type=int, default=None, help="layer copies to rotate")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches only")
    ap.add_argument("--path", choices=("auto", "gemv", "mfma"), default="auto",
                    help="kernel family: the plan's choice (default) or forced")
    ap.add_argument("--fused", action="store_true",
                    help="time moe_forward_fused: the pre-norm's weight (when the workload has the "
                         "pre-norm) and the residual stream updated in place")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run 5 plain 256 MiB device copies (counter calibration) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path)", file=sys.stderr)
        return 2

    import torch
    if args.copy_probe:
        # A plain device copy of known size: the reference reading of the HBM
        # byte counters (FETCH_SIZE, WRITE_SIZE) under rocprofv3 --pmc.
        n = 256 << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_per_copy": n, "copies": 5}), flush=True)
        return 0
    import synth
    torch.cuda.set_device(0)

    if args.workload:
        spec = synth.SPECS[args.workload]
        todo = [(args.workload, args.tokens or spec.token_counts[0])]
    else:
        todo = list(DEFAULT_POINTS)
    points = []
    for n, (name, M) in enumerate(todo):
        print(f"[bench] {name} M={M}: measuring", file=sys.stderr, flush=True)
        pt = measure_point(synth.SPECS[name], M, args, want_cpu=(n == 0 and not args.no_cpu_baseline))
        print(f"[bench] {name} M={M}: {pt['ms_per_call'] * 1e3:.1f} us/call, "
              f"{pt['tokens_per_s']:.4g} tokens/s, layer {pt['layer']['hbm_frac']:.3f} of HBM",
              file=sys.stderr, flush=True)
        points.append(pt)
    head = points[0]
    result = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_call"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": dict(head["config"], workload=head["workload"], tokens_per_call=head["tokens_per_call"]),
        "timing": head["timing"],
        "eager": head["eager"],
        "roofline": head["roofline"],
        "layer": head["layer"],
        "points": [{k: v for k, v in p.items() if k != "cpu_baseline"} for p in points],
        "setup_s": sum(p["setup_s"] for p in points),
    }
    if "cpu_baseline" in head:
        result["cpu_baseline"] = head["cpu_baseline"]
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
