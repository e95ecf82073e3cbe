"""Helpers for the GPU parity tests: device layers, the near-tie rule, tolerances."""

from __future__ import annotations

import functools
import sys

import numpy as np

import oracle
import synth
from pins import dequant
from synth import SIGMOID_NORM

# Output tolerance for fp32 accumulation over bf16 / Q8_0 weights.
Y_MAX_ABS = 2e-2
Y_REL_L2 = 5e-3
# Routing-weight tolerance (fp32 softmax vs fp64).
W_ABS = 1e-5
# Near-tie bound: a GPU logit in fp32 differs from the exact one by at most
# TAU_REL * sum_i |x_i * w_i| (+|b|) for the summation orders used here.
TAU_REL = 2.0 ** -17
# Relative error of a value carried as bf16 hi plus bf16 lo (lo rounds v - hi).
SPLIT_REL = 2.0 ** -18
# Sigmoid scoring: the fp32 sigmoid of a logit and the add of the correction
# bias are each within a few units of 2^-24 of the exact values.
SIGMOID_TAU = 2.0 ** -20


def say(msg: str) -> None:
    print(f"[gpu-test] {msg}", flush=True)
    sys.stdout.flush()


@functools.lru_cache(maxsize=4)
def host_layer(name: str):
    spec = synth.SPECS[name]
    return spec, synth.make_layer(spec)


def device_layer(spec, layer, max_tokens, path=0):
    from mixture_experts_gemv_amd.layer import MoeLayer
    dl = MoeLayer(hidden=spec.hidden, num_experts=spec.num_experts, top_k=spec.top_k,
                  expert_inter=spec.expert_inter, shared_inter=spec.shared_inter,
                  select=spec.select, bias_mode=spec.bias_mode,
                  swiglu_limit=spec.swiglu_limit, rms_eps=spec.rms_eps,
                  x_dtype=spec.x_dtype, router_dtype=spec.router_dtype,
                  expert_dtype=spec.expert_dtype, shared_dtype=spec.shared_dtype,
                  max_tokens=max_tokens, path=path)
    dl.load(layer["router"], layer["bias"], layer["gate"], layer["up"], layer["down"],
            layer.get("shared_gate"), layer.get("shared_up"), layer.get("shared_down"),
            layer.get("router_x_scale"))
    return dl


def selection_keys(spec, layer, x, norm_w=None, split=False):
    """fp64 selection keys s[t][e] and the near-tie bound tau[t].

    ``split``: the router read the weighted normed rows as bf16 hi + lo (the
    grouped-GEMM path of moe_forward_fused with a norm weight), which holds
    each value to 2^-18 of itself and so adds 2^-18 * A to the bound; every
    other path reads fp32 rows and keeps the plain bound."""
    xf = dequant(x, spec.x_dtype, x.shape[0], spec.hidden)
    if spec.rms_eps > 0:
        xf = xf / np.sqrt(np.mean(xf * xf, axis=1, keepdims=True) + spec.rms_eps)
        if norm_w is not None:
            xf = xf * dequant(np.asarray(norm_w).reshape(1, -1), spec.x_dtype, 1, spec.hidden)
    wr = dequant(layer["router"], spec.router_dtype, spec.num_experts, spec.hidden)
    if layer.get("router_x_scale") is not None:
        # the router's per-element input scale
        wr = wr * synth.bf16_to_f32(layer["router_x_scale"]).astype(np.float64)[None, :]
    logits = xf @ wr.T
    b = np.zeros(spec.num_experts) if layer.get("bias") is None else layer["bias"].astype(np.float64)
    A = np.abs(xf) @ np.abs(wr).T + (np.abs(b) if spec.bias_mode != 0 else 0.0)
    tau = TAU_REL * A.max(axis=1)
    if split and norm_w is not None:
        tau = tau + SPLIT_REL * A.max(axis=1)
    if spec.select == SIGMOID_NORM:
        # key sigmoid(l) + b: sigmoid' <= 1/4 carries the logit bound over, and
        # the fp32 sigmoid and add are covered by SIGMOID_TAU
        return 1.0 / (1.0 + np.exp(-logits)) + (b if spec.bias_mode != 0 else 0.0), tau / 4 + SIGMOID_TAU
    s = logits + (b if spec.bias_mode != 0 else 0.0)
    return s, tau


def check_ids(spec, layer, x, gpu_ids, ora_ids, norm_w=None, split=False):
    """Apply the near-tie rule; return (forced ids for the oracle, number of near-tie tokens).

    Tokens whose k-th and (k+1)-th fp64 keys are further apart than tau must get
    exactly the oracle's expert set.  For near-tie tokens the GPU set must hold
    every expert whose key clears the boundary by more than tau and draw the
    rest from keys within tau of it; the oracle is then re-run on the GPU's set.
    """
    s, tau = selection_keys(spec, layer, x, norm_w, split)
    return check_ids_keys(s, tau, spec.top_k, gpu_ids, ora_ids)


def check_ids_keys(s, tau, k, gpu_ids, ora_ids):
    """The near-tie rule on given fp64 keys s[t][e] and bounds tau[t]."""
    E = s.shape[1]
    forced = ora_ids.copy()
    near = 0
    for t in range(s.shape[0]):
        order = np.argsort(-s[t], kind="stable")
        sk = s[t, order[k - 1]]
        sk1 = s[t, order[k]] if k < E else -np.inf
        gset = set(int(e) for e in gpu_ids[t])
        assert len(gset) == k, f"token {t}: repeated expert in {gpu_ids[t]}"
        assert all(0 <= e < E for e in gset), f"token {t}: expert id out of range {gpu_ids[t]}"
        if sk - sk1 > tau[t]:
            assert gset == set(int(e) for e in ora_ids[t]), \
                f"token {t}: ids {sorted(gset)} vs oracle {sorted(ora_ids[t])}"
        else:
            near += 1
            must = {e for e in range(E) if s[t, e] > sk + tau[t]}
            may = {e for e in range(E) if s[t, e] >= sk - tau[t]}
            assert must <= gset <= may, f"near-tie token {t}: ids {sorted(gset)}"
            forced[t] = gpu_ids[t]
    return forced, near


def check_y(y_gpu, y_ref, what=""):
    y_gpu = np.asarray(y_gpu, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    err = np.abs(y_gpu - y_ref)
    max_abs = float(err.max()) if err.size else 0.0
    rel = float(np.linalg.norm(y_gpu - y_ref) / max(np.linalg.norm(y_ref), 1e-30))
    say(f"{what}: max-abs {max_abs:.3e}, rel-L2 {rel:.3e}")
    assert max_abs <= Y_MAX_ABS, f"{what}: max-abs error {max_abs:.3e} > {Y_MAX_ABS}"
    assert rel <= Y_REL_L2, f"{what}: relative L2 error {rel:.3e} > {Y_REL_L2}"
    return max_abs, rel


def run_forward(dl, x_host, M=None, fused=None):
    """moe_forward, or with fused = (norm_w host array or None, residual host
    array or None, in_place) moe_forward_fused."""
    import torch
    x = dl.x_tensor(x_host)
    M = x.shape[0]
    ids = torch.empty(M, dl.k, dtype=torch.int32, device=dl.device)
    w = torch.empty(M, dl.k, dtype=torch.float32, device=dl.device)
    counts = torch.empty(dl.E, dtype=torch.int32, device=dl.device)
    if fused is None:
        y = dl.forward(x, ids=ids, w=w, counts=counts)
    else:
        norm_w, residual, in_place = fused
        nw = None if norm_w is None else dl.x_tensor(np.ascontiguousarray(norm_w))
        res = None if residual is None else torch.from_numpy(np.ascontiguousarray(residual, np.float32)).to(dl.device)
        if in_place:
            y = dl.forward_fused(x, norm_weight=nw, residual=res, y=res, ids=ids, w=w, counts=counts)
        else:
            y = dl.forward_fused(x, norm_weight=nw, residual=res, ids=ids, w=w, counts=counts)
    torch.cuda.synchronize()
    return y.cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy(), counts.cpu().numpy()


def hot_expert_sample(ids, E, stride=32):
    """Tokens routed to the most-loaded expert, one every ``stride`` of its
    routes in sorted (token-ascending) order, and its last: with ``stride`` the
    smallest grouped-GEMM tile height (32 rows), every tile of that expert
    holds one of them."""
    counts = np.bincount(ids.reshape(-1), minlength=E)
    hot = int(np.argmax(counts))
    toks = np.nonzero((ids == hot).any(axis=1))[0]
    pick = list(toks[::stride]) + ([toks[-1]] if len(toks) else [])
    return np.asarray(pick, dtype=np.int64), hot, int(counts[hot])


def forward_parity(spec, layer, x, dl, sample=None, what="", fused=None):
    """Whole-layer parity against the oracle (fused: as run_forward; the
    oracle takes the same norm weight and residual).

    Every token's expert set is checked under the near-tie rule and the
    per-expert counts must equal those of the oracle's selection (with the
    GPU's set forced on near-tie tokens), over the whole batch.  Weights and
    y are compared on ``sample`` (all tokens when None), which is widened with
    tokens in every tile of the most-loaded expert."""
    import mixture_experts_gemv_amd as m
    y, ids, w, counts = run_forward(dl, x, fused=fused)
    M = x.shape[0]
    norm_w = res_all = None
    if fused is not None:
        norm_w = fused[0]
        res_all = fused[1]
    # (the grouped-GEMM router takes the weighted normed rows as bf16 hi + lo)
    split = (m.moe_forward_path(dl.plan, M) == m.MOE_RUN_NAMES.index("mfma")
             and spec.router_dtype == synth.BF16)
    # the selection of every token
    r = oracle.route(spec, layer, x, norm_w=norm_w)
    forced, near = check_ids(spec, layer, x, ids, r["ids"], norm_w, split)
    want_counts = np.bincount(forced.reshape(-1), minlength=spec.num_experts)
    assert np.array_equal(counts, want_counts), "per-expert counts differ from the oracle's"
    if sample is None:
        sample = np.arange(M)
    else:
        hot_tokens, hot, hot_n = hot_expert_sample(forced, spec.num_experts)
        sample = np.unique(np.concatenate([np.asarray(sample, np.int64), hot_tokens]))
        say(f"{what}: y sampled on {len(sample)} tokens (expert {hot} holds {hot_n} routes)")
    xs = np.ascontiguousarray(x[sample])
    res = None if res_all is None else np.ascontiguousarray(res_all[sample], np.float32)
    o = oracle.forward(spec, layer, xs, forced_ids=np.ascontiguousarray(forced[sample]), norm_w=norm_w,
                       residual=res)
    # weights, matched by expert id
    for i, t in enumerate(sample):
        for j in range(spec.top_k):
            e = ids[t, j]
            jj = list(o["ids"][i]).index(e)
            assert abs(w[t, j] - o["w"][i, jj]) <= W_ABS, f"{what}: weight token {t} expert {e}"
    ma, rel = check_y(y[sample], o["y"], what=f"{what} (near-tie tokens: {near} of {M})")
    return dict(max_abs=ma, rel_l2=rel, near_ties=near, ids=ids, counts=counts)
