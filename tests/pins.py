"""Pins for the CPU oracle: checks against what the pages and mathematics fix.

Each ``pin_*`` function raises ``AssertionError`` when the oracle disagrees
with an independent statement of the method: a closed form in numpy written
here (not calling the oracle's code), a pure-Python brute force on tiny shapes,
an invariant, or a hand-derived fixture in ``tests/golden``.  The tests call
every pin on the oracle as built, and again with each deliberate mistake the
oracle can switch on, to show that every such mistake fails some pin.

Passages (turbospark-runtime 0.3.0 source pages):
  * softmax over the selected k -- gptoss/state.rs, RealGptOssState.per_expert_ones;
  * softmax over all experts, top-k, no renormalisation -- deepseek2/state.rs,
    module doc (decoder-layer sketch);
  * router bias before the top-k -- gptoss/state.rs, RealGptOssState.router_bias;
  * clamped SwiGLU -- gptoss/state.rs, module doc;
  * y = shared + sum(w * expert) -- deepseek2/state.rs, RealDeepseek2State.shared_out;
  * route list and phase 1/phase 2 -- gptoss/state.rs, BatchedRoutedScratch;
  * Q8_0 32-element blocks -- deepseek2/state.rs, RealDeepseek2State::build;
  * MXFP4 routed experts -- gptoss/state.rs, module doc and
    RealGptOssState::ensure_batched; the element (FP4 E2M1) and scale (E8M0)
    encodings are the OCP Microscaling Formats (MX) v1.0 specification's.
"""

from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np

import oracle
import synth
from synth import BF16, F32, MXFP4, Q8_0, BIAS_LOGIT, BIAS_NONE, BIAS_SELECT_ONLY
from synth import SIGMOID_NORM, SOFTMAX_ALL_NORENORM, TOPK_SOFTMAX

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# The FP4 E2M1 element values by code, as the OCP MX v1.0 specification lists
# them (codes 8..15 are the negatives of codes 0..7).
E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
                        -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0])


# ---------------------------------------------------------------------------
# independent numpy statement of the layer (dense, fp64)
# ---------------------------------------------------------------------------
def dequant(buf, fmt, rows, cols):
    """Stored matrix -> fp64 [rows][cols] (numpy decoding, not the oracle's)."""
    if fmt == F32:
        return np.asarray(buf, np.float32).reshape(rows, cols).astype(np.float64)
    if fmt == BF16:
        return synth.bf16_to_f32(np.asarray(buf).reshape(rows, cols)).astype(np.float64)
    if fmt == MXFP4:
        codes, e8 = synth.mx_unpack(np.asarray(buf).reshape(rows, -1), cols)
        scale = np.where(e8 == 255, np.nan, np.ldexp(1.0, e8.astype(np.int64) - 127))
        return (E2M1_VALUES[codes].reshape(rows, cols // 32, 32) * scale[:, :, None]).reshape(rows, cols)
    q, d = synth.q8_unpack(np.asarray(buf).reshape(rows, -1), cols)
    return (q.astype(np.float64).reshape(rows, cols // 32, 32)
            * d.astype(np.float64)[:, :, None]).reshape(rows, cols)


def np_tokens(spec, x):
    xf = dequant(x, spec.x_dtype, x.shape[0], spec.hidden)
    if spec.rms_eps > 0:
        xf = xf / np.sqrt(np.mean(xf * xf, axis=1, keepdims=True) + spec.rms_eps)
    return xf


def np_swiglu(xf, g_w, u_w, d_w, limit=0.0):
    g = xf @ g_w.T
    v = xf @ u_w.T
    if limit > 0:
        g = np.clip(g, -limit, limit)
        v = np.clip(v, -limit, limit)
    return (g / (1.0 + np.exp(-g)) * v) @ d_w.T


def np_expert(spec, layer, e, xf):
    H, I = spec.hidden, spec.expert_inter
    gw = dequant(layer["gate"][e], spec.expert_dtype, I, H)
    uw = dequant(layer["up"][e], spec.expert_dtype, I, H)
    dw = dequant(layer["down"][e], spec.expert_dtype, H, I)
    return np_swiglu(xf, gw, uw, dw, spec.swiglu_limit)


def np_shared(spec, layer, xf):
    if spec.shared_inter == 0:
        return np.zeros((xf.shape[0], spec.hidden))
    H, Is = spec.hidden, spec.shared_inter
    return np_swiglu(xf, dequant(layer["shared_gate"], spec.shared_dtype, Is, H),
                     dequant(layer["shared_up"], spec.shared_dtype, Is, H),
                     dequant(layer["shared_down"], spec.shared_dtype, H, Is))


def np_logits(spec, layer, xf):
    return xf @ dequant(layer["router"], spec.router_dtype, spec.num_experts, spec.hidden).T


def _close(a, b, rtol=1e-12, atol=1e-12, what=""):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    err = np.max(np.abs(a - b)) if a.size else 0.0
    scale = max(1.0, float(np.max(np.abs(b)))) if b.size else 1.0
    assert err <= atol + rtol * scale, f"{what}: max abs diff {err:.3e}"


def _spec(**kw):
    base = dict(hidden=32, num_experts=5, top_k=2, expert_inter=32, x_dtype=F32,
                router_dtype=BF16, expert_dtype=BF16, shared_dtype=BF16, seed=777)
    base.update(kw)
    return synth.small_spec(**base)


# ---------------------------------------------------------------------------
# P1: k = E equals the dense softmax-weighted sum over all experts
# ---------------------------------------------------------------------------
def pin_dense_equivalence():
    for select in (TOPK_SOFTMAX, SOFTMAX_ALL_NORENORM):
        spec = _spec(num_experts=4, top_k=4, select=select, bias_mode=BIAS_LOGIT,
                     bias_kind="normal", bias_std=0.5, shared_inter=64, seed=11)
        layer = synth.make_layer(spec)
        x = synth.make_tokens(spec, 3)
        o = oracle.forward(spec, layer, x)
        xf = np_tokens(spec, x)
        u = np_logits(spec, layer, xf) + layer["bias"].astype(np.float64)
        p = np.exp(u - u.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        y = np_shared(spec, layer, xf)
        for e in range(spec.num_experts):
            y = y + p[:, e:e + 1] * np_expert(spec, layer, e, xf)
        _close(o["y"], y, what=f"dense equivalence (select={select})")


# ---------------------------------------------------------------------------
# P2: a one-hot router reduces the layer to one expert's SwiGLU
# ---------------------------------------------------------------------------
def pin_one_hot_router():
    for k in (1, 3):
        spec = _spec(num_experts=5, top_k=k, bias_mode=BIAS_LOGIT, bias_kind="normal", seed=12)
        layer = synth.make_layer(spec)
        layer["router"] = np.zeros_like(layer["router"])
        estar = 3
        b = np.zeros(spec.num_experts, np.float32)
        b[estar] = 50.0
        layer["bias"] = b
        x = synth.make_tokens(spec, 2)
        o = oracle.forward(spec, layer, x)
        assert np.all(o["ids"][:, 0] == estar), "one-hot expert not selected first"
        ref = np_expert(spec, layer, estar, np_tokens(spec, x))
        # the other k-1 experts carry weight e^-50 each
        _close(o["y"], ref, rtol=1e-15 + (k - 1) * 1e-20, atol=(k - 1) * 1e-19,
               what=f"one-hot router k={k}")


# ---------------------------------------------------------------------------
# P3: weight sums
# ---------------------------------------------------------------------------
def pin_weight_sums():
    spec = _spec(num_experts=7, top_k=3, seed=13)
    layer = synth.make_layer(spec)
    logits = np.random.default_rng(5).standard_normal((20, 7))
    _, w = oracle.select(spec, logits)
    assert np.all(np.abs(w.sum(axis=1) - 1.0) <= 1e-12), "softmax over the selected must sum to 1"
    spec_all = spec.replace(select=SOFTMAX_ALL_NORENORM)
    _, w2 = oracle.select(spec_all, logits)
    s = w2.sum(axis=1)
    assert np.all(s < 1.0 - 1e-6), "no-renorm weights of k < E experts must sum below 1"
    spec_full = spec_all.replace(top_k=7)
    _, w3 = oracle.select(spec_full, logits)
    assert np.all(np.abs(w3.sum(axis=1) - 1.0) <= 1e-12), "k = E no-renorm weights sum to 1"
    del layer


# ---------------------------------------------------------------------------
# P4: bias semantics
# ---------------------------------------------------------------------------
def pin_bias_semantics():
    spec = _spec(num_experts=6, top_k=2, bias_mode=BIAS_LOGIT, bias_kind="normal", seed=14)
    rng = np.random.default_rng(14)
    logits = rng.standard_normal((16, 6))
    # multiples of 2^-10, so that adding 2 is exact in fp32
    bias = (np.round(rng.standard_normal(6) * 0.3 * 1024) / 1024).astype(np.float32)
    ids0, w0 = oracle.select(spec, logits, bias)
    ids1, w1 = oracle.select(spec, logits, bias + np.float32(2.0))
    assert np.array_equal(ids0, ids1), "a constant added to every logit bias moved the top-k"
    _close(w0, w1, rtol=1e-12, what="constant logit-bias shift changed the weights")
    # A bias on the first-choice expert only: the set does not change.
    none = spec.replace(bias_mode=BIAS_NONE)
    idsn, wn = oracle.select(none, logits)
    for t in range(logits.shape[0]):
        b = np.zeros(6, np.float32)
        b[idsn[t, 0]] = 0.75
        so = spec.replace(bias_mode=BIAS_SELECT_ONLY)
        ids_s, w_s = oracle.select(so, logits[t:t + 1], b)
        ids_l, w_l = oracle.select(spec, logits[t:t + 1], b)
        assert set(ids_s[0]) == set(idsn[t]) and set(ids_l[0]) == set(idsn[t])
        order = [list(ids_s[0]).index(e) for e in idsn[t]]
        _close(w_s[0][order], wn[t], rtol=1e-13, what="selection-only bias changed the weights")
        order = [list(ids_l[0]).index(e) for e in idsn[t]]
        assert abs(w_l[0][order][0] - wn[t][0]) > 1e-3, "logit bias did not enter the softmax"
    # A bias that lifts a non-selected expert above the boundary changes the ids.
    for mode in (BIAS_LOGIT, BIAS_SELECT_ONLY):
        for t in range(logits.shape[0]):
            out = [e for e in range(6) if e not in idsn[t]][0]
            b = np.zeros(6, np.float32)
            b[out] = 100.0
            ids_b, _ = oracle.select(spec.replace(bias_mode=mode), logits[t:t + 1], b)
            assert ids_b[0, 0] == out, f"bias mode {mode} did not move the selection"


# ---------------------------------------------------------------------------
# sigmoid scoring with a selection-only correction bias
# (llama/state.rs, RealLlamaState::build, MiniMax branch; weights read as the
# selected scores divided by their sum)
# ---------------------------------------------------------------------------
def _sig(v):
    return 1.0 / (1.0 + math.exp(-v))


def pin_sigmoid_scoring():
    spec = _spec(num_experts=6, top_k=3, select=SIGMOID_NORM, seed=17)
    rng = np.random.default_rng(17)
    logits = rng.standard_normal((24, 6)) * 2.0
    bias = (rng.standard_normal(6) * 0.2).astype(np.float32)
    for mode, b in ((BIAS_NONE, None), (BIAS_SELECT_ONLY, bias)):
        ids, w = oracle.select(spec.replace(bias_mode=mode), logits, b)
        assert np.all(np.abs(w.sum(axis=1) - 1.0) <= 1e-12), "sigmoid weights must sum to 1"
        for t in range(logits.shape[0]):
            sc = [_sig(v) for v in logits[t]]
            key = [sc[e] + (float(b[e]) if b is not None else 0.0) for e in range(6)]
            want = sorted(range(6), key=lambda e: (-key[e], e))[:3]
            assert list(ids[t]) == want, f"sigmoid selection: {ids[t]} vs {want}"
            z = sum(sc[e] for e in want)
            for j, e in enumerate(want):
                assert abs(w[t, j] - sc[e] / z) <= 1e-13, "weight = score / sum of selected scores"
    # without a bias the selection is the plain top-k of the logits (sigmoid is monotone)
    ids_s, _ = oracle.select(spec, logits)
    ids_t, _ = oracle.select(spec.replace(select=TOPK_SOFTMAX), logits)
    assert np.array_equal(ids_s, ids_t)
    # the correction bias is added to the score, not to the logit: with logits
    # (10, 0, -3) and bias (0, 0.6, 0), sigmoid(10) + 0 < sigmoid(0) + 0.6 picks
    # expert 1, while sigmoid(10) > sigmoid(0 + 0.6) would pick expert 0
    one = spec.replace(num_experts=3, top_k=1, bias_mode=BIAS_SELECT_ONLY)
    ids1, w1 = oracle.select(one, np.array([[10.0, 0.0, -3.0]]), np.array([0.0, 0.6, 0.0], np.float32))
    assert ids1[0, 0] == 1 and abs(w1[0, 0] - 1.0) <= 1e-15, ids1
    # a bias that keeps the set keeps the weights
    idsn, wn = oracle.select(spec, logits)
    for t in range(logits.shape[0]):
        bb = np.zeros(6, np.float32)
        bb[idsn[t, 0]] = 0.5
        ids_b, w_b = oracle.select(spec.replace(bias_mode=BIAS_SELECT_ONLY), logits[t:t + 1], bb)
        assert set(ids_b[0]) == set(idsn[t])
        order = [list(ids_b[0]).index(e) for e in idsn[t]]
        _close(w_b[0][order], wn[t], rtol=1e-13, what="correction bias changed the weights")
    # two experts, k = 2: closed form
    two = spec.replace(num_experts=2, top_k=2)
    ids2, w2 = oracle.select(two, np.array([[1.5, -0.5]]))
    a, b2 = _sig(1.5), _sig(-0.5)
    assert list(ids2[0]) == [0, 1]
    _close(w2[0], np.array([a / (a + b2), b2 / (a + b2)]), rtol=1e-14, what="two-expert sigmoid weights")


# ---------------------------------------------------------------------------
# P5: brute force on tiny shapes (pure Python, no numpy algebra)
# ---------------------------------------------------------------------------
def _py_f16(bits):
    s, ex, m = bits >> 15, (bits >> 10) & 31, bits & 1023
    v = m * 2.0 ** -24 if ex == 0 else (1 + m / 1024.0) * 2.0 ** (ex - 15)
    return -v if s else v


def _py_matrix(buf, fmt, rows, cols):
    """Pure-Python decoding of one stored matrix into a list of rows."""
    flat = np.asarray(buf).reshape(-1)
    out = []
    for r in range(rows):
        row = []
        for c in range(cols):
            if fmt == F32:
                row.append(float(np.float32(flat[r * cols + c])))
            elif fmt == BF16:
                row.append(float(np.uint32(int(flat[r * cols + c]) << 16).view(np.float32)))
            elif fmt == MXFP4:
                base = r * (cols // 32 * 17) + (c // 32) * 17
                byte = int(flat[base + 1 + (c % 32) // 2])
                code = byte >> 4 if c % 2 else byte & 15
                row.append(float(E2M1_VALUES[code]) * 2.0 ** (int(flat[base]) - 127))
            else:
                rb = cols // 32 * 34
                base = r * rb + (c // 32) * 34
                d = _py_f16(int(flat[base]) | (int(flat[base + 1]) << 8))
                q = int(flat[base + 2 + c % 32])
                q = q - 256 if q > 127 else q
                row.append(d * q)
        out.append(row)
    return out


def _py_layer(spec, layer, x):
    H, E, I, Is, k = spec.hidden, spec.num_experts, spec.expert_inter, spec.shared_inter, spec.top_k
    M = x.shape[0]
    X = _py_matrix(x, spec.x_dtype, M, H)
    if spec.rms_eps > 0:
        X = [[v / math.sqrt(sum(a * a for a in row) / H + spec.rms_eps) for v in row] for row in X]
    R = _py_matrix(layer["router"], spec.router_dtype, E, H)
    G = [_py_matrix(layer["gate"][e], spec.expert_dtype, I, H) for e in range(E)]
    U = [_py_matrix(layer["up"][e], spec.expert_dtype, I, H) for e in range(E)]
    D = [_py_matrix(layer["down"][e], spec.expert_dtype, H, I) for e in range(E)]
    bias = [0.0] * E if layer.get("bias") is None else [float(b) for b in layer["bias"]]
    lim = spec.swiglu_limit

    def swiglu(g_rows, u_rows, d_rows, xr, limit):
        act = []
        for gr, ur in zip(g_rows, u_rows):
            g = sum(a * b for a, b in zip(gr, xr))
            v = sum(a * b for a, b in zip(ur, xr))
            if limit > 0:
                g = min(max(g, -limit), limit)
                v = min(max(v, -limit), limit)
            act.append(g / (1 + math.exp(-g)) * v)
        return [sum(a * b for a, b in zip(dr, act)) for dr in d_rows]

    results = []
    for t in range(M):
        xr = X[t]
        lg = [sum(a * b for a, b in zip(R[e], xr)) for e in range(E)]
        if spec.select == SIGMOID_NORM:
            u = [1.0 / (1.0 + math.exp(-lg[e])) for e in range(E)]
            s = [u[e] + (bias[e] if spec.bias_mode != BIAS_NONE else 0.0) for e in range(E)]
        else:
            s = [lg[e] + (bias[e] if spec.bias_mode in (BIAS_LOGIT, BIAS_SELECT_ONLY) else 0.0)
                 for e in range(E)]
            u = [lg[e] + (bias[e] if spec.bias_mode == BIAS_LOGIT else 0.0) for e in range(E)]
        best = None
        for sub in itertools.combinations(range(E), k):    # lexicographic order
            tot = sum(s[e] for e in sub)
            if best is None or tot > best[0]:
                best = (tot, sub)
        # A set whose total equals the best total but that is lexicographically
        # smaller was met first, so ties resolve to lower ids.
        sub = best[1]
        if spec.select == TOPK_SOFTMAX:
            m = max(u[e] for e in sub)
            z = sum(math.exp(u[e] - m) for e in sub)
            w = {e: math.exp(u[e] - m) / z for e in sub}
        elif spec.select == SIGMOID_NORM:
            z = sum(u[e] for e in sub)
            w = {e: u[e] / z for e in sub}
        else:
            m = max(u)
            z = sum(math.exp(v - m) for v in u)
            w = {e: math.exp(u[e] - m) / z for e in sub}
        if Is > 0:
            y = swiglu(_py_matrix(layer["shared_gate"], spec.shared_dtype, Is, H),
                       _py_matrix(layer["shared_up"], spec.shared_dtype, Is, H),
                       _py_matrix(layer["shared_down"], spec.shared_dtype, H, Is), xr, 0.0)
        else:
            y = [0.0] * H
        for e in sub:
            ye = swiglu(G[e], U[e], D[e], xr, lim)
            y = [a + w[e] * b for a, b in zip(y, ye)]
        results.append((set(sub), w, y))
    return results


BRUTE_CASES = [
    dict(hidden=8, num_experts=5, top_k=2, expert_inter=4, expert_dtype=F32, router_dtype=F32),
    dict(hidden=8, num_experts=6, top_k=3, expert_inter=4, select=SOFTMAX_ALL_NORENORM,
         bias_mode=BIAS_LOGIT, bias_kind="normal", bias_std=0.8),
    dict(hidden=8, num_experts=4, top_k=2, expert_inter=6, bias_mode=BIAS_SELECT_ONLY,
         bias_kind="normal", bias_std=1.0, shared_inter=4, swiglu_limit=0.05),
    dict(hidden=64, num_experts=4, top_k=2, expert_inter=32, expert_dtype=Q8_0,
         router_dtype=BF16, x_dtype=BF16, rms_eps=1e-3),
    dict(hidden=8, num_experts=6, top_k=3, expert_inter=4, select=SIGMOID_NORM,
         bias_mode=BIAS_SELECT_ONLY, bias_kind="normal", bias_std=0.3, router_dtype=F32),
    dict(hidden=64, num_experts=4, top_k=2, expert_inter=32, expert_dtype=MXFP4,
         shared_dtype=MXFP4, shared_inter=32, bias_mode=BIAS_LOGIT, bias_kind="normal",
         swiglu_limit=0.5),
]


def pin_brute_force():
    for n, kw in enumerate(BRUTE_CASES):
        spec = synth.small_spec(seed=100 + n, **kw)
        layer = synth.make_layer(spec)
        x = synth.make_tokens(spec, 3)
        o = oracle.forward(spec, layer, x)
        ref = _py_layer(spec, layer, x)
        for t, (sub, w, y) in enumerate(ref):
            assert set(o["ids"][t]) == sub, f"case {n} token {t}: ids {o['ids'][t]} vs {sorted(sub)}"
            for j, e in enumerate(o["ids"][t]):
                assert abs(o["w"][t, j] - w[e]) <= 1e-13, f"case {n}: weight of expert {e}"
            _close(o["y"][t], y, rtol=1e-12, atol=1e-14, what=f"brute force case {n} token {t}")
    # exact ties at the selection boundary go to the lower expert id
    spec = synth.small_spec(hidden=8, num_experts=5, top_k=2, expert_inter=4, seed=120,
                            x_dtype=F32, router_dtype=F32, expert_dtype=F32)
    layer = synth.make_layer(spec)
    r = layer["router"].reshape(5, 8)
    r[1] = np.abs(r[1])
    r[2] = r[1]
    r[4] = r[1]          # experts 1, 2 and 4 share one positive logit
    r[0] = 2.0 * r[1]    # expert 0 leads
    r[3] = -np.abs(r[3])  # expert 3 trails
    x = np.abs(synth.make_tokens(spec, 2)).astype(np.float32)
    o = oracle.forward(spec, layer, x)
    ref = _py_layer(spec, layer, x)
    for t in range(2):
        assert set(o["ids"][t]) == ref[t][0] == {0, 1}, f"tie rule: {o['ids'][t]}"


# ---------------------------------------------------------------------------
# P6: x = 0
# ---------------------------------------------------------------------------
def pin_zero_input():
    for select in (TOPK_SOFTMAX, SOFTMAX_ALL_NORENORM, SIGMOID_NORM):
        spec = _spec(num_experts=6, top_k=3, select=select, shared_inter=32, rms_eps=1e-6, seed=15)
        layer = synth.make_layer(spec)
        x = np.zeros((2, spec.hidden), np.float32)
        o = oracle.forward(spec, layer, x)
        assert np.all(o["logits"] == 0.0)
        assert np.array_equal(o["ids"], np.tile(np.arange(3, dtype=np.int32), (2, 1))), o["ids"]
        want = 1.0 / 6 if select == SOFTMAX_ALL_NORENORM else 1.0 / 3
        _close(o["w"], np.full((2, 3), want), what="uniform weights at x = 0")
        assert np.all(o["y"] == 0.0), "y must vanish at x = 0"


# ---------------------------------------------------------------------------
# P7: relabelling experts permutes ids and leaves y unchanged
# ---------------------------------------------------------------------------
def pin_relabel_invariance():
    spec = _spec(num_experts=6, top_k=2, bias_mode=BIAS_LOGIT, bias_kind="normal", seed=16)
    layer = synth.make_layer(spec)
    x = synth.make_tokens(spec, 4)
    perm = np.array([3, 5, 0, 1, 4, 2])      # new expert n is old expert perm[n]
    L2 = dict(layer)
    L2["router"] = np.ascontiguousarray(layer["router"].reshape(6, -1)[perm])
    L2["bias"] = np.ascontiguousarray(layer["bias"][perm])
    for key in ("gate", "up", "down"):
        L2[key] = np.ascontiguousarray(layer[key][perm])
    a = oracle.forward(spec, layer, x)
    b = oracle.forward(spec, L2, x)
    inv = np.argsort(perm)
    assert np.array_equal(inv[a["ids"]], b["ids"]), "relabelled ids"
    _close(a["y"], b["y"], rtol=1e-13, what="relabelled y")


# ---------------------------------------------------------------------------
# P8: tokens are independent; counts add over sub-batches
# ---------------------------------------------------------------------------
def pin_token_independence():
    spec = _spec(num_experts=6, top_k=2, shared_inter=32, seed=17)
    layer = synth.make_layer(spec)
    x = synth.make_tokens(spec, 5)
    full = oracle.forward(spec, layer, x)
    total = np.zeros(6, np.int64)
    for t in range(5):
        one = oracle.forward(spec, layer, np.ascontiguousarray(x[t:t + 1]))
        assert np.array_equal(one["ids"][0], full["ids"][t])
        assert np.array_equal(one["y"][0], full["y"][t]), "token result depends on the batch"
        total += one["counts"]
    assert np.array_equal(total, full["counts"])
    assert full["counts"].sum() == 5 * spec.top_k


# ---------------------------------------------------------------------------
# P9: the clamp
# ---------------------------------------------------------------------------
def pin_clamp():
    spec = _spec(num_experts=4, top_k=2, seed=18, x_dtype=F32)
    layer = synth.make_layer(spec)
    x = (synth.make_tokens(spec, 3) * np.float32(8.0)).astype(np.float32)
    off = oracle.forward(spec, layer, x, want_act=True)
    huge = oracle.forward(spec.replace(swiglu_limit=1e30), layer, x, want_act=True)
    _close(off["y"], huge["y"], rtol=0, atol=0, what="an unreachable clamp changed y")
    L = 0.05
    cl = oracle.forward(spec.replace(swiglu_limit=L), layer, x, want_act=True)
    assert np.max(np.abs(cl["act"])) <= L * L * (1 + 1e-12), "clamped |silu(g)*v| exceeds limit^2"
    assert np.max(np.abs(off["act"])) > L * L, "test input never reaches the clamp"
    # The pre-activations of the unclamped layer, from numpy, decide which side binds.
    xf = np_tokens(spec, x)
    for t in range(3):
        for j in range(2):
            e = cl["ids"][t, j]
            g = xf[t] @ dequant(layer["gate"][e], spec.expert_dtype, 32, 32).T
            v = xf[t] @ dequant(layer["up"][e], spec.expert_dtype, 32, 32).T
            gc, vc = np.clip(g, -L, L), np.clip(v, -L, L)
            _close(cl["act"][t * 2 + j], gc / (1 + np.exp(-gc)) * vc, what="clamped act")


# ---------------------------------------------------------------------------
# P10: Q8_0 equals the bf16 layer built from its dequantised weights
# ---------------------------------------------------------------------------
def pin_q8_vs_bf16():
    spec = _spec(hidden=64, expert_inter=64, num_experts=4, top_k=2, expert_dtype=Q8_0,
                 x_dtype=BF16, seed=19)
    layer = synth.make_layer(spec)
    rng = np.random.default_rng(19)
    bf = dict(layer)
    for key, (rows, cols) in (("gate", (64, 64)), ("up", (64, 64)), ("down", (64, 64))):
        blocks = []
        vals = []
        for e in range(4):
            q = rng.integers(-127, 128, size=(rows, cols), dtype=np.int8)
            d = np.ldexp(1.0, rng.integers(-12, -6, size=(rows, cols // 32))).astype(np.float16)
            blocks.append(synth.q8_pack(q, d))
            vals.append((q.astype(np.float32).reshape(rows, cols // 32, 32)
                         * d.astype(np.float32)[:, :, None]).reshape(rows, cols))
        layer[key] = np.stack(blocks)
        v = np.stack(vals)
        bits = synth.bf16_bits(v)
        assert np.array_equal(synth.bf16_to_f32(bits), v), "power-of-two scales must be bf16-exact"
        bf[key] = bits
    x = synth.make_tokens(spec, 3)
    a = oracle.forward(spec, layer, x)
    b = oracle.forward(spec.replace(expert_dtype=BF16), bf, x)
    assert np.array_equal(a["ids"], b["ids"])
    assert np.array_equal(a["y"], b["y"]), "Q8_0 and its bf16 image disagree"


# ---------------------------------------------------------------------------
# P10b: MXFP4 equals the bf16 layer built from its dequantised weights (every
# E2M1 value times a power-of-two scale in bf16's range is a bf16 value)
# ---------------------------------------------------------------------------
def pin_mxfp4_vs_bf16():
    spec = _spec(hidden=64, expert_inter=96, num_experts=4, top_k=2, expert_dtype=MXFP4,
                 shared_dtype=MXFP4, shared_inter=64, x_dtype=BF16, seed=23)
    layer = synth.make_layer(spec)
    rng = np.random.default_rng(23)
    bf = dict(layer)
    shapes = {"gate": (4, 96, 64), "up": (4, 96, 64), "down": (4, 64, 96),
              "shared_gate": (1, 64, 64), "shared_up": (1, 64, 64), "shared_down": (1, 64, 64)}
    for key, (n, rows, cols) in shapes.items():
        blocks, vals = [], []
        for _ in range(n):
            codes = rng.integers(0, 16, size=(rows, cols), dtype=np.uint8)
            # scales differ from block to block, so a wrong block index shows
            e8 = rng.integers(110, 131, size=(rows, cols // 32), dtype=np.uint8)
            blocks.append(synth.mx_pack(codes, e8))
            vals.append((E2M1_VALUES[codes].reshape(rows, cols // 32, 32)
                         * np.ldexp(1.0, e8.astype(np.int64) - 127)[:, :, None]).reshape(rows, cols))
        v = np.stack(vals).astype(np.float32)
        bits = synth.bf16_bits(v)
        assert np.array_equal(synth.bf16_to_f32(bits), v), "MXFP4 values must be bf16-exact"
        layer[key] = np.stack(blocks) if n > 1 else blocks[0]
        bf[key] = bits if n > 1 else bits[0]
    x = synth.make_tokens(spec, 3)
    a = oracle.forward(spec, layer, x)
    b = oracle.forward(spec.replace(expert_dtype=BF16, shared_dtype=BF16), bf, x)
    assert np.array_equal(a["ids"], b["ids"])
    assert np.array_equal(a["y"], b["y"]), "MXFP4 and its bf16 image disagree"


# ---------------------------------------------------------------------------
# P11: one expert, k = 1 is a plain dense SwiGLU FFN (with and without pre-norm)
# ---------------------------------------------------------------------------
def pin_single_expert_dense():
    for eps in (0.0, 1e-2):
        for fmt in (F32, BF16, Q8_0, MXFP4):
            spec = _spec(num_experts=1, top_k=1, hidden=64, expert_inter=96, expert_dtype=fmt,
                         rms_eps=eps, seed=20)
            layer = synth.make_layer(spec)
            x = synth.make_tokens(spec, 3)
            o = oracle.forward(spec, layer, x)
            assert np.all(o["w"] == 1.0)
            xf = dequant(x, spec.x_dtype, 3, 64)
            if eps > 0:
                xf = xf / np.sqrt((xf ** 2).mean(axis=1, keepdims=True) + eps)
            ref = np_swiglu(xf, dequant(layer["gate"][0], fmt, 96, 64),
                            dequant(layer["up"][0], fmt, 96, 64),
                            dequant(layer["down"][0], fmt, 64, 96))
            _close(o["y"], ref, what=f"dense SwiGLU fmt={fmt} eps={eps}")


# ---------------------------------------------------------------------------
# P12: the permutation
# ---------------------------------------------------------------------------
def pin_permute():
    rng = np.random.default_rng(21)
    for E, M, k in ((8, 10, 3), (5, 1, 5), (16, 64, 4)):
        ids = np.stack([rng.permutation(E)[:k] for _ in range(M)]).astype(np.int32)
        counts, offsets, sr, rp = oracle.permute(E, ids)
        flat = ids.reshape(-1)
        assert counts.sum() == M * k
        assert np.array_equal(counts, np.bincount(flat, minlength=E))
        assert offsets[0] == 0 and np.array_equal(np.diff(offsets), counts)
        keys = [(flat[r], r) for r in sr]
        assert keys == sorted(keys), "routes not in (expert, route) order"
        assert np.array_equal(rp[sr], np.arange(M * k)), "route_pos is not the inverse"


# ---------------------------------------------------------------------------
# P13: the RMS pre-norm makes the layer invariant to the scale of x
# ---------------------------------------------------------------------------
def pin_prenorm_scale_invariance():
    spec = _spec(num_experts=5, top_k=2, rms_eps=1e-12, shared_inter=32, seed=22)
    layer = synth.make_layer(spec)
    x = synth.make_tokens(spec, 3)
    a = oracle.forward(spec, layer, x)
    b = oracle.forward(spec, layer, (x * np.float32(4.0)).astype(np.float32))
    assert np.array_equal(a["ids"], b["ids"])
    _close(a["y"], b["y"], rtol=1e-9, what="pre-norm scale invariance")


def pin_fused_norm_weight_and_residual():
    """The fused neighbours (deepseek2/state.rs module doc: the post-attention
    RMSNorm's output feeds the router and the experts; the routed sum plus the
    shared expert is added to the residual stream).  A unit norm weight is the unit-gain pre-norm; the
    weighted norm stays invariant under scaling x; the residual adds to y."""
    spec = _spec(num_experts=6, top_k=2, rms_eps=1e-12, shared_inter=64, x_dtype=BF16, seed=31)
    layer = synth.make_layer(spec)
    x = synth.make_tokens(spec, 4)
    plain = oracle.forward(spec, layer, x)
    ones = synth.bf16_bits(np.ones(spec.hidden, np.float32))
    unit = oracle.forward(spec, layer, x, norm_w=ones)
    assert np.array_equal(plain["ids"], unit["ids"])
    _close(plain["y"], unit["y"], rtol=0, atol=0, what="unit norm weight")
    rng = np.random.default_rng(5)
    gamma = synth.bf16_bits(rng.uniform(0.5, 1.5, spec.hidden).astype(np.float32))
    a = oracle.forward(spec, layer, x, norm_w=gamma)
    x4 = synth.bf16_bits(synth.bf16_to_f32(x) * np.float32(4.0))
    c = oracle.forward(spec, layer, x4, norm_w=gamma)
    assert np.array_equal(a["ids"], c["ids"])
    _close(a["y"], c["y"], rtol=1e-9, what="weighted norm scale invariance")
    res = rng.standard_normal((4, spec.hidden)).astype(np.float32)
    r = oracle.forward(spec, layer, x, norm_w=gamma, residual=res)
    assert np.array_equal(a["ids"], r["ids"])
    _close(r["y"] - a["y"], res.astype(np.float64), rtol=1e-12, atol=1e-12, what="residual add")
    # a norm weight needs the pre-norm on
    try:
        oracle.forward(spec.replace(rms_eps=0.0), layer, x, norm_w=gamma)
    except ValueError:
        pass
    else:
        raise AssertionError("a norm weight without the pre-norm was accepted")


def pin_fused_closed_form():
    """Hand-derived case: H = I = 32, x = ones, eps = 3, so mean(x^2) + eps =
    4 and f = gamma / 2.  Router rows e_0 and e_1 with gamma_0 = 2 and
    gamma_1 = 4 give logits 1 and 2: expert 1 is picked (k = 1, weight 1),
    whereas without the weight the logits tie at 0.5 and expert 0 (all-zero
    weights) would win.  Expert 1 has identity gate, up and down, so
    y_i = r_i + f_i * silu(f_i) = r_i + f_i^2 / (1 + exp(-f_i))."""
    H = 32
    spec = synth.small_spec(hidden=H, num_experts=2, top_k=1, expert_inter=H, rms_eps=3.0,
                            x_dtype=F32, router_dtype=F32, expert_dtype=F32, shared_dtype=F32)
    eye = np.eye(H, dtype=np.float32)
    router = np.zeros((2, H), np.float32)
    router[0, 0] = router[1, 1] = 1.0
    zeros = np.zeros((H, H), np.float32)
    layer = {"router": router, "bias": None,
             "gate": np.stack([zeros, eye]), "up": np.stack([zeros, eye]), "down": np.stack([zeros, eye])}
    gamma = np.array([2.0, 4.0] + [i / 4 for i in range(2, H)], np.float32)
    x = np.ones((1, H), np.float32)
    res = np.arange(H, dtype=np.float32).reshape(1, H) - 7.0
    o = oracle.forward(spec, layer, x, norm_w=gamma, residual=res)
    assert o["ids"].tolist() == [[1]], f"ids {o['ids'].tolist()}"
    f = gamma.astype(np.float64) / 2.0
    want = res.astype(np.float64)[0] + f * f / (1.0 + np.exp(-f))
    _close(o["y"][0], want, rtol=1e-15, atol=1e-15, what="fused closed form")


# ---------------------------------------------------------------------------
# P16: the INT8 router (llama/state.rs, RealLlamaState.router_ones: the INT8
# router kernel scales each input element by an effective scale, identically
# 1 for the pages' architectures).  The scale acts on the router's input
# only, so folding it into the router rows gives the same layer (every
# product below is exact in fp64: bf16 x, bf16 scale, bf16 router); a uniform
# scale c is a softmax temperature on the selected logits; Q8_0 router rows
# equal their bf16 image when the block scales are powers of two.
# ---------------------------------------------------------------------------
def pin_router_input_scale():
    spec = _spec(num_experts=6, top_k=2, shared_inter=32, x_dtype=BF16, router_dtype=BF16, seed=41)
    layer = synth.make_layer(spec)
    x = synth.make_tokens(spec, 5)
    rng = np.random.default_rng(41)
    rs = synth.bf16_bits(rng.uniform(0.5, 1.5, spec.hidden).astype(np.float32))
    a = oracle.forward(spec, dict(layer, router_x_scale=rs), x)
    folded = dict(layer)
    w = synth.bf16_to_f32(layer["router"]).astype(np.float64) * synth.bf16_to_f32(rs).astype(np.float64)
    folded["router"] = w.astype(np.float32)
    assert np.array_equal(folded["router"].astype(np.float64), w), "bf16 x bf16 must be fp32-exact"
    b = oracle.forward(spec.replace(router_dtype=F32), folded, x)
    assert np.array_equal(a["ids"], b["ids"]), "input scale vs folded router: ids"
    assert np.array_equal(a["logits"], b["logits"]), "input scale vs folded router: logits"
    assert np.array_equal(a["y"], b["y"]), "the router's input scale reached the experts"
    # uniform scale 2: same picks, weights softmax(2 l) over the picks
    two = synth.bf16_bits(np.full(spec.hidden, 2.0, np.float32))
    c = oracle.forward(spec, dict(layer, router_x_scale=two), x)
    p = oracle.forward(spec, layer, x)
    assert np.array_equal(c["ids"], p["ids"])
    for t in range(x.shape[0]):
        sel = 2.0 * p["logits"][t, p["ids"][t]]
        ww = np.exp(sel - sel.max())
        _close(c["w"][t], ww / ww.sum(), rtol=1e-12, atol=1e-14, what="scale 2 as a temperature")


def pin_q8_router_vs_bf16():
    spec = _spec(hidden=64, expert_inter=32, num_experts=5, top_k=2, x_dtype=BF16, router_dtype=Q8_0, seed=43)
    layer = synth.make_layer(spec)
    rng = np.random.default_rng(43)
    q = rng.integers(-127, 128, size=(5, 64), dtype=np.int8)
    d = np.ldexp(1.0, rng.integers(-12, -6, size=(5, 2))).astype(np.float16)
    layer["router"] = synth.q8_pack(q, d)
    v = (q.astype(np.float32).reshape(5, 2, 32) * d.astype(np.float32)[:, :, None]).reshape(5, 64)
    bf = dict(layer, router=synth.bf16_bits(v))
    assert np.array_equal(synth.bf16_to_f32(bf["router"]), v), "power-of-two scales must be bf16-exact"
    rs = synth.bf16_bits(rng.uniform(0.5, 1.5, 64).astype(np.float32))
    x = synth.make_tokens(spec, 4)
    a = oracle.forward(spec, dict(layer, router_x_scale=rs), x)
    b = oracle.forward(spec.replace(router_dtype=BF16), dict(bf, router_x_scale=rs), x)
    assert np.array_equal(a["logits"], b["logits"]) and np.array_equal(a["y"], b["y"]), \
        "Q8_0 router and its bf16 image disagree"
    # and the logits against a numpy statement of the scaled router
    xf = dequant(x, BF16, 4, 64) * synth.bf16_to_f32(rs).astype(np.float64)
    _close(a["logits"], xf @ v.astype(np.float64).T, rtol=1e-12, what="Q8_0 router logits")


# ---------------------------------------------------------------------------
# Hand-derived fixtures (tests/golden/*.json)
# ---------------------------------------------------------------------------
def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def pin_golden_selection():
    for name in ("select_topk_softmax.json", "select_softmax_all.json"):
        g = _golden(name)
        spec = _spec(num_experts=len(g["logits"][0]), top_k=g["top_k"], select=g["select"],
                     bias_mode=g["bias_mode"])
        bias = None if g["bias"] is None else np.array(g["bias"], np.float32)
        ids, w = oracle.select(spec, np.array(g["logits"]), bias)
        assert ids.tolist() == g["ids"], f"{name}: ids {ids.tolist()}"
        _close(w, np.array(g["w"]), rtol=1e-15, atol=1e-15, what=name)


def pin_golden_layer():
    for name in ("swiglu_clamp.json", "rms_prenorm.json"):
        g = _golden(name)
        spec = synth.small_spec(hidden=g["hidden"], num_experts=g["num_experts"],
                                top_k=g["top_k"], expert_inter=g["expert_inter"],
                                swiglu_limit=g["swiglu_limit"], rms_eps=g["rms_eps"],
                                x_dtype=F32, router_dtype=F32, expert_dtype=F32)
        E, I, H = g["num_experts"], g["expert_inter"], g["hidden"]
        layer = {"router": np.array(g["router"], np.float32),
                 "bias": None,
                 "gate": np.array(g["gate"], np.float32).reshape(E, I, H),
                 "up": np.array(g["up"], np.float32).reshape(E, I, H),
                 "down": np.array(g["down"], np.float32).reshape(E, H, I)}
        o = oracle.forward(spec, layer, np.array(g["x"], np.float32), want_act=True)
        assert o["ids"].tolist() == g["ids"], f"{name}: ids"
        _close(o["act"], np.array(g["act"]), rtol=1e-15, atol=1e-15, what=name + " act")
        _close(o["y"], np.array(g["y"]), rtol=1e-15, atol=1e-15, what=name + " y")


def pin_golden_q8_0():
    g = _golden("q8_0_block.json")
    raw = np.array(g["bytes"], np.uint8).reshape(1, -1)
    cols = g["cols"]
    for c, want in enumerate(g["values"]):
        got = oracle.element(raw, Q8_0, 0, cols, c)
        assert got == want, f"Q8_0 element {c}: {got} != {want}"


def pin_golden_mxfp4():
    g = _golden("mxfp4_block.json")
    raw = np.array(g["bytes"], np.uint8).reshape(1, -1)
    cols = g["cols"]
    for c, want in enumerate(g["values"]):
        got = oracle.element(raw, MXFP4, 0, cols, c)
        if want is None:
            assert math.isnan(got), f"MXFP4 element {c}: {got} is not NaN"
        else:
            assert got == want and math.copysign(1.0, got) == math.copysign(1.0, want), \
                f"MXFP4 element {c}: {got} != {want}"


PINS = [
    pin_dense_equivalence, pin_one_hot_router, pin_weight_sums, pin_bias_semantics,
    pin_brute_force, pin_zero_input, pin_relabel_invariance, pin_token_independence,
    pin_clamp, pin_q8_vs_bf16, pin_single_expert_dense, pin_permute,
    pin_prenorm_scale_invariance, pin_golden_selection, pin_golden_layer, pin_golden_q8_0,
    pin_sigmoid_scoring, pin_mxfp4_vs_bf16, pin_golden_mxfp4,
    pin_fused_norm_weight_and_residual, pin_fused_closed_form,
    pin_router_input_scale, pin_q8_router_vs_bf16,
]
