"""GPU parity: the HIP path through the C ABI against the CPU oracle."""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from synth import BF16, F32, MXFP4, Q8_0, BIAS_LOGIT, BIAS_SELECT_ONLY, SIGMOID_NORM, SOFTMAX_ALL_NORENORM
from gpu_helpers import (SIGMOID_TAU, W_ABS, Y_REL_L2, check_ids, check_ids_keys, check_y, device_layer,
                         forward_parity, host_layer, run_forward, say)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixture_experts_gemv_amd as m
    m.lib()  # loud failure if the library was not built
    yield


def _t(a, dtype=None):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda() if dtype is None else \
        torch.from_numpy(np.ascontiguousarray(a)).to(dtype).cuda()


# ------------------------------------------------------------- block splits
@pytest.mark.parametrize("fmt", ["q8_0", "mxfp4"])
def test_block_split_bit_exact(fmt):
    """moe_q8_0_split / moe_mxfp4_split against the block definition (bytes
    copied, never converted), on random bytes and ragged shapes."""
    import mixture_experts_gemv_amd as m
    rng = np.random.default_rng(7)
    for rows, cols in [(1, 32), (37, 96), (5, 2880), (3, 4608)]:
        nb = cols // 32
        say(f"split {fmt} {rows}x{cols}")
        if fmt == "mxfp4":
            blocks = rng.integers(0, 256, size=(rows, nb, 17), dtype=np.uint8)
            vals = torch.empty(rows * cols // 2, dtype=torch.uint8, device="cuda")
            sc = torch.empty(rows * nb, dtype=torch.uint8, device="cuda")
            m.moe_mxfp4_split(_t(blocks.reshape(-1)), rows, cols, vals, sc)
            want_vals, want_sc = blocks[:, :, 1:].reshape(-1), blocks[:, :, 0].reshape(-1)
            got_vals, got_sc = vals.cpu().numpy(), sc.cpu().numpy()
        else:
            blocks = rng.integers(0, 256, size=(rows, nb, 34), dtype=np.uint8)
            vals = torch.empty(rows * cols, dtype=torch.int8, device="cuda")
            sc = torch.empty(rows * nb, dtype=torch.int16, device="cuda")
            m.moe_q8_0_split(_t(blocks.reshape(-1)), rows, cols, vals, sc)
            want_vals = blocks[:, :, 2:].reshape(-1)
            want_sc = np.ascontiguousarray(blocks[:, :, :2]).reshape(-1).view(np.uint16)
            got_vals, got_sc = vals.cpu().numpy().view(np.uint8), sc.cpu().numpy().view(np.uint16)
        torch.cuda.synchronize()
        assert np.array_equal(got_vals, want_vals), f"{fmt} {rows}x{cols}: value plane differs"
        assert np.array_equal(got_sc, want_sc), f"{fmt} {rows}x{cols}: scale plane differs"


# --------------------------------------------------------------------- routing
ROUTE_CASES = [
    dict(num_experts=8, top_k=2),
    dict(num_experts=64, top_k=6, select=SOFTMAX_ALL_NORENORM),
    dict(num_experts=32, top_k=4, bias_mode=BIAS_LOGIT, bias_kind="normal"),
    dict(num_experts=128, top_k=8, bias_mode=BIAS_SELECT_ONLY, bias_kind="normal"),
    dict(num_experts=256, top_k=8, bias_mode=BIAS_LOGIT, bias_kind="zipf"),
    dict(num_experts=5, top_k=5),
    dict(num_experts=1, top_k=1),
    dict(num_experts=100, top_k=3, select=SOFTMAX_ALL_NORENORM, bias_mode=BIAS_LOGIT,
         bias_kind="normal"),
]


@pytest.mark.parametrize("case", ROUTE_CASES, ids=lambda c: f"E{c['num_experts']}k{c['top_k']}")
def test_route_from_logits_bit_exact(case):
    """With given fp32 logits, selection is pure comparison: ids bit-exact."""
    import mixture_experts_gemv_amd as m
    spec = synth.small_spec(hidden=64, expert_inter=32, seed=900, **case)
    layer = synth.make_layer(spec)
    E, k = spec.num_experts, spec.top_k
    rng = np.random.default_rng(E * 31 + k)
    M = 67
    logits = rng.standard_normal((M, E)).astype(np.float32)
    logits[1] = 0.0                               # all equal
    logits[2, ::2] = -0.0                         # signed zeros mixed with +0
    logits[3] = np.round(logits[3] * 2) / 2       # many exact ties
    logits[4] = logits[4, 0]                      # all equal, non-zero
    if E > 3:
        logits[5, E - 1] = logits[5, 0] = logits[5].max() + 1.0   # tie at the top
    say(f"route from logits E={E} k={k}")
    plan = m.moe_plan_create(64, E, k, 32, max_tokens=M, select=spec.select,
                             bias_mode=spec.bias_mode, x_dtype=m.MOE_BF16)
    bias = layer["bias"]
    wts = m.make_weights(bias=None if bias is None else _t(bias))
    ws = torch.empty(m.moe_workspace_bytes(plan, M), dtype=torch.uint8, device="cuda")
    lg = _t(logits)
    ids = torch.empty(M, k, dtype=torch.int32, device="cuda")
    w = torch.empty(M, k, dtype=torch.float32, device="cuda")
    m.moe_route(plan, None, wts, M, lg, m.MOE_LOGITS_IN, ids, w, ws)
    torch.cuda.synchronize()
    oid, ow = oracle.select(spec, logits.astype(np.float64), bias)
    assert np.array_equal(ids.cpu().numpy(), oid), "ids differ from the oracle on identical logits"
    assert np.max(np.abs(w.cpu().numpy() - ow)) <= W_ABS


SIGMOID_ROUTE_CASES = [
    dict(num_experts=32, top_k=4, select=SIGMOID_NORM),
    dict(num_experts=256, top_k=8, select=SIGMOID_NORM, bias_mode=BIAS_SELECT_ONLY, bias_kind="normal",
         bias_std=0.1),
    dict(num_experts=7, top_k=7, select=SIGMOID_NORM, bias_mode=BIAS_SELECT_ONLY, bias_kind="normal"),
]


@pytest.mark.parametrize("case", SIGMOID_ROUTE_CASES, ids=lambda c: f"E{c['num_experts']}k{c['top_k']}")
def test_route_from_logits_sigmoid(case):
    """Sigmoid scoring from given fp32 logits.  The key sigmoid(l) + b is
    computed in fp32, so two logits can share a key (large logits saturate to
    1): ids follow the near-tie rule with SIGMOID_TAU on the fp64 keys, and
    weights match the oracle run on the GPU's selection."""
    import mixture_experts_gemv_amd as m
    spec = synth.small_spec(hidden=64, expert_inter=32, seed=910, **case)
    layer = synth.make_layer(spec)
    E, k = spec.num_experts, spec.top_k
    rng = np.random.default_rng(E * 37 + k)
    M = 40
    logits = (rng.standard_normal((M, E)) * 2.0).astype(np.float32)
    logits[1] = 0.0                                            # all equal
    logits[2] = 20.0 + 0.25 * np.arange(E, dtype=np.float32)   # scores saturate to 1 in fp32
    logits[3] = np.round(logits[3] * 2) / 2                    # many exact ties
    logits[4, ::2] = -0.0
    say(f"sigmoid route from logits E={E} k={k}")
    plan = m.moe_plan_create(64, E, k, 32, max_tokens=M, select=spec.select,
                             bias_mode=spec.bias_mode, x_dtype=m.MOE_BF16)
    bias = layer["bias"]
    wts = m.make_weights(bias=None if bias is None else _t(bias))
    ws = torch.empty(m.moe_workspace_bytes(plan, M), dtype=torch.uint8, device="cuda")
    ids = torch.empty(M, k, dtype=torch.int32, device="cuda")
    w = torch.empty(M, k, dtype=torch.float32, device="cuda")
    m.moe_route(plan, None, wts, M, _t(logits), m.MOE_LOGITS_IN, ids, w, ws)
    torch.cuda.synchronize()
    gids, gw = ids.cpu().numpy(), w.cpu().numpy()
    l64 = logits.astype(np.float64)
    b64 = np.zeros(E) if bias is None else bias.astype(np.float64)
    keys = 1.0 / (1.0 + np.exp(-l64)) + (b64 if spec.bias_mode else 0.0)
    oid, _ = oracle.select(spec, l64, bias)
    forced, near = check_ids_keys(keys, np.full(M, SIGMOID_TAU), k, gids, oid)
    say(f"near-tie tokens: {near}")
    if not spec.bias_mode:
        assert near >= 1, "the saturated row must count as a near-tie"
    fid, fw = oracle.select(spec, l64, bias, forced_ids=forced)
    for t in range(M):
        for j in range(k):
            jj = list(fid[t]).index(gids[t, j])
            assert abs(gw[t, j] - fw[t, jj]) <= W_ABS, f"token {t}: weight of expert {gids[t, j]}"
        assert abs(gw[t].sum() - 1.0) <= 1e-5


def test_route_from_x_small():
    import mixture_experts_gemv_amd as m
    for n, kw in enumerate([dict(num_experts=8, top_k=2, x_dtype=F32, router_dtype=F32),
                            dict(num_experts=64, top_k=6, select=SOFTMAX_ALL_NORENORM),
                            dict(num_experts=128, top_k=8, bias_mode=BIAS_LOGIT, bias_kind="zipf",
                                 rms_eps=1e-6),
                            dict(num_experts=32, top_k=4, router_dtype=Q8_0, router_x_scale="uniform",
                                 bias_mode=BIAS_LOGIT, bias_kind="normal")]):
        spec = synth.small_spec(hidden=256, expert_inter=32, seed=950 + n, **kw)
        layer = synth.make_layer(spec)
        M = 37
        x = synth.make_tokens(spec, M)
        say(f"route from x case {n}")
        dl = device_layer(spec, layer, M)
        xt = dl.x_tensor(x)
        lg = torch.empty(M, spec.num_experts, dtype=torch.float32, device="cuda")
        ids = torch.empty(M, spec.top_k, dtype=torch.int32, device="cuda")
        w = torch.empty(M, spec.top_k, dtype=torch.float32, device="cuda")
        m.moe_route(dl.plan, xt, dl.weights, M, lg, 0, ids, w, dl.workspace(M))
        torch.cuda.synchronize()
        o = oracle.forward(spec, layer, x)
        np.testing.assert_allclose(lg.cpu().numpy(), o["logits"], rtol=0, atol=1e-4)
        forced, near = check_ids(spec, layer, x, ids.cpu().numpy(), o["ids"])
        assert near <= 2


# ------------------------------------------------------------------- permute
@pytest.mark.parametrize("E,M,k,skew", [(8, 4, 2, 0), (32, 16, 4, 0), (64, 1, 6, 0),
                                         (128, 2048, 8, 1), (256, 300, 8, 1), (3, 1000, 3, 0)])
def test_permute_bit_exact(E, M, k, skew):
    import mixture_experts_gemv_amd as m
    rng = np.random.default_rng(E + M + k)
    if skew:
        p = 1.0 / np.arange(1, E + 1) ** 1.1
        p = p[rng.permutation(E)]
        ids = np.stack([rng.choice(E, size=k, replace=False, p=p / p.sum()) for _ in range(M)])
    else:
        ids = np.stack([rng.permutation(E)[:k] for _ in range(M)])
    ids = ids.astype(np.int32)
    say(f"permute E={E} M={M} k={k}")
    plan = m.moe_plan_create(64, E, k, 32, max_tokens=M)
    ws = torch.empty(m.moe_workspace_bytes(plan, M), dtype=torch.uint8, device="cuda")
    dids = _t(ids)
    outs = [torch.full((n,), -7, dtype=torch.int32, device="cuda") for n in (E, E + 1, M * k, M * k)]
    m.moe_permute(plan, dids, M, *outs, ws)
    torch.cuda.synchronize()
    want = oracle.permute(E, ids)
    for got, ref, name in zip(outs, want, ("counts", "offsets", "sorted_routes", "route_pos")):
        assert np.array_equal(got.cpu().numpy(), ref), name


# --------------------------------------------------------------- stage parity
def test_stages_match_forward_and_oracle():
    """moe_route -> moe_permute -> moe_expert_ffn -> moe_combine equals the oracle."""
    import mixture_experts_gemv_amd as m
    spec = synth.small_spec(hidden=256, num_experts=8, top_k=3, expert_inter=160,
                            bias_mode=BIAS_LOGIT, bias_kind="normal", swiglu_limit=0.5, seed=970)
    layer = synth.make_layer(spec)
    M = 13
    x = synth.make_tokens(spec, M)
    say("stage chain")
    dl = device_layer(spec, layer, M)
    xt = dl.x_tensor(x)
    ws = dl.workspace(M)
    E, k, H, I = spec.num_experts, spec.top_k, spec.hidden, spec.expert_inter
    ids = torch.empty(M, k, dtype=torch.int32, device="cuda")
    w = torch.empty(M, k, dtype=torch.float32, device="cuda")
    m.moe_route(dl.plan, xt, dl.weights, M, None, 0, ids, w, ws)
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    sr = torch.empty(M * k, dtype=torch.int32, device="cuda")
    rp = torch.empty(M * k, dtype=torch.int32, device="cuda")
    m.moe_permute(dl.plan, ids, M, counts, offsets, sr, rp, ws)
    act = torch.empty(M * k, I, dtype=torch.float32, device="cuda")
    m.moe_expert_ffn(dl.plan, xt, dl.weights, M, offsets, sr, act, ws)
    seed = torch.randn(M, H, dtype=torch.float32, device="cuda")
    y = torch.empty(M, H, dtype=torch.float32, device="cuda")
    m.moe_combine(dl.plan, act, dl.weights, M, offsets, sr, rp, w, seed, y, ws)
    torch.cuda.synchronize()
    gids = ids.cpu().numpy()
    o = oracle.forward(spec, layer, x, want_act=True)
    forced, near = check_ids(spec, layer, x, gids, o["ids"])
    o = oracle.forward(spec, layer, x, forced_ids=forced, want_act=True)
    # act rows are in sorted order: row route_pos[r] holds route r
    a = act.cpu().numpy()[rp.cpu().numpy()]
    rel = np.linalg.norm(a - o["act"]) / np.linalg.norm(o["act"])
    assert rel <= 5e-3, f"act rel-L2 {rel:.3e}"
    check_y(y.cpu().numpy() - seed.cpu().numpy(), o["y"], "stage chain")


# ------------------------------------------------------------- small forwards
SMALL = [
    ("tiny", {}, (4, 1, 7)),
    ("q8-bias-clamp", dict(hidden=288, num_experts=12, top_k=4, expert_inter=320,
                           bias_mode=BIAS_LOGIT, bias_kind="normal", swiglu_limit=7.0,
                           expert_dtype=Q8_0), (1, 5, 16)),
    ("softmax-all-shared", dict(hidden=256, num_experts=16, top_k=6, expert_inter=160,
                                shared_inter=320, select=SOFTMAX_ALL_NORENORM), (1, 3, 16)),
    ("bf16-k2", dict(hidden=512, num_experts=8, top_k=2, expert_inter=1056), (1, 16, 70)),
    ("zipf-rms", dict(hidden=256, num_experts=128, top_k=8, expert_inter=96,
                      bias_mode=BIAS_LOGIT, bias_kind="zipf", rms_eps=1e-6), (65, 130)),
    ("q8-shared-many", dict(hidden=128, num_experts=6, top_k=2, expert_inter=64,
                            shared_inter=96, expert_dtype=Q8_0, shared_dtype=Q8_0), (1, 64, 100)),
    ("shared-clamp", dict(hidden=320, num_experts=10, top_k=3, expert_inter=128, shared_inter=192,
                          swiglu_limit=0.05), (1, 7, 33)),
    ("f32x-q8", dict(hidden=160, num_experts=5, top_k=2, expert_inter=64, x_dtype=F32,
                     router_dtype=F32, expert_dtype=Q8_0), (1, 2, 12)),
    ("wide-h", dict(hidden=4608, num_experts=4, top_k=2, expert_inter=64), (1, 3)),
    ("sigmoid-bias", dict(hidden=256, num_experts=16, top_k=4, expert_inter=128, select=SIGMOID_NORM,
                          bias_mode=BIAS_SELECT_ONLY, bias_kind="normal", bias_std=0.05,
                          router_dtype=F32), (1, 5, 16)),
    ("mx4-bias-clamp", dict(hidden=288, num_experts=12, top_k=4, expert_inter=320,
                            bias_mode=BIAS_LOGIT, bias_kind="normal", swiglu_limit=7.0,
                            expert_dtype=MXFP4), (1, 5, 16)),
    ("mx4-shared-many", dict(hidden=128, num_experts=6, top_k=2, expert_inter=64,
                             shared_inter=96, expert_dtype=MXFP4, shared_dtype=MXFP4), (1, 64, 100)),
    ("f32x-mx4", dict(hidden=160, num_experts=5, top_k=2, expert_inter=64, x_dtype=F32,
                      router_dtype=F32, expert_dtype=MXFP4), (1, 2, 12)),
    ("mx4-wide-h", dict(hidden=4608, num_experts=4, top_k=2, expert_inter=96, expert_dtype=MXFP4),
     (1, 3)),
    ("mx4-all-shared-rms", dict(hidden=192, num_experts=16, top_k=6, expert_inter=2112,
                                shared_inter=160, select=SOFTMAX_ALL_NORENORM, rms_eps=1e-6,
                                expert_dtype=MXFP4, shared_dtype=MXFP4), (1, 9)),
    ("mx4-dense", dict(hidden=256, num_experts=1, top_k=1, expert_inter=1088, expert_dtype=MXFP4), (1, 16, 70)),
    # one expert (no router runs) with the pre-norm and a logit bias: the
    # token scale from the norm kernel, the routing from the one-expert kernel
    ("dense-rms-bias", dict(hidden=256, num_experts=1, top_k=1, expert_inter=320, rms_eps=1e-6,
                            bias_mode=BIAS_LOGIT, bias_kind="normal"), (1, 5, 40)),
    ("q8-dense", dict(hidden=256, num_experts=1, top_k=1, expert_inter=320, expert_dtype=Q8_0), (1, 5, 40)),
    # the INT8 router: Q8_0 router rows and a per-element input scale
    ("q8router-scale", dict(hidden=288, num_experts=12, top_k=4, expert_inter=320, bias_mode=BIAS_LOGIT,
                            bias_kind="normal", router_dtype=Q8_0, router_x_scale="uniform",
                            expert_dtype=Q8_0), (1, 5, 16, 40)),
    ("f32x-q8router-shared", dict(hidden=160, num_experts=5, top_k=2, expert_inter=64, shared_inter=96,
                                  x_dtype=F32, router_dtype=Q8_0, router_x_scale="uniform"), (1, 12)),
]


@pytest.mark.parametrize("name,kw,Ms", SMALL, ids=[c[0] for c in SMALL])
def test_forward_small(name, kw, Ms):
    """The per-row (GEMV) kernels, forced, against the oracle."""
    import mixture_experts_gemv_amd as m
    if name == "tiny":
        spec = synth.SPECS["tiny"]
    else:
        spec = synth.small_spec(name=name, seed=1100 + len(name), **kw)
    layer = synth.make_layer(spec)
    dl = device_layer(spec, layer, max(Ms), path=m.MOE_PATH_GEMV)
    for M in Ms:
        x = synth.make_tokens(spec, M, batch=3)
        say(f"forward {name} M={M}")
        forward_parity(spec, layer, x, dl, what=f"{name} M={M}")


MFMA_SMALL = [
    ("k2", dict(hidden=256, num_experts=8, top_k=2, expert_inter=192), (64, 70, 200, 300)),
    ("bias-clamp", dict(hidden=128, num_experts=6, top_k=3, expert_inter=128, bias_mode=BIAS_LOGIT,
                        bias_kind="normal", swiglu_limit=0.3), (65, 130)),
    ("all-shared", dict(hidden=192, num_experts=16, top_k=6, expert_inter=64, shared_inter=320,
                        select=SOFTMAX_ALL_NORENORM), (3, 100)),
    ("zipf-rms", dict(hidden=256, num_experts=64, top_k=8, expert_inter=128, bias_mode=BIAS_LOGIT,
                      bias_kind="zipf", rms_eps=1e-6), (1, 257)),
    ("wide-n", dict(hidden=128, num_experts=4, top_k=1, expert_inter=576), (129,)),
    # Q8_0 at 32-, 64-, 96- and (M = 400: about 110 expected routes an
    # expert) 128-row tiles
    ("q8", dict(hidden=256, num_experts=8, top_k=2, expert_inter=192, expert_dtype=Q8_0),
     (16, 70, 200, 300, 400, 520)),
    ("q8-shared-bias-clamp", dict(hidden=192, num_experts=16, top_k=4, expert_inter=128, shared_inter=256,
                                  expert_dtype=Q8_0, shared_dtype=Q8_0, bias_mode=BIAS_LOGIT,
                                  bias_kind="normal", swiglu_limit=0.5), (3, 33, 100)),
    ("sigmoid-e64", dict(hidden=256, num_experts=64, top_k=8, expert_inter=128, select=SIGMOID_NORM,
                         bias_mode=BIAS_SELECT_ONLY, bias_kind="normal", bias_std=0.05), (1, 70)),
    ("mx4", dict(hidden=256, num_experts=8, top_k=2, expert_inter=192, expert_dtype=MXFP4), (16, 70, 200, 300)),
    ("mx4-shared-bias-clamp", dict(hidden=192, num_experts=16, top_k=4, expert_inter=128, shared_inter=256,
                                   expert_dtype=MXFP4, shared_dtype=MXFP4, bias_mode=BIAS_LOGIT,
                                   bias_kind="normal", swiglu_limit=0.5), (3, 33, 100)),
    ("mx4-wide", dict(hidden=576, num_experts=4, top_k=1, expert_inter=704, expert_dtype=MXFP4), (129,)),
    ("mx4-dense", dict(hidden=256, num_experts=1, top_k=1, expert_inter=1088, expert_dtype=MXFP4), (70,)),
    # about 128 routes an expert: 160-row tiles (M = 512, 560; at 560 some
    # experts spill into a second, ragged tile), two 96-row tiles an expert
    # (M = 600) and two or three 160-row tiles an expert (M = 1100)
    ("k2-wide-tiles", dict(hidden=256, num_experts=8, top_k=2, expert_inter=192), (512, 560, 600, 1100)),
    # MXFP4 beyond 64 routes an expert: several 64-row tiles an expert
    ("mx4-wide-tiles", dict(hidden=256, num_experts=8, top_k=2, expert_inter=192, expert_dtype=MXFP4),
     (512, 560)),
    # one expert: a single ragged 160-row tile (M = 150), two 160-row tiles
    # (M = 300), three 128-row tiles (M = 330)
    ("dense-tiles", dict(hidden=256, num_experts=1, top_k=1, expert_inter=320), (150, 300, 330)),
    # one expert with the pre-norm (scaled in the GEMM epilogue, no router)
    ("dense-rms-bias", dict(hidden=256, num_experts=1, top_k=1, expert_inter=320, rms_eps=1e-6,
                            bias_mode=BIAS_LOGIT, bias_kind="normal"), (70, 150)),
    # Q8_0 one-expert layer: one 96-row tile (M = 70), two (M = 150)
    ("q8-dense", dict(hidden=256, num_experts=1, top_k=1, expert_inter=320, expert_dtype=Q8_0), (70, 150)),
    # 256 experts: the sliced router's widest expert split (four 16-expert
    # tiles a wave), four logits a lane in the top-k, a 256-expert scatter
    ("e256-zipf", dict(hidden=256, num_experts=256, top_k=8, expert_inter=64, bias_mode=BIAS_LOGIT,
                       bias_kind="zipf"), (40, 70, 300)),
    # the INT8 router on the grouped-GEMM path (its logits from the GEMV router)
    ("q8router-scale", dict(hidden=256, num_experts=16, top_k=4, expert_inter=192, router_dtype=Q8_0,
                            router_x_scale="uniform", rms_eps=1e-6), (70, 130)),
]


@pytest.mark.parametrize("name,kw,Ms", MFMA_SMALL, ids=[c[0] for c in MFMA_SMALL])
def test_forward_mfma_small(name, kw, Ms):
    """The MFMA grouped-GEMM path (forced), at sizes spanning several tiles with
    ragged row and column tails, against the oracle."""
    import mixture_experts_gemv_amd as m
    spec = synth.small_spec(name=name, seed=1300 + len(name), **kw)
    layer = synth.make_layer(spec)
    dl = device_layer(spec, layer, max(Ms), path=m.MOE_PATH_MFMA)
    for M in Ms:
        x = synth.make_tokens(spec, M, batch=5)
        say(f"forward (MFMA) {name} M={M}")
        forward_parity(spec, layer, x, dl, what=f"mfma {name} M={M}")


def test_forward_mfma_act_saturates():
    """The grouped-GEMM path carries act as fp16 and saturates values beyond
    +-65504 (the reading of the pages' fp16 act rows, gptoss/state.rs,
    BatchedRoutedScratch.batch_acts).  Weights of std 8 drive some act values
    past the fp16 range: y stays finite and matches the oracle's layer with
    its act rows clamped to +-65504, and not the unclamped one."""
    import mixture_experts_gemv_amd as m
    spec = synth.small_spec(name="act-sat", hidden=256, num_experts=8, top_k=2, expert_inter=128,
                            weight_std=8.0, seed=1391)
    layer = synth.make_layer(spec)
    M = 64
    dl = device_layer(spec, layer, M, path=m.MOE_PATH_MFMA)
    x = synth.make_tokens(spec, M, batch=2)
    say("forward (MFMA) act saturation")
    y, ids, w, counts = run_forward(dl, x)
    assert np.isfinite(y).all(), "non-finite output"
    o = oracle.forward(spec, layer, x, want_act=True)
    forced, near = check_ids(spec, layer, x, ids, o["ids"])
    o = oracle.forward(spec, layer, x, forced_ids=forced, want_act=True)
    act = o["act"]
    sat = int((np.abs(act) > 65504.0).sum())
    assert sat > 0, "no act value exceeds the fp16 range; the case does not test saturation"
    clamped = np.clip(act, -65504.0, 65504.0)
    k = spec.top_k
    y_sat = np.zeros_like(o["y"])
    for t in range(M):
        for j in range(k):
            y_sat[t] += o["w"][t, j] * oracle.down(spec, layer, o["ids"][t, j], clamped[t * k + j])
    rel = lambda a, b: float(np.linalg.norm(a - b) / np.linalg.norm(b))
    r_sat, r_raw = rel(y, y_sat), rel(y, o["y"])
    say(f"act saturation: {sat} of {act.size} act values past 65504; rel-L2 against the clamped "
        f"oracle {r_sat:.3e}, against the unclamped {r_raw:.3e} (near-tie tokens: {near})")
    assert r_sat <= Y_REL_L2, f"rel-L2 {r_sat:.3e} against the clamped oracle"
    assert r_raw > 4 * r_sat, "the output does not show the saturation"


@pytest.mark.parametrize("wdt", [BF16, Q8_0, MXFP4], ids=["bf16", "q8", "mx4"])
def test_stages_mfma(wdt):
    """moe_expert_ffn and moe_combine on the MFMA path equal the oracle (with
    Q8_0 experts moe_combine's fp32 act takes the row kernels)."""
    import mixture_experts_gemv_amd as m
    spec = synth.small_spec(hidden=256, num_experts=8, top_k=2, expert_inter=320,
                            bias_mode=BIAS_LOGIT, bias_kind="normal", swiglu_limit=1.0, seed=1350,
                            expert_dtype=wdt)
    layer = synth.make_layer(spec)
    M = 150
    x = synth.make_tokens(spec, M)
    say("stage chain (MFMA)")
    dl = device_layer(spec, layer, M, path=m.MOE_PATH_MFMA)
    xt = dl.x_tensor(x)
    ws = dl.workspace(M)
    E, k, H, I = spec.num_experts, spec.top_k, spec.hidden, spec.expert_inter
    ids = torch.empty(M, k, dtype=torch.int32, device="cuda")
    w = torch.empty(M, k, dtype=torch.float32, device="cuda")
    m.moe_route(dl.plan, xt, dl.weights, M, None, 0, ids, w, ws)
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    sr = torch.empty(M * k, dtype=torch.int32, device="cuda")
    rp = torch.empty(M * k, dtype=torch.int32, device="cuda")
    m.moe_permute(dl.plan, ids, M, counts, offsets, sr, rp, ws)
    act = torch.empty(M * k, I, dtype=torch.float32, device="cuda")
    m.moe_expert_ffn(dl.plan, xt, dl.weights, M, offsets, sr, act, ws)
    y = torch.empty(M, H, dtype=torch.float32, device="cuda")
    m.moe_combine(dl.plan, act, dl.weights, M, offsets, sr, rp, w, None, y, ws)
    torch.cuda.synchronize()
    o = oracle.forward(spec, layer, x, want_act=True)
    forced, near = check_ids(spec, layer, x, ids.cpu().numpy(), o["ids"])
    o = oracle.forward(spec, layer, x, forced_ids=forced, want_act=True)
    a = act.cpu().numpy()[rp.cpu().numpy()]
    rel = np.linalg.norm(a - o["act"]) / np.linalg.norm(o["act"])
    assert rel <= 5e-3, f"act rel-L2 {rel:.3e}"
    check_y(y.cpu().numpy(), o["y"], "stage chain (MFMA)")


def test_workspace_reuse_across_calls():
    """One workspace, many calls of different M: each result equals a
    fresh-workspace result."""
    spec = synth.small_spec(hidden=256, num_experts=16, top_k=4, expert_inter=192,
                            bias_mode=BIAS_LOGIT, bias_kind="normal", seed=1210)
    layer = synth.make_layer(spec)
    dl = device_layer(spec, layer, 16)
    ws = dl.workspace(16)
    for n, M in enumerate((1, 16, 3, 1, 9, 16, 1)):
        x = dl.x_tensor(synth.make_tokens(spec, M, batch=n))
        say(f"workspace reuse call {n} M={M}")
        a = dl.forward(x, ws=ws).cpu().numpy()
        b = dl.forward(x).cpu().numpy()
        assert np.array_equal(a, b), f"call {n} (M={M}) differs with a reused workspace"


def test_forward_repeatable():
    """Two calls give bitwise-identical y (no atomics in the combine)."""
    spec = synth.small_spec(hidden=256, num_experts=16, top_k=4, expert_inter=192, seed=1200)
    layer = synth.make_layer(spec)
    dl = device_layer(spec, layer, 16)
    x = dl.x_tensor(synth.make_tokens(spec, 16))
    say("repeatability")
    a = dl.forward(x).cpu().numpy()
    b = dl.forward(x).cpu().numpy()
    assert np.array_equal(a, b)


@pytest.mark.parametrize("M,path,fused", [(1, 0, False), (9, 1, False), (130, 2, False), (1, 0, True),
                                          (40, 2, True)],
                         ids=["single", "gemv", "mfma", "single-fused", "mfma-fused"])
def test_graph_replay_matches_eager(M, path, fused):
    """The layer captured in a HIP graph (as bench.py times it): every replay,
    with eager work and synchronisations between replays, equals the eager
    result bitwise (the kernels are deterministic; nothing in a call is a
    memset node)."""
    import mixture_experts_gemv_amd as m
    spec = synth.small_spec(hidden=256, num_experts=16, top_k=4, expert_inter=192, shared_inter=128,
                            bias_mode=BIAS_LOGIT, bias_kind="normal", swiglu_limit=7.0, expert_dtype=Q8_0,
                            shared_dtype=Q8_0, rms_eps=1e-6 if fused else 0.0, seed=1250)
    layer = synth.make_layer(spec)
    dl = device_layer(spec, layer, M, path=path)
    x = dl.x_tensor(synth.make_tokens(spec, M))
    ws = dl.workspace(M)
    gamma = dl.x_tensor(synth.bf16_bits(np.linspace(0.5, 1.5, spec.hidden).astype(np.float32)))
    res = torch.randn(M, spec.hidden, dtype=torch.float32, device="cuda")
    y = torch.empty(M, spec.hidden, dtype=torch.float32, device="cuda")

    def call():
        if fused:
            m.moe_forward_fused(dl.plan, x, gamma, res, dl.weights, M, y, None, None, None, ws)
        else:
            m.moe_forward(dl.plan, x, dl.weights, M, y, None, None, None, ws)

    say(f"graph replay M={M} path={path} fused={fused}")
    call()
    torch.cuda.synchronize()
    eager = y.clone()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            call()
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    for rep in range(3):
        y.fill_(float("nan"))
        other = torch.randn(64, 64, device="cuda") @ torch.randn(64, 64, device="cuda")  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, eager), f"replay {rep} differs from the eager call"
        del other
    del g


@pytest.mark.parametrize("M,path,want", [
    (1, 0, ["router", "gateup", "down"]),
    (9, 1, ["router", "gateup", "down", "combine"]),
    (128, 2, ["router", "topk", "permute", "gateup", "down", "combine"]),
])
def test_forward_timed_matches_forward(M, path, want):
    """moe_forward_timed launches the same kernels (bitwise-equal y), brackets
    each stage with a positive event interval, and leaves later untimed calls
    unaffected."""
    import mixture_experts_gemv_amd as m
    from mixture_experts_gemv_amd.events import HipEvents
    spec = synth.small_spec(hidden=256, num_experts=16, top_k=4, expert_inter=192,
                            bias_mode=BIAS_LOGIT, bias_kind="normal", seed=1230)
    layer = synth.make_layer(spec)
    dl = device_layer(spec, layer, M, path=path)
    x = dl.x_tensor(synth.make_tokens(spec, M))
    ws = dl.workspace(M)
    say(f"timed forward M={M} path={path}")
    ref = dl.forward(x, ws=ws).cpu().numpy()
    y = torch.empty(M, spec.hidden, dtype=torch.float32, device="cuda:0")
    ev = HipEvents(16)
    try:
        st = m.moe_forward_timed(dl.plan, x, dl.weights, M, y, None, None, None, ws, ev.ev)
        torch.cuda.synchronize()
        assert [m.MOE_STAGE_NAMES[i] for i in st] == want
        for j in range(len(st)):
            assert ev.elapsed_ms(2 * j, 2 * j + 1) > 0.0
            if j:
                assert ev.elapsed_ms(2 * j - 1, 2 * j) >= 0.0
        assert np.array_equal(y.cpu().numpy(), ref)
        with pytest.raises(m.MoeError):
            m.moe_forward_timed(dl.plan, x, dl.weights, M, y, None, None, None, ws, ev.ev[:2 * len(st) - 1])
        torch.cuda.synchronize()
    finally:
        ev.close()
    after = dl.forward(x, ws=ws).cpu().numpy()
    assert np.array_equal(after, ref)


# ------------------------------------------------------- fused neighbours
FUSED = [
    # name, layer, token counts, path, norm weight, residual, in place
    ("single-norm-res", dict(hidden=256, num_experts=8, top_k=2, expert_inter=192, rms_eps=1e-6),
     (1,), 0, True, True, False),
    ("gemv-norm-inplace", dict(hidden=288, num_experts=12, top_k=4, expert_inter=320, rms_eps=1e-6,
                               bias_mode=BIAS_LOGIT, bias_kind="normal", swiglu_limit=7.0,
                               expert_dtype=Q8_0), (5, 16), 1, True, True, True),
    ("gemv-shared-norm", dict(hidden=256, num_experts=16, top_k=6, expert_inter=160, shared_inter=320,
                              select=SOFTMAX_ALL_NORENORM, rms_eps=1e-5), (1, 3, 16), 1, True, False, False),
    ("mfma-norm-res", dict(hidden=256, num_experts=8, top_k=2, expert_inter=192, rms_eps=1e-6),
     (64, 130), 2, True, True, False),
    ("mfma-shared-q8-norm", dict(hidden=192, num_experts=16, top_k=4, expert_inter=128, shared_inter=256,
                                 expert_dtype=Q8_0, shared_dtype=Q8_0, rms_eps=1e-6, bias_mode=BIAS_LOGIT,
                                 bias_kind="zipf"), (3, 100), 2, True, True, True),
    ("f32x-norm-res", dict(hidden=160, num_experts=5, top_k=2, expert_inter=64, x_dtype=F32,
                           router_dtype=F32, rms_eps=1e-6), (1, 12), 0, True, True, False),
    ("residual-only", dict(hidden=256, num_experts=8, top_k=2, expert_inter=192), (1, 16, 64), 0,
     False, True, True),
    ("mx4-norm-res", dict(hidden=288, num_experts=12, top_k=4, expert_inter=320, rms_eps=1e-6,
                          expert_dtype=MXFP4), (1, 16), 0, True, True, False),
    ("mfma-wide-tiles-norm-res", dict(hidden=256, num_experts=8, top_k=2, expert_inter=192, rms_eps=1e-6),
     (512,), 2, True, True, False),
    ("q8router-norm-res", dict(hidden=256, num_experts=16, top_k=4, expert_inter=192, rms_eps=1e-6,
                               router_dtype=Q8_0, router_x_scale="uniform"), (1, 9, 100), 0, True, True, True),
    ("dense-norm-res", dict(hidden=256, num_experts=1, top_k=1, expert_inter=320, rms_eps=1e-6),
     (1, 5, 70), 0, True, True, False),
]


@pytest.mark.parametrize("name,kw,Ms,path,use_norm,use_res,in_place", FUSED, ids=[c[0] for c in FUSED])
def test_forward_fused(name, kw, Ms, path, use_norm, use_res, in_place):
    """moe_forward_fused (the post-attention norm with its weight, and the
    residual add) on each kernel family against the oracle."""
    spec = synth.small_spec(name=name, seed=1500 + len(name), **kw)
    layer = synth.make_layer(spec)
    dl = device_layer(spec, layer, max(Ms), path=path)
    rng = np.random.default_rng(len(name))
    gamma = rng.uniform(0.25, 2.0, spec.hidden).astype(np.float32)
    norm_w = (synth.bf16_bits(gamma) if spec.x_dtype == BF16 else gamma) if use_norm else None
    for M in Ms:
        x = synth.make_tokens(spec, M, batch=7)
        res = rng.standard_normal((M, spec.hidden)).astype(np.float32) if use_res else None
        say(f"forward fused {name} M={M}")
        forward_parity(spec, layer, x, dl, what=f"fused {name} M={M}", fused=(norm_w, res, in_place))


# ------------------------------------------------------------ full-size layers
FULL = [("tiny", 4, None), ("gpt-oss-20b", 1, None), ("gpt-oss-20b", 16, None), ("gpt-oss-20b", 64, 8),
        ("deepseek-v2-lite", 1, None), ("deepseek-v2-lite", 16, None),
        ("mixtral-8x7b", 1, None), ("mixtral-8x7b", 16, None),
        ("mixtral-8x7b", 512, 12), ("qwen3-30b-a3b", 2048, 24),
        ("deepseek-v2-lite-dense", 1, None), ("deepseek-v2-lite-dense", 16, None),
        ("deepseek-v2-lite-dense", 512, 8), ("sigmoid-e256", 1, None), ("sigmoid-e256", 16, None),
        ("gpt-oss-20b-mxfp4", 1, None), ("gpt-oss-20b-mxfp4", 16, None), ("gpt-oss-20b-mxfp4", 64, 8),
        ("gpt-oss-20b-mxfp4", 256, 8), ("gpt-oss-20b-int8-router", 1, None),
        ("gpt-oss-20b-int8-router", 16, None), ("gpt-oss-20b-int8-router", 64, 8)]


@pytest.mark.parametrize("name,M,nsample", FULL, ids=[f"{n}-M{m}" for n, m, _ in FULL])
def test_forward_full_size(name, M, nsample):
    """Every workload at its real shape (gpt-oss-shaped M = 64: the Q8_0
    grouped GEMM, 2880-wide matrices with a ragged last column tile)."""
    say(f"generate {name}")
    spec, layer = host_layer(name)
    say(f"upload {name}")
    dl = device_layer(spec, layer, M)
    x = synth.make_tokens(spec, M)
    sample = None
    if nsample:
        rng = np.random.default_rng(M)
        sample = np.sort(rng.choice(M, size=nsample, replace=False))
    say(f"forward {name} M={M}")
    r = forward_parity(spec, layer, x, dl, sample=sample, what=f"{name} M={M}")
    del dl
    torch.cuda.empty_cache()
    say(f"{name} M={M}: touched experts {int((r['counts'] > 0).sum())}")


@pytest.mark.parametrize("name,M,nsample", [("qwen3-30b-a3b", 2048, 16), ("gpt-oss-20b", 1, None),
                                             ("deepseek-v2-lite", 16, None)],
                         ids=["qwen3-30b-a3b-M2048", "gpt-oss-20b-M1", "deepseek-v2-lite-M16"])
def test_forward_fused_full_size(name, M, nsample):
    """The fused layer at full size: the post-attention norm's weight where the
    workload has the pre-norm on, and the residual stream updated in place."""
    say(f"generate {name}")
    spec, layer = host_layer(name)
    dl = device_layer(spec, layer, M)
    rng = np.random.default_rng(M + 3)
    norm_w = synth.bf16_bits(rng.uniform(0.25, 2.0, spec.hidden).astype(np.float32)) if spec.rms_eps > 0 else None
    x = synth.make_tokens(spec, M, batch=11)
    res = rng.standard_normal((M, spec.hidden)).astype(np.float32)
    sample = None
    if nsample:
        sample = np.sort(rng.choice(M, size=nsample, replace=False))
    say(f"forward fused {name} M={M}")
    forward_parity(spec, layer, x, dl, sample=sample, what=f"fused {name} M={M}", fused=(norm_w, res, True))
    del dl
    torch.cuda.empty_cache()
