"""The C ABI without a GPU: symbols, plan validation, workspace sizing, and
argument checks that must refuse before anything is enqueued."""

from __future__ import annotations

import ctypes
import os
import re

import pytest

import mixture_experts_gemv_amd as m

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
           if f.endswith(".h")]


def declared_functions():
    names = set()
    for h in HEADERS:
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for mm in re.finditer(r"^[A-Za-z_][\w\s\*]*?\b(moe_\w+)\s*\(", text, flags=re.M):
            names.add(mm.group(1))
    return sorted(names)


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 10, names
    lib = m.lib()
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/ but not exported"


def test_binding_has_every_entry_point():
    for n in declared_functions():
        assert callable(getattr(m, n)), f"binding lacks {n}"


BASE = dict(hidden=256, num_experts=8, top_k=2, expert_inter=512, max_tokens=16)


def _create(**kw):
    cfg = dict(BASE)
    cfg.update(kw)
    return m.moe_plan_create(**cfg)


@pytest.mark.parametrize("kw,status", [
    (dict(num_experts=0, top_k=0), m.MOE_ERR_INVALID),
    (dict(num_experts=8, top_k=0), m.MOE_ERR_INVALID),
    (dict(num_experts=-1, top_k=1), m.MOE_ERR_INVALID),
    (dict(top_k=9, num_experts=16), m.MOE_ERR_UNSUPPORTED),
    (dict(top_k=3, num_experts=2), m.MOE_ERR_INVALID),
    (dict(num_experts=257), m.MOE_ERR_UNSUPPORTED),
    (dict(hidden=0), m.MOE_ERR_INVALID),
    (dict(hidden=100), m.MOE_ERR_UNSUPPORTED),
    (dict(expert_inter=48), m.MOE_ERR_UNSUPPORTED),
    (dict(shared_inter=-32), m.MOE_ERR_INVALID),
    (dict(shared_inter=40), m.MOE_ERR_UNSUPPORTED),
    (dict(max_tokens=0), m.MOE_ERR_INVALID),
    (dict(bias_mode=3), m.MOE_ERR_INVALID),
    (dict(swiglu_limit=-1.0), m.MOE_ERR_INVALID),
    (dict(rms_eps=-1e-6), m.MOE_ERR_INVALID),
    (dict(x_dtype=m.MOE_Q8_0), m.MOE_ERR_UNSUPPORTED),
    (dict(expert_dtype=7), m.MOE_ERR_INVALID),
    (dict(shared_inter=64, shared_dtype=m.MOE_Q8_0), m.MOE_ERR_UNSUPPORTED),
    (dict(path=5), m.MOE_ERR_INVALID),
    (dict(select=3), m.MOE_ERR_INVALID),
    (dict(select=m.MOE_SIGMOID_NORM, bias_mode=m.MOE_BIAS_LOGIT), m.MOE_ERR_UNSUPPORTED),
    (dict(path=m.MOE_PATH_MFMA, x_dtype=m.MOE_F32), m.MOE_ERR_UNSUPPORTED),
    (dict(path=m.MOE_PATH_MFMA, expert_dtype=m.MOE_F32), m.MOE_ERR_UNSUPPORTED),
    (dict(x_dtype=m.MOE_MXFP4), m.MOE_ERR_UNSUPPORTED),
    (dict(router_dtype=m.MOE_MXFP4), m.MOE_ERR_UNSUPPORTED),
    (dict(shared_inter=64, expert_dtype=m.MOE_MXFP4, shared_dtype=m.MOE_Q8_0), m.MOE_ERR_UNSUPPORTED),
    (dict(path=m.MOE_PATH_MFMA, expert_dtype=m.MOE_MXFP4, hidden=288), m.MOE_ERR_UNSUPPORTED),
])
def test_plan_refusals(kw, status):
    with pytest.raises(m.MoeError) as ei:
        _create(**kw)
    assert ei.value.status == status, str(ei.value)


def test_plan_accepts_every_workload_shape():
    import synth
    for spec in synth.SPECS.values():
        p = m.moe_plan_create(spec.hidden, spec.num_experts, spec.top_k, spec.expert_inter,
                              spec.shared_inter, max(spec.token_counts), spec.select,
                              spec.bias_mode, spec.swiglu_limit, spec.rms_eps, spec.x_dtype,
                              spec.router_dtype, spec.expert_dtype, spec.shared_dtype)
        for M in spec.token_counts:
            assert m.moe_workspace_bytes(p, M) > 0


def test_workspace_sizes():
    p = _create(shared_inter=0)
    assert m.moe_workspace_bytes(p, 0) == 0
    assert m.moe_workspace_bytes(p, 17) == 0            # beyond max_tokens
    sizes = [m.moe_workspace_bytes(p, M) for M in range(1, 17)]
    assert all(b > a for a, b in zip(sizes, sizes[1:]))
    assert all(s % 256 == 0 for s in sizes)
    with_shared = _create(shared_inter=1024)
    assert m.moe_workspace_bytes(with_shared, 4) > m.moe_workspace_bytes(p, 4)


FAKE = 1 << 40  # a 256-byte-aligned address; never dereferenced (validation fails first)


def test_call_refusals_before_any_launch():
    p = _create()
    w = m.make_weights(router=FAKE, gate=FAKE, up=FAKE, down=FAKE)
    need = m.moe_workspace_bytes(p, 4)
    L = m.lib()
    st = L.moe_forward(p.handle, FAKE, ctypes.byref(w), 17, FAKE, None, None, None, FAKE, need, None)
    assert st == m.MOE_ERR_INVALID and "max_tokens" in m.moe_last_error()
    st = L.moe_forward(p.handle, FAKE, ctypes.byref(w), 4, FAKE, None, None, None, FAKE, need - 1, None)
    assert st == m.MOE_ERR_WORKSPACE
    st = L.moe_forward(p.handle, None, ctypes.byref(w), 4, FAKE, None, None, None, FAKE, need, None)
    assert st == m.MOE_ERR_INVALID and "x" in m.moe_last_error()
    st = L.moe_forward(p.handle, FAKE + 8, ctypes.byref(w), 4, FAKE, None, None, None, FAKE, need, None)
    assert st == m.MOE_ERR_INVALID and "aligned" in m.moe_last_error()
    st = L.moe_forward(p.handle, FAKE, ctypes.byref(w), 4, FAKE, None, None, None, FAKE + 16, need, None)
    assert st == m.MOE_ERR_INVALID
    nodown = m.make_weights(router=FAKE, gate=FAKE, up=FAKE)
    st = L.moe_forward(p.handle, FAKE, ctypes.byref(nodown), 4, FAKE, None, None, None, FAKE, need, None)
    assert st == m.MOE_ERR_INVALID and "down" in m.moe_last_error()
    # M = 0 is a no-op even with NULL buffers
    assert L.moe_forward(p.handle, None, ctypes.byref(w), 0, None, None, None, None, None, 0, None) == m.MOE_OK
    # bias required when the plan has a bias mode
    pb = _create(bias_mode=m.MOE_BIAS_LOGIT)
    st = L.moe_route(pb.handle, FAKE, ctypes.byref(w), 4, None, 0, FAKE, FAKE, FAKE,
                     m.moe_workspace_bytes(pb, 4), None)
    assert st == m.MOE_ERR_INVALID and "bias" in m.moe_last_error()
    # Q8_0 needs its scale planes
    pq = _create(expert_dtype=m.MOE_Q8_0)
    st = L.moe_expert_ffn(pq.handle, FAKE, ctypes.byref(w), 4, FAKE, FAKE, FAKE, FAKE,
                          m.moe_workspace_bytes(pq, 4), None)
    assert st == m.MOE_ERR_INVALID and "scale" in m.moe_last_error()
    # the INT8 router: Q8_0 router rows need their scale plane; the input
    # scale, when given, must be 16-byte aligned
    pr = _create(router_dtype=m.MOE_Q8_0)
    needr = m.moe_workspace_bytes(pr, 4)
    st = L.moe_route(pr.handle, FAKE, ctypes.byref(w), 4, None, 0, FAKE, FAKE, FAKE, needr, None)
    assert st == m.MOE_ERR_INVALID and "router_scale" in m.moe_last_error()
    wr = m.make_weights(router=FAKE, router_scale=FAKE, router_x_scale=FAKE + 8, gate=FAKE, up=FAKE, down=FAKE)
    st = L.moe_route(pr.handle, FAKE, ctypes.byref(wr), 4, None, 0, FAKE, FAKE, FAKE, needr, None)
    assert st == m.MOE_ERR_INVALID and "router_x_scale" in m.moe_last_error()
    # unknown route flags
    st = L.moe_route(p.handle, FAKE, ctypes.byref(w), 4, None, 6, FAKE, FAKE, FAKE, need, None)
    assert st == m.MOE_ERR_INVALID
    # combine output may not alias act
    st = L.moe_combine(p.handle, FAKE, ctypes.byref(w), 4, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                       FAKE, need, None)
    assert st == m.MOE_ERR_INVALID and "alias" in m.moe_last_error()
    assert L.moe_q8_0_split(FAKE, 4, 33, FAKE, FAKE, None) == m.MOE_ERR_INVALID
    assert L.moe_q8_0_split(FAKE, -1, 32, FAKE, FAKE, None) == m.MOE_ERR_INVALID
    assert L.moe_q8_0_split(None, 0, 32, None, None, None) == m.MOE_OK
    # MXFP4 needs its scale planes (2-byte aligned) and code planes 16-byte aligned
    px = _create(expert_dtype=m.MOE_MXFP4)
    st = L.moe_expert_ffn(px.handle, FAKE, ctypes.byref(w), 4, FAKE, FAKE, FAKE, FAKE,
                          m.moe_workspace_bytes(px, 4), None)
    assert st == m.MOE_ERR_INVALID and "scale" in m.moe_last_error()
    unaligned = m.make_weights(router=FAKE, gate=FAKE + 8, up=FAKE, down=FAKE, gate_scale=FAKE + 1,
                               up_scale=FAKE + 3, down_scale=FAKE + 5)
    assert m.moe_workspace_bytes(px, 4) > 0
    st = L.moe_expert_ffn(px.handle, FAKE, ctypes.byref(unaligned), 4, FAKE, FAKE, FAKE, FAKE,
                          m.moe_workspace_bytes(px, 4), None)
    assert st == m.MOE_ERR_INVALID and "gate" in m.moe_last_error()
    odd = m.make_weights(router=FAKE, gate=FAKE, up=FAKE, down=FAKE, gate_scale=FAKE + 2,
                         up_scale=FAKE + 1, down_scale=FAKE + 4)
    st = L.moe_expert_ffn(px.handle, FAKE, ctypes.byref(odd), 4, FAKE, FAKE, FAKE, FAKE,
                          m.moe_workspace_bytes(px, 4), None)
    assert st == m.MOE_ERR_INVALID and "up_scale" in m.moe_last_error()
    assert m.MOE_RUN_NAMES[m.moe_forward_path(px, 1)] == "single"
    assert L.moe_mxfp4_split(FAKE, 4, 48, FAKE, FAKE, None) == m.MOE_ERR_INVALID
    assert L.moe_mxfp4_split(FAKE, -1, 32, FAKE, FAKE, None) == m.MOE_ERR_INVALID
    assert L.moe_mxfp4_split(FAKE, 4, 32, FAKE + 8, FAKE, None) == m.MOE_ERR_INVALID
    assert L.moe_mxfp4_split(None, 0, 32, None, None, None) == m.MOE_OK
    # fused neighbours: a norm weight needs the pre-norm on; weight and
    # residual must be 16-byte aligned; NULL for both is moe_forward
    st = L.moe_forward_fused(p.handle, FAKE, FAKE, None, ctypes.byref(w), 4, FAKE, None, None, None,
                             FAKE, need, None)
    assert st == m.MOE_ERR_INVALID and "rms_eps" in m.moe_last_error()
    pn = _create(rms_eps=1e-6)
    needn = m.moe_workspace_bytes(pn, 4)
    assert needn >= need + 4 * 256 * 4
    st = L.moe_forward_fused(pn.handle, FAKE, FAKE + 8, None, ctypes.byref(w), 4, FAKE, None, None, None,
                             FAKE, needn, None)
    assert st == m.MOE_ERR_INVALID and "norm_weight" in m.moe_last_error()
    st = L.moe_forward_fused(pn.handle, FAKE, FAKE, FAKE + 4, ctypes.byref(w), 4, FAKE, None, None, None,
                             FAKE, needn, None)
    assert st == m.MOE_ERR_INVALID and "residual" in m.moe_last_error()
    st = L.moe_forward_fused(pn.handle, FAKE, FAKE, FAKE, ctypes.byref(w), 4, FAKE, None, None, None,
                             FAKE, needn - 1, None)
    assert st == m.MOE_ERR_WORKSPACE
    assert L.moe_forward_fused(pn.handle, None, None, None, ctypes.byref(w), 0, None, None, None, None,
                               None, 0, None) == m.MOE_OK


def test_forward_path_choice():
    import synth
    # the grouped GEMM from two routes per expert (four with Q8_0 experts):
    # Mixtral M=16: 4, DeepSeek M=16: 1.5, gpt-oss (Q8_0) M=16: 2
    want = {("gpt-oss-20b", 1): "single", ("gpt-oss-20b", 16): "gemv",
            ("mixtral-8x7b", 1): "single", ("mixtral-8x7b", 16): "mfma", ("mixtral-8x7b", 512): "mfma",
            ("qwen3-30b-a3b", 2048): "mfma", ("deepseek-v2-lite", 16): "gemv",
            ("gpt-oss-20b-mxfp4", 1): "single", ("gpt-oss-20b-mxfp4", 16): "gemv"}
    for (name, M), run in want.items():
        spec = synth.SPECS[name]
        p = m.moe_plan_create(spec.hidden, spec.num_experts, spec.top_k, spec.expert_inter,
                              spec.shared_inter, max(spec.token_counts), spec.select,
                              spec.bias_mode, spec.swiglu_limit, spec.rms_eps, spec.x_dtype,
                              spec.router_dtype, spec.expert_dtype, spec.shared_dtype)
        assert m.MOE_RUN_NAMES[m.moe_forward_path(p, M)] == run, (name, M)
        with pytest.raises(m.MoeError):
            m.moe_forward_path(p, 0)
        with pytest.raises(m.MoeError):
            m.moe_forward_path(p, max(spec.token_counts) + 1)
    mix = synth.SPECS["mixtral-8x7b"]
    forced = m.moe_plan_create(mix.hidden, mix.num_experts, mix.top_k, mix.expert_inter, 0, 512,
                               mix.select, mix.bias_mode, mix.swiglu_limit, mix.rms_eps,
                               mix.x_dtype, mix.router_dtype, mix.expert_dtype, mix.shared_dtype,
                               path=m.MOE_PATH_GEMV)
    assert m.moe_forward_path(forced, 512) == 1
    assert m.lib().moe_forward_path(None, 1) == -1
