"""moe_forward_noalloc (the library's static scratch in place of a workspace)
against moe_forward, through the C ABI: two calls in a row, the second with
fewer tokens, on each kernel family; and the refusal beyond the scratch."""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from synth import BIAS_LOGIT, Q8_0, SOFTMAX_ALL_NORENORM
from gpu_helpers import check_ids, check_y, device_layer, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixture_experts_gemv_amd as m
    m.lib()
    yield


CASES = [
    # name, layer, path, (first M, second M): one-token, per-row and grouped-GEMM calls
    ("q8-bias-clamp", dict(hidden=288, num_experts=12, top_k=4, expert_inter=320, bias_mode=BIAS_LOGIT,
                           bias_kind="normal", swiglu_limit=7.0, expert_dtype=Q8_0), 0, (16, 1)),
    ("shared-all", dict(hidden=256, num_experts=16, top_k=6, expert_inter=160, shared_inter=320,
                        select=SOFTMAX_ALL_NORENORM), 1, (16, 5)),
    ("mfma-zipf-rms", dict(hidden=256, num_experts=64, top_k=8, expert_inter=128, bias_mode=BIAS_LOGIT,
                           bias_kind="zipf", rms_eps=1e-6), 2, (257, 65)),
]


@pytest.mark.parametrize("name,kw,path,Ms", CASES, ids=[c[0] for c in CASES])
def test_noalloc_matches_forward(name, kw, path, Ms):
    import mixture_experts_gemv_amd as m
    spec = synth.small_spec(name=name, seed=1700 + len(name), **kw)
    layer = synth.make_layer(spec)
    dl = device_layer(spec, layer, max(Ms), path=path)
    E, k, H = spec.num_experts, spec.top_k, spec.hidden
    for n, M in enumerate(Ms):
        x = synth.make_tokens(spec, M, batch=20 + n)
        xt = dl.x_tensor(x)
        say(f"noalloc {name} call {n}: M={M} ({m.MOE_RUN_NAMES[m.moe_forward_path(dl.plan, M)]})")
        ref_y = torch.empty(M, H, dtype=torch.float32, device="cuda")
        ref_ids = torch.empty(M, k, dtype=torch.int32, device="cuda")
        m.moe_forward(dl.plan, xt, dl.weights, M, ref_y, ref_ids, None, None, dl.workspace(M))
        y = torch.full((M, H), float("nan"), dtype=torch.float32, device="cuda")
        ids = torch.full((M, k), -1, dtype=torch.int32, device="cuda")
        w = torch.empty(M, k, dtype=torch.float32, device="cuda")
        counts = torch.empty(E, dtype=torch.int32, device="cuda")
        m.moe_forward_noalloc(dl.plan, xt, dl.weights, M, y, ids, w, counts)
        torch.cuda.synchronize()
        # the same kernels on the same inputs: identical to moe_forward
        assert torch.equal(ids, ref_ids), f"call {n}: ids differ from moe_forward"
        assert torch.equal(y, ref_y), f"call {n}: y differs from moe_forward"
        # and against the oracle, to the output tolerance
        o = oracle.forward(spec, layer, x)
        forced, near = check_ids(spec, layer, x, ids.cpu().numpy(), o["ids"])
        if near:
            o = oracle.forward(spec, layer, x, forced_ids=forced)
        assert np.array_equal(counts.cpu().numpy(), np.bincount(forced.reshape(-1), minlength=E))
        check_y(y.cpu().numpy(), o["y"], f"noalloc {name} M={M}")


def test_noalloc_refuses_beyond_scratch():
    """A call whose workspace would exceed the static scratch is refused
    before anything runs, and leaves y untouched."""
    import mixture_experts_gemv_amd as m
    plan = m.moe_plan_create(2048, 128, 8, 768, max_tokens=2048, path=m.MOE_PATH_MFMA)
    need = m.moe_workspace_bytes(plan, 2048)
    assert need > 32 << 20
    y = torch.full((2048, 2048), 3.0, dtype=torch.float32, device="cuda")
    wts = m.make_weights()
    with pytest.raises(m.MoeError) as err:
        m.moe_forward_noalloc(plan, y, wts, 2048, y, None, None, None)
    assert err.value.status == m.MOE_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((y == 3.0).all())
