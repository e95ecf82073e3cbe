"""GPU checks of what the layer must not do: write outside its buffers, or let
one token's result depend on the other tokens of its batch.

Canaries: every output buffer and the workspace are carved out of a larger
allocation whose bytes before and after them hold a known pattern; after the
calls the pattern must be intact.  An undersized scratch region silently
overwrites whatever was allocated next to it (deepseek2/state.rs,
RealDeepseek2State.ffn_a doc), which only a check like this catches.  The
workspace itself is filled with 0xff bytes (NaN as fp32) before each call, so
a kernel that reads a workspace region before writing it shows up as a
changed result.

Token independence (pin P8 on the HIP path): each token computed alone gives
the same expert set as inside its batch (bar near-tie tokens) and y within
the output tolerance, and the per-expert counts of a batch are the sums of its
sub-batches' counts.
"""

from __future__ import annotations

import numpy as np
import pytest

import synth
from gpu_helpers import Y_MAX_ABS, Y_REL_L2, device_layer, host_layer, say, selection_keys

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

GUARD = 4096     # bytes of pattern on each side (a multiple of 256 keeps alignment)
PATTERN = 0xA5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixture_experts_gemv_amd as m
    m.lib()
    yield


class Guarded:
    """A device buffer of ``nbytes`` between two pattern-filled guard regions."""

    def __init__(self, nbytes: int):
        self.nbytes = nbytes
        self.big = torch.full((GUARD + nbytes + GUARD,), PATTERN, dtype=torch.uint8, device="cuda")
        self.body = self.big[GUARD:GUARD + nbytes]

    def view(self, dtype, shape):
        return self.body.view(dtype).view(*shape)

    def check(self, what: str):
        torch.cuda.synchronize()
        head = self.big[:GUARD].cpu().numpy()
        tail = self.big[GUARD + self.nbytes:].cpu().numpy()
        bad_h = int((head != PATTERN).sum())
        bad_t = int((tail != PATTERN).sum())
        assert bad_h == 0 and bad_t == 0, \
            f"{what}: {bad_h} guard bytes before and {bad_t} after the buffer were overwritten"


def _ws(plan, M):
    import mixture_experts_gemv_amd as m
    g = Guarded(m.moe_workspace_bytes(plan, M))
    return g


def _fill_ws(plan, g):
    g.body.fill_(0xFF)


CANARY = [("gpt-oss-20b", 1), ("gpt-oss-20b", 16), ("gpt-oss-20b", 64),
          ("gpt-oss-20b-mxfp4", 1), ("gpt-oss-20b-mxfp4", 16), ("gpt-oss-20b-mxfp4", 256),
          ("deepseek-v2-lite", 1), ("deepseek-v2-lite", 16), ("qwen3-30b-a3b", 2048),
          ("gpt-oss-20b-int8-router", 16)]


@pytest.mark.parametrize("name,M", CANARY, ids=[f"{n}-M{m}" for n, m in CANARY])
def test_canaries_full_size(name, M):
    """moe_forward and moe_forward_fused (exact-size workspace, y, ids, w and
    counts between guards; the workspace pre-filled with 0xff) leave every
    guard intact and give the result of a call with fresh buffers."""
    import mixture_experts_gemv_amd as m
    say(f"canary {name} M={M}: generate")
    spec, layer = host_layer(name)
    dl = device_layer(spec, layer, M)
    x = dl.x_tensor(synth.make_tokens(spec, M, batch=2))
    E, k, H = spec.num_experts, spec.top_k, spec.hidden
    ref_y = dl.forward(x).clone()
    torch.cuda.synchronize()
    ws = _ws(dl.plan, M)
    gy = Guarded(M * H * 4)
    gids = Guarded(M * k * 4)
    gw = Guarded(M * k * 4)
    gc = Guarded(E * 4)
    y = gy.view(torch.float32, (M, H))
    ids = gids.view(torch.int32, (M, k))
    w = gw.view(torch.float32, (M, k))
    counts = gc.view(torch.int32, (E,))
    path = m.MOE_RUN_NAMES[m.moe_forward_path(dl.plan, M)]
    say(f"canary {name} M={M}: moe_forward ({path})")
    _fill_ws(dl.plan, ws)
    m.moe_forward(dl.plan, x, dl.weights, M, y, ids, w, counts, ws.body)
    for g, what in ((ws, "workspace"), (gy, "y"), (gids, "ids"), (gw, "w"), (gc, "counts")):
        g.check(f"{name} M={M} moe_forward {what}")
    assert torch.equal(y, ref_y), "result differs with a 0xff-filled exact-size workspace"
    # the fused call: norm weight where the layer has the pre-norm, residual in place
    nw = None
    if spec.rms_eps > 0:
        rng = np.random.default_rng(5)
        nw = dl.x_tensor(synth.bf16_bits(rng.uniform(0.25, 2.0, H).astype(np.float32)))
    res = torch.randn(M, H, dtype=torch.float32, device="cuda")
    ref_f = dl.forward_fused(x, norm_weight=nw, residual=res.clone()).clone()
    y.copy_(res)
    say(f"canary {name} M={M}: moe_forward_fused")
    _fill_ws(dl.plan, ws)
    m.moe_forward_fused(dl.plan, x, nw, y, dl.weights, M, y, ids, w, counts, ws.body)
    for g, what in ((ws, "workspace"), (gy, "y"), (gids, "ids"), (gw, "w"), (gc, "counts")):
        g.check(f"{name} M={M} moe_forward_fused {what}")
    assert torch.equal(y, ref_f), "fused result differs with a 0xff-filled exact-size workspace"
    del dl
    torch.cuda.empty_cache()


STAGES = [("gpt-oss-20b", 16), ("gpt-oss-20b", 64), ("deepseek-v2-lite", 16)]


@pytest.mark.parametrize("name,M", STAGES, ids=[f"{n}-M{m}" for n, m in STAGES])
def test_canaries_stages(name, M):
    """The stage-wise entry points with every output between guards."""
    import mixture_experts_gemv_amd as m
    say(f"stage canary {name} M={M}: generate")
    spec, layer = host_layer(name)
    dl = device_layer(spec, layer, M)
    x = dl.x_tensor(synth.make_tokens(spec, M, batch=4))
    E, k, H, I = spec.num_experts, spec.top_k, spec.hidden, spec.expert_inter
    R = M * k
    ws = _ws(dl.plan, M)
    _fill_ws(dl.plan, ws)
    g = {n: Guarded(b) for n, b in (("logits", M * E * 4), ("ids", R * 4), ("w", R * 4),
                                    ("counts", E * 4), ("offsets", (E + 1) * 4),
                                    ("sorted", R * 4), ("rpos", R * 4), ("act", R * I * 4),
                                    ("y", M * H * 4))}
    logits = g["logits"].view(torch.float32, (M, E))
    ids = g["ids"].view(torch.int32, (M, k))
    w = g["w"].view(torch.float32, (M, k))
    counts = g["counts"].view(torch.int32, (E,))
    offsets = g["offsets"].view(torch.int32, (E + 1,))
    sr = g["sorted"].view(torch.int32, (R,))
    rp = g["rpos"].view(torch.int32, (R,))
    act = g["act"].view(torch.float32, (R, I))
    y = g["y"].view(torch.float32, (M, H))
    say(f"stage canary {name} M={M}: route, permute, expert_ffn, combine")
    m.moe_route(dl.plan, x, dl.weights, M, logits, 0, ids, w, ws.body)
    m.moe_permute(dl.plan, ids, M, counts, offsets, sr, rp, ws.body)
    m.moe_expert_ffn(dl.plan, x, dl.weights, M, offsets, sr, act, ws.body)
    m.moe_combine(dl.plan, act, dl.weights, M, offsets, sr, rp, w, None, y, ws.body)
    for n, gg in g.items():
        gg.check(f"{name} M={M} stages {n}")
    ws.check(f"{name} M={M} stages workspace")
    assert torch.isfinite(y).all()
    del dl
    torch.cuda.empty_cache()


# ----------------------------------------------------------- token independence
INDEP = [("gpt-oss-20b", 16), ("gpt-oss-20b", 64), ("deepseek-v2-lite", 16),
         ("gpt-oss-20b-mxfp4", 256), ("qwen3-30b-a3b", 2048)]


@pytest.mark.parametrize("name,M", INDEP, ids=[f"{n}-M{m}" for n, m in INDEP])
def test_token_independence(name, M):
    """Each token alone (the one-token path) against the same token inside the
    batch (the batched path), and counts additive over two sub-batches."""
    import mixture_experts_gemv_amd as m
    say(f"independence {name} M={M}: generate")
    spec, layer = host_layer(name)
    dl = device_layer(spec, layer, M)
    xh = synth.make_tokens(spec, M, batch=6)
    E, k, H = spec.num_experts, spec.top_k, spec.hidden

    def run(xpart):
        n = xpart.shape[0]
        ids = torch.empty(n, k, dtype=torch.int32, device="cuda")
        cnt = torch.empty(E, dtype=torch.int32, device="cuda")
        y = dl.forward(dl.x_tensor(np.ascontiguousarray(xpart)), ids=ids, counts=cnt)
        return y, ids, cnt

    say(f"independence {name} M={M}: batch ({m.MOE_RUN_NAMES[m.moe_forward_path(dl.plan, M)]})")
    yb, idb, cb = run(xh)
    ws1 = dl.workspace(1)
    y1 = torch.empty(M, H, dtype=torch.float32, device="cuda")
    id1 = torch.empty(M, k, dtype=torch.int32, device="cuda")
    say(f"independence {name} M={M}: {M} one-token calls "
        f"({m.MOE_RUN_NAMES[m.moe_forward_path(dl.plan, 1)]})")
    xd = dl.x_tensor(xh)
    for t in range(M):
        m.moe_forward(dl.plan, xd[t:t + 1], dl.weights, 1, y1[t:t + 1], id1[t:t + 1], None, None, ws1)
    half = M // 2
    ya, ida, ca = run(xh[:half])
    yc, idc, cc = run(xh[half:])
    torch.cuda.synchronize()
    idb, id1 = idb.cpu().numpy(), id1.cpu().numpy()
    s, tau = selection_keys(spec, layer, xh)
    order = np.sort(s, axis=1)[:, ::-1]
    gap = order[:, k - 1] - (order[:, k] if k < E else -np.inf)
    near = gap <= 2 * tau
    same = np.array([set(idb[t]) == set(id1[t]) for t in range(M)])
    assert same[~near].all(), f"tokens {np.nonzero(~same & ~near)[0][:8]} change experts with the batch"
    say(f"independence {name} M={M}: {int(near.sum())} near-tie tokens, {int((~same).sum())} differ")
    yb_h, y1_h = yb.cpu().numpy()[same], y1.cpu().numpy()[same]
    err = np.abs(yb_h - y1_h)
    rel = np.linalg.norm(yb_h - y1_h) / np.linalg.norm(y1_h)
    say(f"independence {name} M={M}: alone vs batch max-abs {err.max():.3e}, rel-L2 {rel:.3e}")
    assert err.max() <= Y_MAX_ABS and rel <= Y_REL_L2
    # counts: each call's counts are its ids' histogram, and the halves add up
    # to the whole wherever the halves chose as the batch did
    cb, ca, cc = cb.cpu().numpy(), ca.cpu().numpy(), cc.cpu().numpy()
    assert np.array_equal(cb, np.bincount(idb.reshape(-1), minlength=E))
    ida, idc = ida.cpu().numpy(), idc.cpu().numpy()
    assert np.array_equal(ca, np.bincount(ida.reshape(-1), minlength=E))
    assert np.array_equal(cc, np.bincount(idc.reshape(-1), minlength=E))
    halves = np.concatenate([ida, idc])
    agree = np.array([set(halves[t]) == set(idb[t]) for t in range(M)])
    assert agree[~near].all()
    if agree.all():
        assert np.array_equal(cb, ca + cc), "counts are not additive over sub-batches"
    ya_h = np.concatenate([ya.cpu().numpy(), yc.cpu().numpy()])[agree]
    err = np.abs(ya_h - yb.cpu().numpy()[agree])
    assert err.max() <= Y_MAX_ABS
    del dl
    torch.cuda.empty_cache()
