"""GPU parity of the whole decode step (stacked MoE layers with the RMS norm
between them, then the FP8 head), checked layer by layer with teacher forcing:
each layer's oracle check consumes the GPU's own residual stream h_l and
normalized input u_l, so no stage inherits another stage's rounding."""

import numpy as np
import pytest
import torch

from oracle import compare as C
from oracle import head as OH
from oracle import moe as OM
from weight_streaming_expert_amd import configs, inputs
import parity as P

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from weight_streaming_expert_amd import ops as _ops
    return _ops


def build_stack(ops, wl, L):
    layers = [inputs.layer_weights(wl, l) for l in range(L)]
    st = lambda key: P.to_dev(np.stack([lw[key] for lw in layers]))
    r = np.stack([lw["router"] for lw in layers])
    router = P.to_dev(r) if r.dtype == np.float32 else P.to_dev_bf16(r)
    shared = tuple(P.to_dev(np.stack([lw["shared"][i] for lw in layers])) for i in range(4))
    stack = ops.MoeStackTensors(router, st("w13c"), st("w13s"), st("w2c"), st("w2s"), shared=shared, k=wl.moe.k)
    return layers, stack


def check_step(wl, layers, out, head_q, head_s, h0):
    m = wl.moe
    ht, ut = P.bits(out["h_trace"]), P.bits(out["u_trace"])
    ids, ws = P.np_(out["ids_trace"]), P.np_(out["w_trace"])
    assert np.array_equal(ht[0], h0)
    for l, lw in enumerate(layers):
        P.check_norm(ht[l], ut[l])
        P.check_routing(ut[l], P.router_values(lw["router"]), m.k, ids[l], ws[l])
        get = lambda e, lw=lw: (lw["w13c"][e], lw["w13s"][e], lw["w2c"][e], lw["w2s"][e])
        y_ref = P.moe_y_ref(ut[l], ids[l], ws[l], get, lw["shared"], m.I)
        P.check_h_next(ht[l], y_ref, ht[l + 1])
    L = len(layers)
    P.check_norm(ht[L], ut[L])
    assert np.array_equal(P.bits(out["h"]), ht[L])
    return P.check_head(head_q, head_s, ut[L], P.np_(out["logits"]), P.np_(out["argmax"]))


@pytest.mark.parametrize("T", [1, 2, 3, 4])
def test_tiny_stack_decode_step(ops, T):
    wl = configs.TINY
    L = 3
    layers, stack = build_stack(ops, wl, L)
    head_w = inputs.head_weights(wl, K=wl.moe.H)
    head = ops.Fp8LmHead.quantize(P.to_dev_bf16(head_w))
    qh, sh = P.np_(head.q), P.np_(head.s)
    for step in range(3):
        h0 = inputs.normal_bf16((wl.seed, inputs.T_X, step, T), (T, wl.moe.H), 1.0)
        out = ops.moe_decode_step(P.to_dev_bf16(h0), stack, head, trace=True)
        check_step(wl, layers, out, qh, sh, h0)
        plain = ops.moe_decode_step(P.to_dev_bf16(h0), stack, head, trace=False)
        assert torch.equal(plain["h"], out["h"]) and torch.equal(plain["argmax"], out["argmax"])
        assert torch.equal(plain["logits"], out["logits"])


@pytest.fixture(scope="module")
def ling_stack(ops):
    wl = configs.DECODE_STEP
    L = 2
    layers, stack = build_stack(ops, wl, L)
    head_w = inputs.head_weights(configs.LM_HEAD)
    head = ops.Fp8LmHead.quantize(P.to_dev_bf16(head_w))
    torch.cuda.synchronize()
    return wl, layers, stack, head, P.np_(head.q), P.np_(head.s)


@pytest.mark.parametrize("T", [1, 2, 3, 4])
def test_ling_shape_stack_decode_step(ops, ling_stack, T):
    wl, layers, stack, head, qh, sh = ling_stack
    for step in range(2):
        h0 = inputs.normal_bf16((wl.seed, inputs.T_X, step, T), (T, wl.moe.H), 1.0)
        out = ops.moe_decode_step(P.to_dev_bf16(h0), stack, head, trace=True)
        check_step(wl, layers, out, qh, sh, h0)


def check_exact_ties(ids, logits):
    """Among exactly equal logits the lower id is selected first and ranks first."""
    for g, l in zip(np.atleast_2d(ids), np.atleast_2d(logits)):
        for a, b in zip(g[:-1], g[1:]):
            assert l[a] != l[b] or a < b, f"tied ids {a}, {b} out of order"
        sel = set(int(e) for e in g)
        for s in sel:
            tied = np.flatnonzero(l == l[s])
            assert all(int(e) in sel for e in tied if e < s), f"id {s} chosen over a lower tied id"


@pytest.mark.parametrize("T", [1, 4])
def test_fused_routing_exact_ties(ops, ling_stack, T):
    """Repeated router rows give exactly tied logits: in layer 0 row e equals row
    e % 64, so each value has eight copies in eight different groups of eight
    ids; in layer 1 row e equals row e - e % 2, a tied pair inside each group.
    The fused step picks and ranks tied experts by lower id ([genai] and [sns],
    the router's top-k; ties are ordered by lower id)."""
    wl, layers, stack, head, qh, sh = ling_stack
    E = wl.moe.E
    idx = (np.arange(E) % 64, np.arange(E) - np.arange(E) % 2)
    tied = [dict(lw, router=lw["router"][ix].copy()) for lw, ix in zip(layers, idx)]
    r = np.stack([lw["router"] for lw in tied])
    router = P.to_dev(r) if r.dtype == np.float32 else P.to_dev_bf16(r)
    st = ops.MoeStackTensors(router, stack.w13_codes, stack.w13_scales, stack.w2_codes, stack.w2_scales,
                             shared=stack.shared, k=stack.k)
    h0 = inputs.normal_bf16((wl.seed, inputs.T_X, 7, T), (T, wl.moe.H), 1.0)
    out = ops.moe_decode_step(P.to_dev_bf16(h0), st, head, trace=True)
    check_step(wl, tied, out, qh, sh, h0)
    ut, ids = P.bits(out["u_trace"]), P.np_(out["ids_trace"])
    for l, lw in enumerate(tied):
        ref = OM.router_logits(ut[l], P.router_values(lw["router"]))
        check_exact_ties(ids[l], ref)
        if l == 0:   # the eight copies of the best value fill the top k
            for t in range(T):
                assert np.all(ids[l][t] % 64 == ids[l][t][0] % 64)
                assert np.all(np.diff(ids[l][t]) == 64)


def test_decode_step_is_deterministic(ops, ling_stack):
    wl, layers, stack, head, qh, sh = ling_stack
    h0 = P.to_dev_bf16(inputs.normal_bf16((3,), (1, wl.moe.H), 1.0))
    a = ops.moe_decode_step(h0, stack, head)
    for _ in range(10):
        b = ops.moe_decode_step(h0, stack, head)
        assert torch.equal(a["h"], b["h"]) and torch.equal(a["logits"], b["logits"])


def test_fused_step_many_consecutive_calls(ops, ling_stack):
    """The single-launch step keeps a per-workspace epoch; consecutive calls on
    one workspace (with and without traces, plain and captured in a graph) must
    all complete without a failed wait and give identical results for
    identical inputs."""
    wl, layers, stack, head, qh, sh = ling_stack
    H = wl.moe.H
    ws = ops.workspace(ops.decode_step_workspace_bytes(1, H, wl.moe.I, wl.moe.E, wl.moe.k, head.V), "cuda")
    xs = [P.to_dev_bf16(inputs.normal_bf16((wl.seed, 77, s), (1, H), 1.0)) for s in range(3)]
    first = [ops.moe_decode_step(x, stack, head, ws=ws) for x in xs]
    torch.cuda.synchronize()
    for o in first:
        assert int(o["argmax"][0]) >= 0
    for rep in range(20):
        for x, f in zip(xs, first):
            o = ops.moe_decode_step(x, stack, head, ws=ws, trace=(rep % 5 == 0))
            assert torch.equal(o["h"], f["h"]) and torch.equal(o["logits"], f["logits"])
            assert torch.equal(o["argmax"], f["argmax"])
    # replayed from a captured graph, with eager work between replays
    h_in = torch.empty_like(xs[0])
    out = dict(h=torch.empty_like(xs[0]), logits=torch.empty_like(first[0]["logits"]),
               argmax=torch.empty_like(first[0]["argmax"]))
    h_in.copy_(xs[0])
    ops.moe_decode_step(h_in, stack, head, ws=ws, out=out)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ops.moe_decode_step(h_in, stack, head, ws=ws, out=out)
    for rep in range(6):
        i = rep % 3
        h_in.copy_(xs[i])
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out["argmax"], first[i]["argmax"]) and torch.equal(out["h"], first[i]["h"])
        assert torch.equal(out["logits"], first[i]["logits"])
        ops.moe_decode_step(xs[(i + 1) % 3], stack, head, ws=ws)     # eager call between replays


def test_same_workspace_decode_and_verify_passes(ops):
    """One workspace serves 1-token steps (single launch) and 4-token verify
    passes (per-phase launches) alternately."""
    wl = configs.TINY
    layers, stack = build_stack(ops, wl, 2)
    head = ops.Fp8LmHead.quantize(P.to_dev_bf16(inputs.head_weights(wl, K=wl.moe.H)))
    qh, sh = P.np_(head.q), P.np_(head.s)
    H = wl.moe.H
    ws = ops.workspace(ops.decode_step_workspace_bytes(4, H, wl.moe.I, wl.moe.E, wl.moe.k, head.V), "cuda")
    for step in range(4):
        T = 1 if step % 2 == 0 else 4
        h0 = inputs.normal_bf16((wl.seed, 55, step), (T, H), 1.0)
        out = ops.moe_decode_step(P.to_dev_bf16(h0), stack, head, trace=True, ws=ws)
        check_step(wl, layers, out, qh, sh, h0)


@pytest.mark.parametrize("shape", ["ling", "tiny"])
def test_failed_wait_reports_minus_one_and_does_not_carry_over(ops, ling_stack, shape):
    """The one-launch step's failure report, forced from the host.  The step's
    error word (workspace bytes 256..259: the line after the 256-byte epoch
    line) is preset to the tag base of the next step, (epoch + 1) << 8.  Every
    wait of that step then gives up within 16 polls, every workgroup still runs
    to its end, and the step reports argmax -1.  The error word is clear
    afterwards, the epoch has advanced, and the next step on the same workspace
    gives the normal result bit for bit."""
    if shape == "ling":
        wl, layers, stack, head, qh, sh = ling_stack
    else:
        wl = configs.TINY
        layers, stack = build_stack(ops, wl, 2)
        head = ops.Fp8LmHead.quantize(P.to_dev_bf16(inputs.head_weights(wl, K=wl.moe.H)))
    m = wl.moe
    ws = ops.workspace(ops.decode_step_workspace_bytes(1, m.H, m.I, m.E, m.k, head.V), "cuda")
    x = P.to_dev_bf16(inputs.normal_bf16((wl.seed, 91), (1, m.H), 1.0))
    ref = ops.moe_decode_step(x, stack, head, ws=ws)
    torch.cuda.synchronize()
    assert int(ref["argmax"][0]) >= 0
    ref = {key: v.clone() for key, v in ref.items()}
    ctl = ws[:512].view(torch.int32)
    epoch = int(ctl[0])
    ctl[64] = (epoch + 1) << 8
    bad = ops.moe_decode_step(x, stack, head, ws=ws)
    torch.cuda.synchronize()
    assert int(bad["argmax"][0]) == -1
    assert int(ctl[64]) == 0 and int(ctl[0]) == epoch + 1
    again = ops.moe_decode_step(x, stack, head, ws=ws)
    torch.cuda.synchronize()
    for key in ("h", "logits", "argmax"):
        assert torch.equal(again[key], ref[key]), key
