"""GPU parity of the grouped MoE layer for a small batch or a longer draft
(5 <= T <= 16 tokens): the router's per-token top-k, the compact expert list
(up to T*k distinct experts, ascending) and slot-weight table, and the
experts over expert-sorted token lists (each active expert's tokens are those
with a nonzero weight in its slot row), in bf16 and W4A8; at the tiny shape
(16 experts, so every expert serves many tokens) and the Ling shape (512
experts top-8, up to 128 distinct experts)."""

import numpy as np
import pytest
import torch

from oracle import compare as C
from oracle import formats as F
from oracle import moe as OM
from weight_streaming_expert_amd import configs, inputs
import parity as P
from test_gpu_moe import check_layer, run_layer
from test_gpu_w4a8 import check_w4a8, run_w4a8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from weight_streaming_expert_amd import ops as _ops
    return _ops


@pytest.fixture(scope="module")
def tiny(ops):
    wl = configs.TINY
    lw = inputs.layer_weights(wl, 0)
    return wl, lw, P.layer_to_dev(lw)


@pytest.fixture(scope="module")
def ling(ops):
    wl = configs.MOE_LAYER
    lw = inputs.layer_weights(wl, 0)
    return wl, lw, P.layer_to_dev(lw)


@pytest.mark.parametrize("T", [5, 8, 13, 16])
def test_grouped_tiny_layer(ops, tiny, T):
    wl, lw, dw = tiny
    for step in range(2):
        x = inputs.normal_bf16((wl.seed, 81, step, T), (T, wl.moe.H), 1.0)
        res = inputs.normal_bf16((wl.seed, 82, step, T), (T, wl.moe.H), 1.0)
        r, y, h = run_layer(ops, wl, dw, x, res)
        assert int(r["expert_list"][0]) <= wl.moe.E
        check_layer(wl, lw, x, res, r, y, h)


@pytest.mark.parametrize("T", [8, 16])
def test_grouped_ling_layer(ops, ling, T):
    wl, lw, dw = ling
    x = inputs.normal_bf16((wl.seed, 83, T), (T, wl.moe.H), 1.0)
    res = inputs.normal_bf16((wl.seed, 84, T), (T, wl.moe.H), 1.0)
    r, y, h = run_layer(ops, wl, dw, x, res)
    n = int(r["expert_list"][0])
    assert T * wl.moe.k // 2 <= n <= T * wl.moe.k
    check_layer(wl, lw, x, res, r, y, h)


def test_grouped_ling_overlapping_tokens(ops, ling):
    """16 tokens that are small perturbations of one another: many experts
    serve several tokens, so slot token lists run past one pass of four."""
    wl, lw, dw = ling
    T = 16
    base = inputs.normal_f32((wl.seed, 85), (1, wl.moe.H), 1.0)
    rows = base + inputs.normal_f32((wl.seed, 86), (T, wl.moe.H), 0.05)
    x = F.f64_to_bf16_rne(rows.astype(np.float64))
    res = inputs.normal_bf16((wl.seed, 87), (T, wl.moe.H), 1.0)
    r, y, h = run_layer(ops, wl, dw, x, res)
    sw = r["slot_w"].reshape(T * wl.moe.k, T)
    assert (sw > 0).sum(axis=1).max() > 4
    check_layer(wl, lw, x, res, r, y, h)


@pytest.mark.parametrize("T", [5, 16])
def test_grouped_planted_experts_bit_exact(ops, T):
    """The planted exact layer (tests/parity.py) with top-1 routing over 4
    experts and the shared expert: every product and sum is exact, so y must
    equal the rational result bit for bit for every token."""
    H, I, E = 2560, 768, 4
    c13, s13, c2, s2 = P.planted_exact_layer(H, I, E + 1, seed=T)
    wr = inputs.normal_f32((9, T), (E, H), 0.02)
    xi = np.random.default_rng(T).integers(1, 3, size=(T, H))
    x = torch.from_numpy(xi.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    xd = P.to_dev_bf16(x)
    r = ops.moe_route_topk(xd, P.to_dev(wr), 1)
    shared = tuple(P.to_dev(a[E]) for a in (c13, s13, c2, s2))
    y, _ = ops.moe_expert_gemv_mxfp4(xd, P.to_dev(c13[:E]), P.to_dev(s13[:E]), P.to_dev(c2[:E]), P.to_dev(s2[:E]),
                                     r["expert_list"], r["slot_w"], 1, shared=shared)
    ids = P.np_(r["topk_ids"])[:, 0]
    W = F.dequant_mxfp4(c13, s13, H)
    want = np.zeros((T, H))
    for t in range(T):
        for e in (ids[t], E):
            g = (W[e, :I] * 8).astype(np.int64) @ xi[t] / 8.0
            want[t, :I] += g * xi[t, np.arange(I) % H]
    assert np.array_equal(P.np_(y).astype(np.float64), want)


def test_grouped_router_ties_resolve_to_lowest_id(ops):
    """Duplicated router rows at T = 9: each token's ties go to the lower id,
    and the compact list holds each tied id once."""
    H, E, k, T = 256, 64, 8, 9
    w = inputs.normal_f32((10,), (E, H), 0.02)
    for dup in ([5, 9, 40], [60, 61, 62, 63]):
        w[dup] = w[dup[0]] + 1.0
    x = np.full((T, H), 0x3F80, dtype=np.uint16)
    r = ops.moe_route_topk(P.to_dev_bf16(x), P.to_dev(w), k)
    ids, lg = P.np_(r["topk_ids"]), P.np_(r["logits"])
    order = sorted(range(E), key=lambda e: (-lg[0, e], e))[:k]
    for t in range(T):
        assert list(ids[t]) == order
    el = P.np_(r["expert_list"])
    assert int(el[0]) == k and list(el[1:1 + k]) == sorted(order)


@pytest.mark.parametrize("T", [8, 16])
def test_grouped_w4a8_ling_layer(ops, ling, T):
    wl, lw, dw = ling
    x = inputs.normal_bf16((wl.seed, 88, T), (T, wl.moe.H), 1.0)
    res = inputs.normal_bf16((wl.seed, 89, T), (T, wl.moe.H), 1.0)
    check_w4a8(wl, lw, x, res, *run_w4a8(ops, wl, dw, x, res))


@pytest.mark.parametrize("T", [5, 13, 16])
def test_grouped_w4a8_tiny_layer(ops, tiny, T):
    """Above four tokens the W4A8 layer quantizes its input rows once, ahead of
    the gate/up workgroups: ragged token counts at the tiny shape."""
    wl, lw, dw = tiny
    for step in range(2):
        x = inputs.normal_bf16((wl.seed, 91, step, T), (T, wl.moe.H), 1.0)
        res = inputs.normal_bf16((wl.seed, 92, step, T), (T, wl.moe.H), 1.0)
        check_w4a8(wl, lw, x, res, *run_w4a8(ops, wl, dw, x, res))
