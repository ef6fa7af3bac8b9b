"""GPU parity of one MoE layer: router + top-k + compact expert list, and the
MXFP4 routed + shared SwiGLU experts with the bf16 residual, at the tiny shape
(H=256, 16 experts top-2), at the Ling shape (H=2560, 512 experts top-8,
I=768) for 1 token and for the 4-token verify pass, plus exact planted cases,
ties, edge cases and determinism."""

import numpy as np
import pytest
import torch

from oracle import compare as C
from oracle import formats as F
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


def run_layer(ops, wl, dw, x_bits, res_bits):
    x = P.to_dev_bf16(x_bits)
    r = ops.moe_route_topk(x, dw["router"], wl.moe.k)
    y, h = ops.moe_expert_gemv_mxfp4(x, dw["w13c"], dw["w13s"], dw["w2c"], dw["w2s"], r["expert_list"], r["slot_w"],
                                     wl.moe.k, shared=dw["shared"], residual=P.to_dev_bf16(res_bits))
    return {k: P.np_(v) for k, v in r.items()}, P.np_(y), P.bits(h)


def check_layer(wl, lw, x_bits, res_bits, r, y, h):
    m = wl.moe
    ties = P.check_routing(x_bits, P.router_values(lw["router"]), m.k, r["topk_ids"], r["topk_w"],
                           r["expert_list"], r["slot_w"], r["logits"])
    get = lambda e: (lw["w13c"][e], lw["w13s"][e], lw["w2c"][e], lw["w2s"][e])
    y_ref = P.moe_y_ref(x_bits, r["topk_ids"], r["topk_w"], get, lw["shared"], m.I)
    ok, worst = C.fp_close(y, y_ref)
    assert ok, f"y off by {worst:.3e} x RMS"
    P.check_residual(res_bits, y, h)
    return ties, worst


# ----------------------------------------------------------------------------- tiny shape


@pytest.fixture(scope="module")
def tiny(ops):
    wl = configs.TINY
    lw = inputs.layer_weights(wl, 0)
    return wl, lw, P.layer_to_dev(lw)


@pytest.mark.parametrize("T", [1, 2, 3, 4])
def test_tiny_layer(ops, tiny, T):
    wl, lw, dw = tiny
    for step in range(4):
        x = inputs.normal_bf16((wl.seed, inputs.T_X, step, T), (T, wl.moe.H), 1.0)
        res = inputs.normal_bf16((wl.seed, 99, step, T), (T, wl.moe.H), 1.0)
        r, y, h = run_layer(ops, wl, dw, x, res)
        check_layer(wl, lw, x, res, r, y, h)


def test_tiny_handmade_expert_list_and_no_shared(ops, tiny):
    wl, lw, dw = tiny
    m = wl.moe
    T = 2
    x = inputs.normal_bf16((3, 1), (T, m.H), 1.0)
    ids = np.array([[3, 11], [11, 15]], dtype=np.int32)
    w = np.array([[0.75, 0.25], [0.5, 0.5]])
    el, sw = OM.expert_list(ids, w)
    el_dev = np.zeros(1 + T * m.k, dtype=np.int32)
    el_dev[0] = len(el)
    el_dev[1:1 + len(el)] = el
    sw_dev = np.zeros((T * m.k, T), dtype=np.float32)
    sw_dev[:len(el)] = sw
    for shared in (dw["shared"], None):
        yd, hd = ops.moe_expert_gemv_mxfp4(P.to_dev_bf16(x), dw["w13c"], dw["w13s"], dw["w2c"], dw["w2s"],
                                           P.to_dev(el_dev), P.to_dev(sw_dev), m.k, shared=shared)
        get = lambda e: (lw["w13c"][e], lw["w13s"][e], lw["w2c"][e], lw["w2s"][e])
        y_ref = P.moe_y_ref(x, ids, w, get, lw["shared"] if shared is not None else None, m.I)
        ok, worst = C.fp_close(P.np_(yd), y_ref)
        assert ok, worst
        assert hd is None


def test_one_token_handmade_lists_and_workspace_reuse(ops, tiny):
    """One token with a caller-built expert list: one workspace serves calls
    with 2, 1 and 0 routed slots and an out-of-range id (which contributes
    nothing), with and without the shared expert, each checked against the
    oracle and against the same call on a fresh workspace, bit for bit."""
    wl, lw, dw = tiny
    m = wl.moe
    dev = torch.device("cuda:0")
    ws = ops.workspace(ops.moe_workspace_bytes(1, m.H, m.I, m.E, m.k), dev)
    get = lambda e: (lw["w13c"][e], lw["w13s"][e], lw["w2c"][e], lw["w2s"][e])
    cases = (([3, 11], [0.75, 0.25]), ([5], [1.0]), ([], []), ([2, 99], [0.625, 0.375]), ([0, 15], [0.5, 0.5]))
    for i, (ids, wts) in enumerate(cases * 2):
        shared = dw["shared"] if i % 3 != 1 else None
        x = inputs.normal_bf16((3, 2, i), (1, m.H), 1.0)
        res = inputs.normal_bf16((3, 3, i), (1, m.H), 1.0)
        el_dev = np.zeros(1 + m.k, dtype=np.int32)
        el_dev[0] = len(ids)
        el_dev[1:1 + len(ids)] = ids
        sw_dev = np.zeros((m.k, 1), dtype=np.float32)
        sw_dev[:len(ids), 0] = wts
        args = (P.to_dev_bf16(x), dw["w13c"], dw["w13s"], dw["w2c"], dw["w2s"], P.to_dev(el_dev), P.to_dev(sw_dev),
                m.k)
        y, h = ops.moe_expert_gemv_mxfp4(*args, shared=shared, residual=P.to_dev_bf16(res), ws=ws)
        y1, h1 = ops.moe_expert_gemv_mxfp4(*args, shared=shared, residual=P.to_dev_bf16(res))
        y, h, y1, h1 = P.np_(y), P.bits(h), P.np_(y1), P.bits(h1)
        assert np.array_equal(y, y1) and np.array_equal(h, h1), (i, ids)
        valid = [(e, wt) for e, wt in zip(ids, wts) if 0 <= e < m.E]
        d = [OM.down(OM.gate_up(x, *get(e)[:2], m.I), *get(e)[2:]) for e, _ in valid]
        d = np.stack(d) if d else np.zeros((0, 1, m.H))
        sw_ref = np.array([[wt] for _, wt in valid]).reshape(len(valid), 1)
        sh = lw["shared"]
        d_sh = OM.down(OM.gate_up(x, sh[0], sh[1], m.I), sh[2], sh[3]) if shared is not None else None
        y_ref = OM.combine(d, sw_ref, d_sh)
        if not valid and shared is None:
            assert np.array_equal(y, np.zeros_like(y)), (i, ids)
        else:
            ok, worst = C.fp_close(y, y_ref)
            assert ok, (i, ids, worst)
        P.check_residual(res, y, h)


@pytest.mark.parametrize("shape", ["tiny", "ling"])
def test_four_tokens_handmade_lists_and_workspace_reuse(ops, tiny, ling, shape):
    """Four tokens with caller-built expert-sorted token lists (one launch for
    gate/up and down, whose slot counters must be back at zero after every
    call): one workspace serves lists with shared and unshared slots, an
    out-of-range id (which contributes nothing), a full list and an empty
    one, with and without the shared expert, each checked against the oracle
    and against the same call on a fresh workspace, bit for bit."""
    wl, lw, dw = tiny if shape == "tiny" else ling
    m = wl.moe
    T = 4
    dev = torch.device("cuda:0")
    ws = ops.workspace(ops.moe_workspace_bytes(T, m.H, m.I, m.E, m.k), dev)
    get = lambda e: (lw["w13c"][e], lw["w13s"][e], lw["w2c"][e], lw["w2s"][e])
    rng = np.random.default_rng(17)
    full = sorted(rng.choice(m.E, size=T * m.k, replace=False).tolist())
    cases = (
        [(1, {0: 0.5, 1: 0.25}), (4, {2: 1.0}), (7, {0: 0.5, 3: 0.75}), (12, {1: 0.25, 2: 0.5}), (m.E + 5, {1: 0.5})],
        [],
        [(e, {t: 1.0 / m.k for t in range(T) if (i + t) % T == 0 or m.k > 2}) for i, e in enumerate(full)],
        [(0, {0: 1.0, 1: 1.0, 2: 1.0, 3: 1.0})],
    )
    for i, case in enumerate(cases * 2):
        shared = dw["shared"] if i % 3 != 1 else None
        x = inputs.normal_bf16((4, 2, i), (T, m.H), 1.0)
        res = inputs.normal_bf16((4, 3, i), (T, m.H), 1.0)
        el = np.zeros(1 + T * m.k, dtype=np.int32)
        el[0] = len(case)
        sw = np.zeros((T * m.k, T), dtype=np.float32)
        for s, (e, tw) in enumerate(case):
            el[1 + s] = e
            for t, wt in tw.items():
                sw[s, t] = wt
        args = (P.to_dev_bf16(x), dw["w13c"], dw["w13s"], dw["w2c"], dw["w2s"], P.to_dev(el), P.to_dev(sw), m.k)
        y, h = ops.moe_expert_gemv_mxfp4(*args, shared=shared, residual=P.to_dev_bf16(res), ws=ws)
        y1, h1 = ops.moe_expert_gemv_mxfp4(*args, shared=shared, residual=P.to_dev_bf16(res))
        y, h, y1, h1 = P.np_(y), P.bits(h), P.np_(y1), P.bits(h1)
        assert np.array_equal(y, y1) and np.array_equal(h, h1), (shape, i)
        valid = [s for s, (e, _) in enumerate(case) if 0 <= e < m.E]
        d = [OM.down(OM.gate_up(x, *get(case[s][0])[:2], m.I), *get(case[s][0])[2:]) for s in valid]
        d = np.stack(d) if d else np.zeros((0, T, m.H))
        sh = lw["shared"]
        d_sh = OM.down(OM.gate_up(x, sh[0], sh[1], m.I), sh[2], sh[3]) if shared is not None else None
        y_ref = OM.combine(d, sw[valid].astype(np.float64).reshape(len(valid), T), d_sh)
        if not valid and shared is None:
            assert np.array_equal(y, np.zeros_like(y)), (shape, i)
        else:
            ok, worst = C.fp_close(y, y_ref)
            assert ok, (shape, i, worst)
        P.check_residual(res, y, h)


def test_router_ties_resolve_to_lowest_id(ops):
    H, E, k = 256, 64, 8
    w = inputs.normal_f32((4,), (E, H), 0.02)
    for dup in ([5, 9, 40], [60, 61, 62, 63]):
        w[dup] = w[dup[0]] + 1.0                            # identical rows with the largest logits
    x = np.full((2, H), 0x3F80, dtype=np.uint16)
    r = ops.moe_route_topk(P.to_dev_bf16(x), P.to_dev(w), k)
    ids = P.np_(r["topk_ids"])
    lg = P.np_(r["logits"])
    assert lg[0, 5] == lg[0, 9] == lg[0, 40] and lg[0, 60] == lg[0, 63]
    order = sorted(range(E), key=lambda e: (-lg[0, e], e))[:k]
    assert list(ids[0]) == order and list(ids[1]) == order


def test_router_ties_resolve_to_lowest_id_many_experts(ops):
    """More than 512 experts: four logits per thread in the rank count."""
    H, E, k = 256, 1024, 8
    w = inputs.normal_f32((5,), (E, H), 0.02)
    for dup in ([7, 300, 1000], [511, 512, 1023]):
        w[dup] = w[dup[0]] + 1.0
    x = np.full((3, H), 0x3F80, dtype=np.uint16)
    r = ops.moe_route_topk(P.to_dev_bf16(x), P.to_dev(w), k)
    ids = P.np_(r["topk_ids"])
    lg = P.np_(r["logits"])
    assert lg[0, 7] == lg[0, 300] == lg[0, 1000] and lg[0, 511] == lg[0, 512] == lg[0, 1023]
    order = sorted(range(E), key=lambda e: (-lg[0, e], e))[:k]
    for t in range(3):
        assert list(ids[t]) == order


def test_router_k_equals_e_and_k_one(ops):
    H = 64
    for E, k in ((8, 8), (16, 1), (1024, 8), (513, 8), (520, 3), (1000, 5)):
        w = inputs.normal_f32((6, E), (E, H), 0.05)
        x = inputs.normal_bf16((7, E), (3, H), 1.0)
        r = ops.moe_route_topk(P.to_dev_bf16(x), P.to_dev(w), k)
        P.check_routing(x, w.astype(np.float64), k, P.np_(r["topk_ids"]), P.np_(r["topk_w"]),
                        P.np_(r["expert_list"]), P.np_(r["slot_w"]), P.np_(r["logits"]))


@pytest.mark.parametrize("T", [1, 2, 4])
@pytest.mark.parametrize("with_shared", [False, True])
def test_planted_experts_bit_exact(ops, T, with_shared):
    H, I, E = 2560, 768, 4
    c13, s13, c2, s2 = P.planted_exact_layer(H, I, E + 1, seed=T)
    wr = inputs.normal_f32((8, T), (E, H), 0.02)
    xi = np.random.default_rng(T).integers(1, 3, size=(T, H))
    x = torch.from_numpy(xi.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    xd = P.to_dev_bf16(x)
    r = ops.moe_route_topk(xd, P.to_dev(wr), 1)
    shared = tuple(P.to_dev(a[E]) for a in (c13, s13, c2, s2)) if with_shared else None
    y, _ = ops.moe_expert_gemv_mxfp4(xd, P.to_dev(c13[:E]), P.to_dev(s13[:E]), P.to_dev(c2[:E]), P.to_dev(s2[:E]),
                                     r["expert_list"], r["slot_w"], 1, shared=shared)
    ids = P.np_(r["topk_ids"])[:, 0]
    W = F.dequant_mxfp4(c13, s13, H)                      # exact multiples of 1/8
    want = np.zeros((T, H))
    for t in range(T):
        experts = [ids[t]] + ([E] if with_shared else [])
        for e in experts:
            g = (W[e, :I] * 8).astype(np.int64) @ xi[t] / 8.0
            want[t, :I] += g * xi[t, np.arange(I) % H]
    assert np.array_equal(P.np_(y).astype(np.float64), want)


# ----------------------------------------------------------------------------- Ling shape


@pytest.fixture(scope="module")
def ling(ops):
    wl = configs.MOE_LAYER
    lw = inputs.layer_weights(wl, 0)
    dw = P.layer_to_dev(lw)
    torch.cuda.synchronize()
    return wl, lw, dw


def test_ling_layer_one_token(ops, ling):
    wl, lw, dw = ling
    worst = 0.0
    for step in range(6):
        x = inputs.activations(wl, step)
        res = inputs.normal_bf16((wl.seed, 99, step), (1, wl.moe.H), 1.0)
        r, y, h = run_layer(ops, wl, dw, x, res)
        assert int(r["expert_list"][0]) == 8
        worst = max(worst, check_layer(wl, lw, x, res, r, y, h)[1])
    print(f"worst y error {worst:.2e} x RMS")


def test_ling_verify_pass_random_tokens(ops, ling):
    wl, lw, dw = ling
    vw = configs.VERIFY
    for step in range(3):
        x = inputs.normal_bf16((vw.seed, inputs.T_X, step), (4, wl.moe.H), 1.0)
        res = inputs.normal_bf16((vw.seed, 99, step), (4, wl.moe.H), 1.0)
        r, y, h = run_layer(ops, wl, dw, x, res)
        D = int(r["expert_list"][0])
        assert 24 <= D <= 32, D
        check_layer(wl, lw, x, res, r, y, h)


def test_ling_verify_pass_overlapping_tokens(ops, ling):
    wl, lw, dw = ling
    vw = configs.VERIFY
    x = inputs.overlapping_activations(vw, 0)
    res = inputs.normal_bf16((vw.seed, 98), (4, wl.moe.H), 1.0)
    r, y, h = run_layer(ops, wl, dw, x, res)
    D = int(r["expert_list"][0])
    assert D < 32                       # tokens share experts
    check_layer(wl, lw, x, res, r, y, h)


def test_identical_tokens_give_identical_rows(ops, ling):
    wl, lw, dw = ling
    x = np.repeat(inputs.activations(wl, 7), 4, axis=0)
    res = np.repeat(inputs.normal_bf16((5,), (1, wl.moe.H), 1.0), 4, axis=0)
    r, y, h = run_layer(ops, wl, dw, x, res)
    assert int(r["expert_list"][0]) == 8
    for t in range(1, 4):
        assert np.array_equal(y[t], y[0]) and np.array_equal(h[t], h[0])
        assert np.array_equal(r["topk_ids"][t], r["topk_ids"][0])
    r1, y1, h1 = run_layer(ops, wl, dw, x[:1], res[:1])
    np.testing.assert_array_equal(r1["topk_ids"][0], r["topk_ids"][0])
    assert C.fp_close(y1, y[:1])[0]


@pytest.mark.parametrize("T", [1, 4])
def test_layer_is_deterministic(ops, ling, T):
    wl, lw, dw = ling
    x = inputs.normal_bf16((31, T), (T, wl.moe.H), 1.0)
    res = inputs.normal_bf16((32, T), (T, wl.moe.H), 1.0)
    first = run_layer(ops, wl, dw, x, res)
    for _ in range(10):
        again = run_layer(ops, wl, dw, x, res)
        assert np.array_equal(first[1], again[1]) and np.array_equal(first[2], again[2])
        for key in first[0]:
            assert np.array_equal(first[0][key], again[0][key])
