"""GPU parity of the W4A8 path (MXFP4 weights x MXFP8 activations on the
matrix cores) against oracle/w4a8.py: the activation quantizer bit for bit,
and one MoE layer at the tiny and Ling shapes for 1 and 4 tokens, with the
device's routing.  The gate/up activations are compared at the fp tolerance;
the down stage is checked on the device's own binary32 activations (the
oracle quantizes those same values, so both sides take the same rounding
decisions); h' must equal RNE_bf16(h + y_gpu)."""

import numpy as np
import pytest
import torch

from oracle import compare as C
from oracle import formats as F
from oracle import w4a8 as W
from weight_streaming_expert_amd import configs, inputs
import parity as P

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from weight_streaming_expert_amd import ops as _ops
    return _ops


def edge_rows(K):
    """bf16 rows exercising the quantizer's edges, one block of 32 per case."""
    g = np.random.default_rng(7)
    rows = []
    base = g.standard_normal((12, K))
    base[0, :32] = 0.0                                     # all-zero block
    base[1, :32] = -0.0                                    # negative zeros
    base[2, :32] *= 1e-3
    base[2, 5] = 1.875 * 2.0 ** 3                          # saturating top (480 -> 448)
    base[3, :32] = g.standard_normal(32) * 2.0 ** 100      # large exponents
    base[4, :32] = g.standard_normal(32) * 2.0 ** -120     # tiny block maximum
    base[5, :32] = g.standard_normal(32) * 2.0 ** -128     # bf16 subnormals
    base[6, :32] = g.standard_normal(32)
    base[6, 0] = 2.0 ** 20                                 # small members underflow to subnormal codes / zero
    base[7, :32] = np.where(g.random(32) < 0.5, 1.75, -1.75) * 2.0 ** 4
    for r in base:
        rows.append(r)
    return F.f64_to_bf16_rne(np.stack(rows))


@pytest.mark.parametrize("T,K", [(1, 2560), (4, 256), (16, 64), (3, 2560)])
def test_act_quantize_bit_exact(ops, T, K):
    x = inputs.normal_bf16((61, T, K), (T, K), 1.0)
    for xb in (x, edge_rows(K)):
        codes, scales = ops.act_quantize_mxfp8(P.to_dev_bf16(xb))
        q, s = W.quantize_bf16_rows(xb)
        assert np.array_equal(P.np_(scales), s)
        assert np.array_equal(P.np_(codes), q)


def run_w4a8(ops, wl, dw, x_bits, res_bits):
    x = P.to_dev_bf16(x_bits)
    r = ops.moe_route_topk(x, dw["router"], wl.moe.k)
    y, h, act = ops.moe_expert_gemv_w4a8(x, dw["w13c"], dw["w13s"], dw["w2c"], dw["w2s"], r["expert_list"],
                                         r["slot_w"], wl.moe.k, shared=dw["shared"],
                                         residual=P.to_dev_bf16(res_bits), want_act=True)
    return {k: P.np_(v) for k, v in r.items()}, P.np_(y), P.bits(h), P.np_(act)


def check_w4a8(wl, lw, x_bits, res_bits, r, y, h, act):
    m = wl.moe
    T = x_bits.shape[0]
    n = int(r["expert_list"][0])
    el = r["expert_list"][1:1 + n]
    sw = r["slot_w"].reshape(T * m.k, T)[:n]
    get = lambda e: (lw["w13c"][e], lw["w13s"][e], lw["w2c"][e], lw["w2s"][e])
    worst_a = 0.0
    for s in range(n + 1):
        c13, s13 = (get(int(el[s]))[:2] if s < n else lw["shared"][:2])
        a_ref = W.gate_up_w4a8(x_bits, c13, s13, m.I)
        ok, wa = C.fp_close(act[s], a_ref)
        assert ok, f"slot {s}: a off by {wa:.3e} x RMS"
        worst_a = max(worst_a, wa)
    y_ref = W.moe_y_w4a8(x_bits, el, sw, get, lw["shared"], m.I, acts=act[:n + 1])
    ok, wy = C.fp_close(y, y_ref)
    assert ok, f"y off by {wy:.3e} x RMS"
    P.check_residual(res_bits, y, h)
    return worst_a, wy


@pytest.fixture(scope="module")
def tiny(ops):
    wl = configs.TINY
    lw = inputs.layer_weights(wl, 0)
    return wl, lw, P.layer_to_dev(lw)


@pytest.mark.parametrize("T", [1, 2, 4])
def test_w4a8_tiny_layer(ops, tiny, T):
    wl, lw, dw = tiny
    for step in range(3):
        x = inputs.normal_bf16((wl.seed, 71, step, T), (T, wl.moe.H), 1.0)
        res = inputs.normal_bf16((wl.seed, 72, step, T), (T, wl.moe.H), 1.0)
        check_w4a8(wl, lw, x, res, *run_w4a8(ops, wl, dw, x, res))


@pytest.fixture(scope="module")
def ling(ops):
    wl = configs.MOE_LAYER
    lw = inputs.layer_weights(wl, 0)
    return wl, lw, P.layer_to_dev(lw)


@pytest.mark.parametrize("T", [1, 4])
def test_w4a8_ling_layer(ops, ling, T):
    wl, lw, dw = ling
    for step in range(2):
        x = inputs.normal_bf16((wl.seed, 73, step, T), (T, wl.moe.H), 1.0)
        res = inputs.normal_bf16((wl.seed, 74, step, T), (T, wl.moe.H), 1.0)
        check_w4a8(wl, lw, x, res, *run_w4a8(ops, wl, dw, x, res))


def test_w4a8_planted_experts_bit_exact(ops):
    """Planted experts (tests/parity.py): positive gate codes so that g >= H/2
    and silu(g) == g, up row i one-hot on input i with scale 1, down the
    identity on the first I outputs.  With inputs in {1, 2} (held exactly by
    MXFP8) every gate/up sum is exact, so the device's a equals the oracle's
    bit for bit; with power-of-two slot weights the down stage and combine are
    exact too, and y equals the oracle's y bit for bit."""
    wl = configs.TINY
    m = wl.moe
    T = 2
    c13, s13, c2, s2 = P.planted_exact_layer(m.H, m.I, m.E, seed=5)
    g = np.random.default_rng(4)
    xb = F.f64_to_bf16_rne(g.integers(1, 3, (T, m.H)).astype(np.float64))
    el = np.zeros(1 + T * m.k, dtype=np.int32)
    el[0], el[1], el[2] = 2, 4, 9
    sw = np.zeros((T * m.k, T), dtype=np.float32)
    sw[0] = [1.0, 0.5]
    sw[1] = [0.0, 0.5]
    y, _, act = ops.moe_expert_gemv_w4a8(P.to_dev_bf16(xb), P.to_dev(c13), P.to_dev(s13), P.to_dev(c2), P.to_dev(s2),
                                         P.to_dev(el), P.to_dev(sw), m.k, shared=None, want_act=True)
    act, y = P.np_(act), P.np_(y)
    for s, e in enumerate((4, 9)):
        assert np.array_equal(act[s].astype(np.float64), W.gate_up_w4a8(xb, c13[e], s13[e], m.I))
    get = lambda e: (c13[e], s13[e], c2[e], s2[e])
    y_ref = W.moe_y_w4a8(xb, np.array([4, 9]), sw[:2].astype(np.float64), get, None, m.I)
    assert np.array_equal(y.astype(np.float64), y_ref)
