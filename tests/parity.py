"""Helpers shared by the GPU parity tests: device transfer, oracle-side stage
checks that consume the GPU's own inputs to each stage, and the planted exact
cases."""

import numpy as np
import torch

from oracle import compare as C
from oracle import formats as F
from oracle import head as OH
from oracle import moe as OM

DEV = "cuda"


def to_dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def bits(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def np_(t):
    return t.detach().cpu().numpy()


def router_values(w):
    """Router weights as exact float64 values (fp32 array or bf16 bits)."""
    return w.astype(np.float64) if w.dtype == np.float32 else F.bf16_to_f64(w)


def layer_to_dev(lw):
    d = {k: to_dev(lw[k]) for k in ("w13c", "w13s", "w2c", "w2s")}
    r = lw["router"]
    d["router"] = to_dev(r) if r.dtype == np.float32 else to_dev_bf16(r)
    d["shared"] = None if lw["shared"] is None else tuple(to_dev(a) for a in lw["shared"])
    return d


def check_routing(x_bits, wr_values, k, ids_gpu, w_gpu, el_gpu=None, sw_gpu=None, logits_gpu=None):
    """Top-k ids, weights and compact list of the GPU against the oracle on the
    same input.  Returns the number of tokens with a near tie."""
    ref_logits = OM.router_logits(x_bits, wr_values)
    T = ref_logits.shape[0]
    if logits_gpu is not None:
        ok, worst = C.fp_close(logits_gpu, ref_logits)
        assert ok, f"router logits off by {worst:.3e} x RMS"
    ok, ties = C.check_topk(ids_gpu, ref_logits, k)
    assert ok, f"top-k mismatch: gpu {ids_gpu} ref {[OM.topk_order(l, k) for l in ref_logits]}"
    for t in range(T):
        sel = ref_logits[t][ids_gpu[t]]
        w_ref = np.exp(sel - sel.max())
        w_ref /= w_ref.sum()
        assert np.max(np.abs(w_gpu[t] - w_ref)) <= C.FP_REL_TOL * C.rms(w_ref)
        assert abs(float(np.sum(w_gpu[t])) - 1.0) <= 1e-6
    if el_gpu is not None:
        el_ref, sw_ref = OM.expert_list(ids_gpu, w_gpu)
        n = int(el_gpu[0])
        assert n == len(el_ref) and np.array_equal(el_gpu[1:1 + n], el_ref)
        assert n <= T * k
        sw = sw_gpu.reshape(T * k, T)
        assert np.array_equal(sw[:n], sw_ref.astype(np.float32))
        assert np.all(sw[n:] == 0)
    return ties


def moe_y_ref(x_bits, ids_gpu, w_gpu, get_expert, shared, I):
    """y of the oracle for the GPU's routing decisions."""
    el, sw = OM.expert_list(ids_gpu, w_gpu)
    d = [OM.down(OM.gate_up(x_bits, *get_expert(int(e))[:2], I), *get_expert(int(e))[2:]) for e in el]
    d_sh = None
    if shared is not None:
        d_sh = OM.down(OM.gate_up(x_bits, shared[0], shared[1], I), shared[2], shared[3])
    return OM.combine(np.stack(d), sw, d_sh)


def check_residual(h_bits, y_gpu, h_gpu_bits):
    """h' must be RNE_bf16(fp32(h + y_gpu)) exactly."""
    s = (F.bf16_to_f64(h_bits).astype(np.float32) + y_gpu.astype(np.float32)).astype(np.float32)
    ref = torch.from_numpy(s).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ref, h_gpu_bits)


def check_h_next(h_bits, y_ref, h_next_bits):
    """Without y from the GPU: h_{l+1} within the fp tolerance of y plus half a
    bf16 ulp of the rounded sum."""
    exact = F.bf16_to_f64(h_bits) + y_ref
    got = F.bf16_to_f64(h_next_bits)
    _, e = np.frexp(exact)
    half_ulp = np.ldexp(1.0, np.maximum(e, -125) - 9)
    tol = C.FP_REL_TOL * C.rms(y_ref)[:, None] + half_ulp
    assert np.all(np.abs(got - exact) <= tol), float(np.max(np.abs(got - exact) - tol))


def check_norm(h_bits, u_gpu_bits):
    """u = RNE_bf16(h / rms(h)): within one bf16 rounding of the exact value."""
    ref = OM.rmsnorm_f64(h_bits)
    got = F.bf16_to_f64(u_gpu_bits)
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) * (1 + 1e-5) + 1e-30)


def check_head(q, s, x_bits, logits_gpu, argmax_gpu, bf16_w=None):
    ref = OH.head_logits_bf16(bf16_w, x_bits) if bf16_w is not None else OH.head_logits(q, s, x_bits)
    if logits_gpu is not None:
        ok, worst = C.fp_close(logits_gpu, ref)
        assert ok, f"head logits off by {worst:.3e} x RMS"
    ok, ties = C.check_argmax(argmax_gpu, ref)
    assert ok, f"argmax gpu {argmax_gpu} ref {np.argmax(ref, axis=-1)}"
    return ties


# ----------------------------------------------------------------------------- planted exact experts


def planted_exact_layer(H, I, E, seed=0):
    """An expert whose gate rows have positive E2M1 codes (so g >= H/2 and
    silu(g) == g exactly in fp32), whose up row i is the one-hot e_{i mod H}
    with scale 1 (so u = x[i mod H]), and whose down matrix is the identity on
    the first I outputs.  With x in {1, 2} every partial sum is a multiple of
    1/8 below 2^24, so y[n] = g[n] * x[n] exactly for n < I and 0 otherwise."""
    g = np.random.default_rng(seed)
    c13 = np.zeros((E, 2 * I, H // 2), dtype=np.uint8)
    s13 = np.full((E, 2 * I, H // 32), 127, dtype=np.uint8)
    c2 = np.zeros((E, H, I // 2), dtype=np.uint8)
    s2 = np.full((E, H, I // 32), 127, dtype=np.uint8)
    for e in range(E):
        lo = g.integers(1, 8, size=(I, H // 2))
        hi = g.integers(1, 8, size=(I, H // 2))
        c13[e, :I] = (lo | (hi << 4)).astype(np.uint8)
        s13[e, :I] = (127 + g.integers(-2, 3, size=(I, H // 32))).astype(np.uint8)
        for i in range(I):
            j = i % H
            c13[e, I + i, j // 2] = 2 << (4 * (j % 2))        # E2M1 code 2 = 1.0
            c2[e, i, i // 2] = 2 << (4 * (i % 2))             # identity on the first I rows
    return c13, s13, c2, s2
