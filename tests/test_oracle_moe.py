"""Pins for the MoE oracle: brute force, exact rational arithmetic, library
routines (scipy, torch) and invariants the method must satisfy."""

import itertools
import math
from fractions import Fraction
import json
import os

import numpy as np
import pytest
import scipy.special
import torch

from oracle import moe as M
from oracle import formats as F

E2M1 = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4), Fraction(6)]


def bf16_bits(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


# ----------------------------------------------------------------------------- top-k


def test_topk_all_orderings_of_8_distinct_logits():
    base = np.array([-3.0, -1.5, -0.25, 0.0, 0.5, 1.0, 2.5, 7.0])
    for perm in itertools.permutations(range(8)):
        l = base[list(perm)]
        for k in (1, 3, 8):
            got = M.topk_order(l, k)
            # brute force: the id holding the r-th largest value, r = 0..k-1
            want = [perm.index(7 - r) for r in range(k)]
            assert list(got) == want


def test_topk_brute_force_subsets_small_e():
    g = np.random.default_rng(3)
    for trial in range(300):
        E = int(g.integers(2, 9))
        k = int(g.integers(1, E + 1))
        l = g.integers(-3, 4, size=E).astype(np.float64)      # many exact ties
        got = M.topk_order(l, k)
        # brute force over all ordered k-tuples: keep those sorted by (value desc, id asc)
        best = None
        for tup in itertools.permutations(range(E), k):
            keys = [(-l[e], e) for e in tup]
            if keys != sorted(keys):
                continue
            rest = [e for e in range(E) if e not in tup]
            if rest and keys[-1] > min((-l[e], e) for e in rest):
                continue
            best = tup
            break
        assert tuple(got) == best, (l, k, got, best)


def test_topk_ties_resolve_to_lowest_id():
    assert list(M.topk_order([1.0, 3.0, 3.0, 2.0, 3.0], 2)) == [1, 2]
    assert list(M.topk_order([5.0, 5.0, 5.0, 5.0], 3)) == [0, 1, 2]


# ----------------------------------------------------------------------------- softmax


def test_softmax_selected_matches_scipy_and_invariants():
    g = np.random.default_rng(4)
    for _ in range(200):
        l = g.normal(0, 3, size=8)
        w = M.softmax_selected(l)
        assert np.allclose(w, scipy.special.softmax(l), rtol=1e-14, atol=0)
        assert abs(w.sum() - 1.0) < 1e-14
        order = np.argsort(-l)
        assert np.all(np.diff(w[order]) <= 1e-18)
    assert M.softmax_selected([2.5])[0] == 1.0
    assert np.all(M.softmax_selected([0.7] * 8) == 1.0 / 8)


# ----------------------------------------------------------------------------- silu / swiglu


def test_silu_matches_expit_and_limits():
    g = np.concatenate([np.linspace(-1e4, 1e4, 200001), np.random.default_rng(0).normal(0, 5, 10000)])
    ref = g * scipy.special.expit(g)
    ours = M.silu(g)
    assert not np.any(np.isnan(ours))
    np.testing.assert_allclose(ours, ref, rtol=1e-13, atol=1e-300)
    assert M.silu(np.array([0.0]))[0] == 0.0
    assert M.silu(np.array([-1e4]))[0] == 0.0


# ----------------------------------------------------------------------------- exact contraction


def _fraction_dequant(codes, scales, N, K):
    """Exact rational MXFP4 decode written directly from the bit layout."""
    W = [[None] * K for _ in range(N)]
    for n in range(N):
        for kk in range(K):
            byte = int(codes[n][kk // 2])
            c = (byte >> 4) if kk % 2 else (byte & 0xF)
            mag = E2M1[c & 7]
            v = -mag if c & 8 else mag
            W[n][kk] = v * Fraction(2) ** (int(scales[n][kk // 32]) - 127)
    return W


def test_gate_up_down_against_exact_rationals():
    g = np.random.default_rng(7)
    H, I, T = 64, 32, 2
    c13 = g.integers(0, 256, size=(2 * I, H // 2), dtype=np.uint8)
    s13 = (127 + g.integers(-4, 3, size=(2 * I, H // 32))).astype(np.uint8)
    c2 = g.integers(0, 256, size=(H, I // 2), dtype=np.uint8)
    s2 = (127 + g.integers(-4, 3, size=(H, I // 32))).astype(np.uint8)
    xb = bf16_bits(g.normal(0, 1, size=(T, H)))
    x = [[Fraction(float(v)) for v in row] for row in F.bf16_to_f64(xb)]
    W13 = _fraction_dequant(c13, s13, 2 * I, H)
    W2 = _fraction_dequant(c2, s2, H, I)
    a = M.gate_up(xb, c13, s13, I)
    for t in range(T):
        for i in range(I):
            gi = sum(W13[i][h] * x[t][h] for h in range(H))
            ui = sum(W13[I + i][h] * x[t][h] for h in range(H))
            ref = float(gi) / (1.0 + math.exp(-float(gi))) * float(ui)
            assert abs(a[t, i] - ref) <= 1e-12 * max(1.0, abs(ref))
    d = M.down(a, c2, s2)
    for t in range(T):
        for n in range(H):
            ref = sum(W2[n][i] * Fraction(float(a[t, i])) for i in range(I))
            assert abs(d[t, n] - float(ref)) <= 1e-12 * max(1.0, abs(float(ref)))


def test_one_hot_input_returns_planted_column():
    g = np.random.default_rng(8)
    H, I = 64, 32
    c13 = g.integers(0, 256, size=(2 * I, H // 2), dtype=np.uint8)
    s13 = np.full((2 * I, H // 32), 127, dtype=np.uint8)
    Wq = _fraction_dequant(c13, s13, 2 * I, H)
    for j in (0, 1, 31, 32, 63):
        x = np.zeros((1, H), dtype=np.float32)
        x[0, j] = 1.0
        a = M.gate_up(bf16_bits(x), c13, s13, I)
        for i in range(I):
            gi, ui = float(Wq[i][j]), float(Wq[I + i][j])
            assert a[0, i] == gi / (1.0 + math.exp(-gi)) * ui


# ----------------------------------------------------------------------------- whole layer


def _rand_expert(g, H, I):
    return (g.integers(0, 256, size=(2 * I, H // 2), dtype=np.uint8),
            (127 + g.integers(-4, 3, size=(2 * I, H // 32))).astype(np.uint8),
            g.integers(0, 256, size=(H, I // 2), dtype=np.uint8),
            (127 + g.integers(-4, 3, size=(H, I // 32))).astype(np.uint8))


def test_identical_experts_give_expert_plus_shared_whatever_the_weights():
    g = np.random.default_rng(9)
    H, I, E, k, T = 64, 32, 8, 3, 2
    ex = _rand_expert(g, H, I)
    sh = _rand_expert(g, H, I)
    wr = g.normal(0, 0.5, size=(E, H))
    xb = bf16_bits(g.normal(0, 1, size=(T, H)))
    out = M.moe_layer(xb, wr, k, lambda e: ex, sh, I=I)
    d_e = M.down(M.gate_up(xb, ex[0], ex[1], I), ex[2], ex[3])
    d_s = M.down(M.gate_up(xb, sh[0], sh[1], I), sh[2], sh[3])
    np.testing.assert_allclose(out["y"], d_e + d_s, rtol=1e-12, atol=1e-9)
    # no shared expert: the routed sum alone
    out2 = M.moe_layer(xb, wr, k, lambda e: ex, None, I=I)
    np.testing.assert_allclose(out2["y"], d_e, rtol=1e-12, atol=1e-9)


def _loop_layer(xrow, wr, k, experts, shared, I):
    """A second, loop-based formulation of one token's MoE layer (plain Python floats)."""
    H = len(xrow)
    E = len(wr)
    logits = [sum(float(wr[e][h]) * xrow[h] for h in range(H)) for e in range(E)]
    order = sorted(range(E), key=lambda e: (-logits[e], e))[:k]
    mx = max(logits[e] for e in order)
    z = [math.exp(logits[e] - mx) for e in order]
    w = [v / sum(z) for v in z]

    def ffn(ex):
        W13 = [[float(v) for v in row] for row in _fraction_dequant(ex[0], ex[1], 2 * I, H)]
        W2 = [[float(v) for v in row] for row in _fraction_dequant(ex[2], ex[3], H, I)]
        a = []
        for i in range(I):
            gi = sum(W13[i][h] * xrow[h] for h in range(H))
            ui = sum(W13[I + i][h] * xrow[h] for h in range(H))
            a.append(gi / (1.0 + math.exp(-gi)) * ui)
        return [sum(W2[n][i] * a[i] for i in range(I)) for n in range(H)]

    y = [0.0] * H
    for wi, e in zip(w, order):
        d = ffn(experts(e))
        y = [y[n] + wi * d[n] for n in range(H)]
    if shared is not None:
        d = ffn(shared)
        y = [y[n] + d[n] for n in range(H)]
    return order, w, y


def test_layer_matches_loop_formulation():
    g = np.random.default_rng(10)
    H, I, E, k = 64, 32, 6, 2
    exps = [_rand_expert(g, H, I) for _ in range(E)]
    sh = _rand_expert(g, H, I)
    wr = g.normal(0, 0.3, size=(E, H)).astype(np.float32)
    xb = bf16_bits(g.normal(0, 1, size=(1, H)))
    out = M.moe_layer(xb, wr, k, lambda e: exps[e], sh, I=I)
    order, w, y = _loop_layer(list(F.bf16_to_f64(xb)[0]), wr, k, lambda e: exps[e], sh, I)
    assert list(out["topk_ids"][0]) == order
    np.testing.assert_allclose(out["topk_w"][0], w, rtol=1e-13)
    np.testing.assert_allclose(out["y"][0], y, rtol=1e-10, atol=1e-9 * np.sqrt(np.mean(np.square(y))))


def test_verify_pass_equals_independent_tokens():
    g = np.random.default_rng(12)
    H, I, E, k, T = 64, 32, 16, 4, 4
    exps = [_rand_expert(g, H, I) for _ in range(E)]
    sh = _rand_expert(g, H, I)
    wr = g.normal(0, 0.3, size=(E, H))
    xb = bf16_bits(g.normal(0, 1, size=(T, H)))
    hb = bf16_bits(g.normal(0, 1, size=(T, H)))
    out = M.moe_layer(xb, wr, k, lambda e: exps[e], sh, residual_bits=hb, I=I)
    assert len(out["expert_list"]) <= T * k
    for t in range(T):
        o1 = M.moe_layer(xb[t:t + 1], wr, k, lambda e: exps[e], sh, residual_bits=hb[t:t + 1], I=I)
        assert np.array_equal(o1["topk_ids"][0], out["topk_ids"][t])
        np.testing.assert_allclose(o1["y"][0], out["y"][t], rtol=1e-12, atol=1e-12)


def test_expert_list_invariants():
    g = np.random.default_rng(13)
    for _ in range(100):
        T, k, E = int(g.integers(1, 5)), int(g.integers(1, 9)), 64
        ids = np.stack([g.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
        w = g.dirichlet(np.ones(k), size=T)
        el, sw = M.expert_list(ids, w)
        assert np.all(np.diff(el) > 0) and len(el) <= T * k
        assert set(el.tolist()) == set(ids.ravel().tolist())
        np.testing.assert_allclose(sw.sum(axis=0), w.sum(axis=1), rtol=1e-14)
        for t in range(T):
            for j in range(k):
                assert sw[list(el).index(ids[t, j]), t] == w[t, j]
            assert np.count_nonzero(sw[:, t]) <= k


def test_verify_union_bound_from_pages(golden_dir):
    facts = json.load(open(os.path.join(golden_dir, "page_facts.json")))
    T = facts["verify_positions"]["value"]
    k = facts["experts_per_token"]["value"]
    E = facts["routed_experts"]["value"]
    g = np.random.default_rng(14)
    worst = 0
    for _ in range(200):
        logits = g.normal(size=(T, E))
        ids, w = M.route(logits, k)
        el, _ = M.expert_list(ids, w)
        worst = max(worst, len(el))
    assert worst <= facts["verify_max_routed_experts"]["value"]
    # disjoint picks reach the bound exactly
    logits = np.full((T, E), -1.0)
    for t in range(T):
        logits[t, t * k:(t + 1) * k] = 1.0
    ids, w = M.route(logits, k)
    assert len(M.expert_list(ids, w)[0]) == facts["verify_max_routed_experts"]["value"]


# ----------------------------------------------------------------------------- norm / residual


def test_rmsnorm_matches_torch():
    g = np.random.default_rng(15)
    hb = bf16_bits(g.normal(0, 30, size=(4, 2560)))
    h = torch.from_numpy(F.bf16_to_f64(hb))
    ref = torch.nn.functional.rms_norm(h, (2560,), eps=1e-6).numpy()
    np.testing.assert_allclose(M.rmsnorm_f64(hb), ref, rtol=1e-14)
    u = F.bf16_to_f64(M.rmsnorm_bf16(hb))
    assert np.max(np.abs(u - ref) / np.abs(ref).clip(1e-30)) <= 2.0 ** -8


def test_residual_rounds_exact_sum():
    h = bf16_bits(np.array([[1.0, 1.0, 3.0]]))
    y = np.array([[2.0 ** -8, 2.0 ** -8 + 2.0 ** -30, -1.0]])
    out = F.bf16_to_f64(M.residual_bf16(h, y))
    assert list(out[0]) == [1.0, 1.0 + 2.0 ** -7, 2.0]
