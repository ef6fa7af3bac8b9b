"""Pins for the sampling oracle (temperature / top-k / top-p with a passed-in
uniform): the hand-worked golden example, argmax limits, scipy's softmax for the
untruncated case, a brute-force smallest-set check of the top-p cut on tiny
vocabularies, the u limits, shift invariance, and frequencies over a u grid."""

import itertools
import json
import os

import numpy as np
import pytest
from scipy.special import softmax

from oracle import sample as Sm

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_page_settings_recorded():
    facts = json.load(open(os.path.join(GOLDEN, "page_facts.json")))
    assert facts["gsm8k_temperature"]["value"] == 0.6
    assert facts["gsm8k_top_p"]["value"] == 0.95
    assert facts["gsm8k_top_k"]["value"] == 29


def test_hand_worked_example():
    d = json.load(open(os.path.join(GOLDEN, "sampling_example.json")))
    z = np.log(np.array(d["logits_ln_args"], dtype=np.float64)).astype(np.float32)
    for c in d["cases"]:
        for draw in c["draws"]:
            tok, ids, p = Sm.sample_row(z, c["temperature"], c["top_k"], c["top_p"], draw["u"])
            assert list(ids) == c["kept_ids"], c["name"]
            assert np.allclose(p, c["probs"], rtol=1e-6, atol=1e-7), (c["name"], p)
            assert tok == draw["token"], (c["name"], draw)


def rand_logits(seed, V, scale=3.0):
    return (np.random.default_rng(seed).standard_normal(V) * scale).astype(np.float32)


@pytest.mark.parametrize("seed", range(5))
def test_top_k_one_and_tiny_top_p_are_greedy(seed):
    z = rand_logits(seed, 1000)
    want = int(np.argmax(z))
    for u in (0.0, 0.3, 0.999):
        assert Sm.sample_row(z, 0.6, 1, 0.95, u)[0] == want
        assert Sm.sample_row(z, 0.6, 29, 1e-6, u)[0] == want


def test_ties_rank_lower_id_first():
    z = np.array([1.0, 5.0, 5.0, 2.0, 5.0], dtype=np.float32)
    ids = Sm.ranked_topk(z, 4)
    assert list(ids) == [1, 2, 4, 3]
    assert Sm.sample_row(z, 1.0, 1, 1.0, 0.9)[0] == 1


@pytest.mark.parametrize("temperature", [0.6, 1.0, 2.5])
def test_untruncated_widths_are_the_softmax(temperature):
    """top_k = V and top_p = 1: the probabilities are softmax(z / temperature)."""
    V = 40
    z = rand_logits(7, V, 1.5)
    _, ids, p = Sm.sample_row(z, temperature, V, 1.0, 0.5)
    ref = softmax(z.astype(np.float64) / temperature)
    assert np.allclose(p, ref[ids], rtol=2e-6, atol=1e-9)
    kept, lo, hi = Sm.cumulative_bounds(z, temperature, V, 1.0)
    assert np.allclose(hi - lo, ref[kept], rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("seed", range(8))
def test_top_p_keeps_the_smallest_heavy_set(seed):
    """Brute force over every subset of a 7-token vocabulary: the kept set is
    the smallest set of mass >= top_p whose members each outweigh every token
    left out."""
    V = 7
    g = np.random.default_rng(100 + seed)
    z = (g.standard_normal(V) * 2).astype(np.float32)
    top_p = float(g.uniform(0.3, 0.99))
    T = 0.8
    prob = softmax(z.astype(np.float64) / T)
    best = None
    for r in range(1, V + 1):
        for sub in itertools.combinations(range(V), r):
            rest = [i for i in range(V) if i not in sub]
            if prob[list(sub)].sum() >= top_p and (not rest or prob[list(sub)].min() > prob[rest].max()):
                best = set(sub)
                break
        if best is not None:
            break
    _, ids, p = Sm.sample_row(z, T, V, top_p, 0.5)
    assert set(ids[p > 0].tolist()) == best


@pytest.mark.parametrize("seed", range(6))
def test_cumulative_bounds_below_top_p_one(seed):
    """cumulative_bounds at top_p < 1, after a top-k cut: the kept ranks are the
    brute-force smallest heavy set of the top k (found by trying every subset
    of the renormalised top-k probabilities), and each interval's width is that
    token's probability renormalised over the kept set, from an fp64 softmax."""
    V, k = 9, 7
    g = np.random.default_rng(300 + seed)
    z = (g.standard_normal(V) * 2).astype(np.float32)
    top_p = float(g.uniform(0.3, 0.95))
    T = 0.7
    top = np.argsort(-z.astype(np.float64), kind="stable")[:k]
    q = softmax(z[top].astype(np.float64) / T)          # the top k, renormalised
    best = None
    for r in range(1, k + 1):
        for sub in itertools.combinations(range(k), r):
            rest = [i for i in range(k) if i not in sub]
            if q[list(sub)].sum() >= top_p and (not rest or q[list(sub)].min() > q[rest].max()):
                best = sorted(sub)
                break
        if best is not None:
            break
    kept, lo, hi = Sm.cumulative_bounds(z, T, k, top_p)
    assert sorted(kept.tolist()) == sorted(top[best].tolist())
    want = q[best] / q[best].sum()
    order = [best[list(top[best]).index(i)] for i in kept]   # the oracle's rank order
    assert np.allclose(hi - lo, q[order] / q[best].sum(), rtol=1e-12, atol=1e-15)
    assert lo[0] == 0.0 and abs(hi[-1] - 1.0) < 1e-12 and np.all(np.diff(hi) > 0)
    assert np.isclose(want.sum(), 1.0)


def test_u_limits_and_shift_invariance():
    z = (np.round(rand_logits(3, 5000) * 1024) / 1024).astype(np.float32)   # 2^-10 grid: z + 16 is exact
    for k, tp in ((29, 0.95), (8, 0.5), (64, 1.0)):
        tok0, ids, p = Sm.sample_row(z, 0.6, k, tp, 0.0)
        assert tok0 == ids[0]
        last = ids[np.nonzero(p)[0][-1]]
        assert Sm.sample_row(z, 0.6, k, tp, np.nextafter(np.float32(1), np.float32(0)))[0] == last
        # adding a constant that is exact in binary32 keeps every difference
        zs = (z + np.float32(16.0)).astype(np.float32)
        assert np.array_equal((zs - np.float32(16.0)).astype(np.float32), z)
        for u in (0.1, 0.45, 0.77):
            assert Sm.sample_row(zs, 0.6, k, tp, u)[0] == Sm.sample_row(z, 0.6, k, tp, u)[0]


def test_frequencies_over_a_u_grid_match_the_probabilities():
    z = rand_logits(11, 300, 1.0)
    T, k, tp = 0.6, 29, 0.95
    _, ids, p = Sm.sample_row(z, T, k, tp, 0.0)
    n = 20000
    us = (np.arange(n) + 0.5) / n
    counts = {}
    for u in us:
        t = Sm.sample_row(z, T, k, tp, u)[0]
        counts[t] = counts.get(t, 0) + 1
    for i, v in enumerate(ids):
        assert abs(counts.get(int(v), 0) / n - p[i]) <= 1.0 / n + 1e-6
