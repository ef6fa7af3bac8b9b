"""Pins for the LM-head oracle: the FP8 quantizer against torch's binary32
division and float8_e4m3fn conversion over every finite bf16 pattern, round-trip
bounds, the page's byte-halving fact, the GEMV against torch, exact cases and
the argmax tie rule."""

import json
import os

import numpy as np
import pytest
import torch

from oracle import head as Hd
from oracle import formats as F


def all_finite_bf16():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = F.bf16_to_f64(b)
    return b[np.isfinite(v)]


def quantizer_rows(K=256):
    """Rows holding every finite bf16 pattern, each row led by a planted absmax
    element so the per-row scale varies over many binades."""
    pats = all_finite_bf16()
    vals = F.bf16_to_f64(pats)
    order = np.argsort(np.abs(vals), kind="stable")
    pats = pats[order]
    rows = []
    for r0 in range(0, len(pats), K):
        row = pats[r0:r0 + K]
        if len(row) < K:
            row = np.concatenate([row, np.zeros(K - len(row), dtype=np.uint16)])
        rows.append(row)
    rows = np.stack(rows)
    # shuffle positions inside each row so the absmax is not always last
    g = np.random.default_rng(0)
    for r in rows:
        g.shuffle(r)
    zero = np.zeros((1, K), dtype=np.uint16)
    negz = np.full((1, K), 0x8000, dtype=np.uint16)
    return np.concatenate([rows, zero, negz])


def torch_quantize(w_bits):
    w = torch.from_numpy(F.bf16_to_f64(w_bits).astype(np.float32))
    amax = w.abs().amax(dim=1)
    s = amax / torch.tensor(448.0, dtype=torch.float32)
    v = torch.where(s[:, None] > 0, w / torch.where(s > 0, s, torch.ones_like(s))[:, None], torch.zeros_like(w))
    v = v.clamp(-448.0, 448.0)
    q = v.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    q[(s == 0).numpy()] = 0
    return q, s.numpy()


def test_quantizer_exhaustive_bf16_matches_torch():
    w = quantizer_rows()
    q, s = Hd.quantize_fp8(w)
    tq, ts = torch_quantize(w)
    assert np.array_equal(s.view(np.uint32), ts.view(np.uint32))
    assert np.array_equal(q, tq)


def test_quantizer_round_trip_bounds_and_saturation_code():
    w = quantizer_rows()
    q, s = Hd.quantize_fp8(w)
    wv = F.bf16_to_f64(w)
    back = F.decode_e4m3fn(q) * s.astype(np.float64)[:, None]
    nz = s > 0
    rel = np.abs(wv[nz]) / s[nz][:, None].astype(np.float64)
    err = np.abs(back[nz] - wv[nz])
    normal = rel >= 2.0 ** -6
    slack = 1 + 2.0 ** -20
    assert np.all(err[normal] <= 2.0 ** -4 * np.abs(wv[nz][normal]) * slack)
    assert np.all(err[~normal] <= 2.0 ** -10 * np.broadcast_to(s[nz][:, None], err.shape)[~normal] * slack)
    mag = np.abs(F.decode_e4m3fn(q[nz]))
    assert np.all(mag.max(axis=1) == 448.0)
    # zero rows: scale 0, all codes 0
    assert np.all(s[~nz] == 0) and np.all(q[~nz] == 0)


def test_fp8_head_halves_the_bytes(golden_dir):
    facts = json.load(open(os.path.join(golden_dir, "page_facts.json")))
    V, K = facts["vocab"]["value"], facts["hidden"]["value"]
    bf16_bytes = V * K * 2
    fp8_bytes = V * K * 1
    assert fp8_bytes / bf16_bytes == facts["fp8_head_bytes_ratio"]["value"]
    w = np.random.default_rng(1).integers(0, 0x3F00, size=(8, 64)).astype(np.uint16)
    q, s = Hd.quantize_fp8(w)
    assert q.nbytes * 2 == w.nbytes and s.dtype == np.float32


def test_head_logits_match_torch_matmul():
    g = np.random.default_rng(2)
    V, K, T = 3000, 256, 3
    w = torch.from_numpy(g.normal(0, 0.02, size=(V, K)).astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    x = torch.from_numpy(g.normal(0, 1, size=(T, K)).astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    q, s = Hd.quantize_fp8(w)
    Wt = torch.from_numpy(q).view(torch.float8_e4m3fn).to(torch.float64)
    xt = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(torch.float64)
    ref = (xt @ Wt.T) * torch.from_numpy(s.astype(np.float64))[None, :]
    np.testing.assert_allclose(Hd.head_logits(q, s, x, chunk=700), ref.numpy(), rtol=1e-12, atol=1e-15)
    refb = xt @ torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).to(torch.float64).T
    np.testing.assert_allclose(Hd.head_logits_bf16(w, x, chunk=999), refb.numpy(), rtol=1e-12, atol=1e-15)


def test_head_exact_small_integers():
    g = np.random.default_rng(3)
    V, K = 50, 64
    q = g.integers(0, 256, size=(V, K)).astype(np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x11             # no NaN codes
    s = (2.0 ** g.integers(-3, 4, size=V)).astype(np.float32)
    xi = g.integers(-3, 4, size=(1, K))
    x = torch.from_numpy(xi.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    # exact: every E4M3 value is m * 2^-9 for an integer m
    m = np.round(F.decode_e4m3fn(q) * 512).astype(np.int64)
    ref = np.array([[int(np.dot(m[v], xi[0])) for v in range(V)]], dtype=np.float64) / 512.0 * s.astype(np.float64)
    assert np.array_equal(Hd.head_logits(q, s, x), ref)


def test_argmax_ties_to_lowest_index():
    l = np.array([[1.0, 5.0, 5.0, 2.0], [7.0, 7.0, 7.0, 7.0], [-1.0, -3.0, -1.0, -2.0]])
    assert list(Hd.greedy_argmax(l)) == [1, 0, 0]
