"""GPU parity of the sampling epilogue (temperature / top-k / top-p with a
caller-supplied uniform): the hand-worked example, ranked top-k ids bit-exact
against the oracle on the same binary32 logits over ragged vocabularies, ties,
an all-equal vocabulary (the k * k survivor bound), the GSM8K settings on the
full 157,184-row head, and the fused head + sampler entry point."""

import json
import os

import numpy as np
import pytest
import torch

from oracle import compare as C
from oracle import formats as F
from oracle import head as OH
from oracle import sample as OS
from weight_streaming_expert_amd import configs, inputs
import parity as P

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
EDGE = 1e-5   # a uniform this close to an interval edge may fall either side (binary32 exp)


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from weight_streaming_expert_amd import ops as _ops
    return _ops


def check_row(z, temp, k, p, u, tok, ids, probs):
    """z: the binary32 logits both sides sampled from."""
    rt, rids, rprobs = OS.sample_row(z, temp, k, p, u)
    assert np.array_equal(ids, rids)
    assert np.allclose(probs, rprobs, rtol=1e-5, atol=1e-7)
    if tok != rt:
        kept, lo, hi = OS.cumulative_bounds(z, temp, k, p)
        j = list(kept).index(tok) if tok in kept else list(rids).index(tok)
        near = j < len(kept) and lo[j] - EDGE <= u <= hi[j] + EDGE
        assert near, (tok, rt, u)


def run_sampler(ops, z, temp, k, p, u):
    tok, ids, probs = ops.lm_sample_topk_topp(P.to_dev(z), temp, k, p, P.to_dev(u))
    return P.np_(tok), P.np_(ids), P.np_(probs)


def test_hand_worked_example(ops):
    d = json.load(open(os.path.join(GOLDEN, "sampling_example.json")))
    z = np.log(np.array(d["logits_ln_args"], dtype=np.float64)).astype(np.float32)
    for c in d["cases"]:
        for draw in c["draws"]:
            tok, ids, probs = run_sampler(ops, z[None, :], c["temperature"], c["top_k"], c["top_p"],
                                          np.array([draw["u"]], dtype=np.float32))
            assert list(ids[0]) == c["kept_ids"]
            assert np.allclose(probs[0], c["probs"], rtol=1e-6, atol=1e-7)
            assert tok[0] == draw["token"], (c["name"], draw)


RAGGED = [(V, k) for V in (1, 5, 64, 65, 255, 256, 257, 1000, 7937, 65536 + 3) for k in (1, 29, 64) if k <= V]


@pytest.mark.parametrize("V,k", RAGGED)
def test_random_logits_ragged(ops, V, k):
    for T, temp, p in ((1, 0.6, 0.95), (3, 1.0, 1.0), (4, 0.3, 0.5)):
        z = inputs.normal_f32((21, V, k, T), (T, V), 3.0)
        u = inputs.uniform_f32((22, V, k, T), (T,))
        tok, ids, probs = run_sampler(ops, z, temp, k, p, u)
        for t in range(T):
            check_row(z[t], temp, k, p, float(u[t]), int(tok[t]), ids[t], probs[t])


def test_ties_and_all_equal(ops):
    V, k = 157184, 64
    z = np.zeros((2, V), dtype=np.float32)                  # every logit equal: ids 0..63 in order
    z[1, [70000, 5, 150000, 99]] = 2.0                       # four tied leaders, then the rest tied
    u = np.array([0.5, 0.99], dtype=np.float32)
    tok, ids, probs = run_sampler(ops, z, 1.0, k, 1.0, u)
    assert list(ids[0]) == list(range(64))
    assert list(ids[1][:4]) == [5, 99, 70000, 150000]
    assert list(ids[1][4:]) == [i for i in range(70) if i not in (5, 99)][:60]
    for t in range(2):
        check_row(z[t], 1.0, k, 1.0, float(u[t]), int(tok[t]), ids[t], probs[t])
    assert tok[0] == 32                                      # u = 0.5 of 64 equal weights


def test_quantized_logits_grid(ops):
    """Logits on a coarse grid (many exact ties across chunks)."""
    V = 20000
    z = np.round(inputs.normal_f32((23,), (4, V), 2.0) * 4) / 4
    z = z.astype(np.float32)
    u = inputs.uniform_f32((24,), (4,))
    tok, ids, probs = run_sampler(ops, z, 0.6, 29, 0.95, u)
    for t in range(4):
        check_row(z[t], 0.6, 29, 0.95, float(u[t]), int(tok[t]), ids[t], probs[t])


@pytest.fixture(scope="module")
def full_head(ops):
    wl = configs.LM_HEAD
    w = inputs.head_weights(wl)
    q, s = ops.lm_head_quantize_fp8(P.to_dev_bf16(w))
    torch.cuda.synchronize()
    return dict(q=q, s=s, qh=P.np_(q), sh=P.np_(s))


@pytest.mark.parametrize("T", [1, 4])
def test_fused_head_and_sampler_full_head(ops, full_head, T):
    """GSM8K settings on the full head.  The sampler's ids and token are
    checked on the GPU's own logits (whose parity with the head oracle is
    checked beside), and the top-k set against the oracle's fp64 logits up to
    near-ties."""
    x = inputs.normal_bf16((25, T), (T, 2560), 1.0)
    u = inputs.uniform_f32((26, T), (T,))
    logits, tok, ids, probs = ops.lm_head_gemv_fp8_sample(full_head["q"], full_head["s"], P.to_dev_bf16(x),
                                                          0.6, 29, 0.95, P.to_dev(u))
    lg = P.np_(logits)
    ref = OH.head_logits(full_head["qh"], full_head["sh"], x)
    ok, worst = C.fp_close(lg, ref)
    assert ok, worst
    for t in range(T):
        check_row(lg[t], 0.6, 29, 0.95, float(u[t]), int(P.np_(tok)[t]), P.np_(ids)[t], P.np_(probs)[t])
        want = OS.ranked_topk(ref[t].astype(np.float32), 29)
        got = P.np_(ids)[t]
        if not np.array_equal(got, want):
            # only near-ties may reorder: every id the two lists disagree on is within rounding of the cut
            kth = np.sort(ref[t])[::-1][28]
            for v in set(got) ^ set(want):
                assert abs(ref[t][v] - kth) <= 1e-5 * max(1.0, abs(kth)), v


def test_fused_exact_integer_head(ops):
    """Integer-valued FP8 head (exact binary32 logits): the fused call's ids,
    probabilities and token equal the oracle's from the exact logits."""
    g = np.random.default_rng(4)
    V, K, T = 3001, 2560, 4
    q = g.integers(0, 256, size=(V, K)).astype(np.uint8)
    big = ((q >> 3) & 0xF) > 7
    q[big] = (q[big] & 0x87) | 0x38
    s = (2.0 ** g.integers(-3, 4, size=V)).astype(np.float32)
    xi = g.integers(-3, 4, size=(T, K))
    x = torch.from_numpy(xi.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ref = OH.head_logits(q, s, x).astype(np.float32)
    u = inputs.uniform_f32((28,), (T,))
    logits, tok, ids, probs = ops.lm_head_gemv_fp8_sample(P.to_dev(q), P.to_dev(s), P.to_dev_bf16(x), 2.0, 64, 0.9,
                                                          P.to_dev(u))
    assert np.array_equal(P.np_(logits), ref)
    for t in range(T):
        check_row(ref[t], 2.0, 64, 0.9, float(u[t]), int(P.np_(tok)[t]), P.np_(ids)[t], P.np_(probs)[t])


@pytest.mark.parametrize("V,K,T", [(4099, 256, 1), (4099, 256, 3), (1000, 2560, 2), (65, 2560, 1)])
def test_fused_ragged_heads(ops, V, K, T):
    """The fused entry on other head instances (K = 256, the 2-4 row paths):
    its logits against the head oracle, its ids, probabilities and token
    against the sampling oracle on those logits."""
    w = inputs.normal_bf16((31, V, K), (V, K), 0.02)
    q, s = ops.lm_head_quantize_fp8(P.to_dev_bf16(w))
    x = inputs.normal_bf16((32, V, K, T), (T, K), 1.0)
    u = inputs.uniform_f32((33, V, K, T), (T,))
    k = min(64, V)
    logits, tok, ids, probs = ops.lm_head_gemv_fp8_sample(q, s, P.to_dev_bf16(x), 1.3, k, 0.5, P.to_dev(u))
    lg = P.np_(logits)
    ok, worst = C.fp_close(lg, OH.head_logits(P.np_(q), P.np_(s), x))
    assert ok, worst
    for t in range(T):
        check_row(lg[t], 1.3, k, 0.5, float(u[t]), int(P.np_(tok)[t]), P.np_(ids)[t], P.np_(probs)[t])


def test_sampler_is_deterministic(ops):
    z = inputs.normal_f32((29,), (4, 157184), 3.0)
    u = inputs.uniform_f32((30,), (4,))
    a = run_sampler(ops, z, 0.6, 29, 0.95, u)
    for _ in range(3):
        b = run_sampler(ops, z, 0.6, 29, 0.95, u)
        for x, y in zip(a, b):
            assert np.array_equal(x, y)


# ---------------------------------------------------------------- the one-launch form (T = 1)

def test_one_launch_path_is_taken(ops):
    assert ops.lm_head_sample_path(1, 157184, 2560, 29) == 1
    assert ops.lm_head_sample_path(1, 157184, 2560, 64) == 1
    assert ops.lm_head_sample_path(1, 4099, 256, 64) == 1
    assert ops.lm_head_sample_path(4, 157184, 2560, 29) == 0      # several rows: head, then the sampler
    assert ops.lm_head_sample_path(1, 65, 2560, 64) == 0          # fewer workgroups with rows than top_k
    assert ops.lm_head_sample_path(1, 157184, 2560, 65) == -1


def fused_vs_two_launch(ops, q, s, x_bits, temp, k, p, u):
    """The one-launch call and the two-launch sampler on the logits it wrote:
    token, ids and probabilities must be identical."""
    logits, tok, ids, probs = ops.lm_head_gemv_fp8_sample(q, s, P.to_dev_bf16(x_bits), temp, k, p, P.to_dev(u))
    t2, i2, p2 = ops.lm_sample_topk_topp(logits, temp, k, p, P.to_dev(u))
    assert np.array_equal(P.np_(ids), P.np_(i2))
    assert np.array_equal(P.np_(probs).view(np.uint32), P.np_(p2).view(np.uint32))
    assert np.array_equal(P.np_(tok), P.np_(t2))
    return P.np_(logits), P.np_(tok), P.np_(ids), P.np_(probs)


@pytest.mark.parametrize("k,temp,p", [(1, 0.6, 0.95), (29, 0.6, 0.95), (64, 1.7, 0.5), (8, 0.05, 1.0)])
def test_one_launch_equals_two_launch_full_head(ops, full_head, k, temp, p):
    assert ops.lm_head_sample_path(1, 157184, 2560, k) == 1
    for j in range(3):
        x = inputs.normal_bf16((41, k, j), (1, 2560), 1.0)
        u = inputs.uniform_f32((42, k, j), (1,))
        lg, tok, ids, probs = fused_vs_two_launch(ops, full_head["q"], full_head["s"], x, temp, k, p, u)
        check_row(lg[0], temp, k, p, float(u[0]), int(tok[0]), ids[0], probs[0])


def test_one_launch_all_equal_logits(ops, full_head):
    """A zero activation row: every logit is 0, so the top k are rows 0..k-1
    in order, spread over the first wavefronts of the first workgroup, and
    the tail's cuts run on maxima that differ only by row."""
    x = np.zeros((1, 2560), dtype=np.uint16)
    for k in (1, 29, 64):
        u = np.array([0.999], dtype=np.float32)
        lg, tok, ids, probs = fused_vs_two_launch(ops, full_head["q"], full_head["s"], x, 1.0, k, 1.0, u)
        assert np.all(lg == 0.0)
        assert list(ids[0]) == list(range(k))
        assert tok[0] == k - 1


def test_one_launch_planted_leaders(ops):
    """A head whose top rows are planted in one workgroup's rows and tied
    across workgroups: rows with equal codes give equal logits, so the ranking
    must fall back to the lower row across chunk and workgroup boundaries."""
    V, K = 157184, 2560
    g = np.random.default_rng(9)
    q = (g.integers(0, 256, size=(V, K)).astype(np.uint8) & 0x87) | 0x20     # |e4m3| small
    s = np.ones(V, dtype=np.float32)
    lead = np.array([5, 6, 7, 8, 1000, 64 * 16 * 4 + 5, 150001, 157183])      # several in one group, one in the tail
    q[lead] = 0x40                                                             # 2.0 everywhere: the largest logits, tied
    x = F.f64_to_bf16_rne(np.ones((1, K)))
    qd, sd = P.to_dev(q), P.to_dev(s)
    for k in (4, 8, 29):
        u = inputs.uniform_f32((43, k), (1,))
        lg, tok, ids, probs = fused_vs_two_launch(ops, qd, sd, x, 0.6, k, 0.95, u)
        assert list(ids[0][:min(k, 8)]) == sorted(lead)[:min(k, 8)]
        check_row(lg[0], 0.6, k, 0.95, float(u[0]), int(tok[0]), ids[0], probs[0])


@pytest.mark.parametrize("V,K,k", [(4099, 256, 64), (2048, 256, 29), (16384 + 7, 256, 29), (70001, 2560, 29)])
def test_one_launch_other_vocabularies(ops, V, K, k):
    assert ops.lm_head_sample_path(1, V, K, k) == 1
    w = inputs.normal_bf16((44, V, K), (V, K), 0.02)
    q, s = ops.lm_head_quantize_fp8(P.to_dev_bf16(w))
    x = inputs.normal_bf16((45, V, K), (1, K), 1.0)
    u = inputs.uniform_f32((46, V, K), (1,))
    lg, tok, ids, probs = fused_vs_two_launch(ops, q, s, x, 0.6, k, 0.95, u)
    ok, worst = C.fp_close(lg, OH.head_logits(P.np_(q), P.np_(s), x))
    assert ok, worst
    check_row(lg[0], 0.6, k, 0.95, float(u[0]), int(tok[0]), ids[0], probs[0])


def test_one_launch_reuses_its_workspace(ops, full_head):
    """One workspace, many calls with changing inputs: the counter returns to
    zero and every published maximum is rewritten, so each call equals a call
    on a fresh workspace."""
    ws = ops.workspace(int(_lib_mod().load().wsx_lm_head_sample_workspace_bytes(1, 157184, 2560, 29)), "cuda")
    for j in range(4):
        x = inputs.normal_bf16((47, j), (1, 2560), 1.0)
        u = inputs.uniform_f32((48, j), (1,))
        a = ops.lm_head_gemv_fp8_sample(full_head["q"], full_head["s"], P.to_dev_bf16(x), 0.6, 29, 0.95, P.to_dev(u),
                                        ws=ws)
        b = ops.lm_head_gemv_fp8_sample(full_head["q"], full_head["s"], P.to_dev_bf16(x), 0.6, 29, 0.95, P.to_dev(u))
        for y, z in zip(a, b):
            assert torch.equal(y, z)


def _lib_mod():
    from weight_streaming_expert_amd import _lib
    return _lib
