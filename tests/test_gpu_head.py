"""GPU parity of the LM-head path: load-time FP8 quantizer (bit-exact codes and
scales), FP8 and BF16 GEMVs with the fused argmax, at small ragged shapes and
at the full 157,184 x 2,560 head."""

import numpy as np
import pytest
import torch

from oracle import compare as C
from oracle import formats as F
from oracle import head as OH
from weight_streaming_expert_amd import configs, inputs
import parity as P

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from weight_streaming_expert_amd import ops as _ops
    return _ops


def all_finite_bf16_rows(K=256):
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = F.bf16_to_f64(b)
    b = b[np.isfinite(v)]
    b = b[np.argsort(np.abs(F.bf16_to_f64(b)), kind="stable")]
    pad = (-len(b)) % K
    b = np.concatenate([b, np.zeros(pad, dtype=np.uint16)]).reshape(-1, K)
    g = np.random.default_rng(0)
    for r in b:
        g.shuffle(r)
    return np.concatenate([b, np.zeros((1, K), np.uint16), np.full((1, K), 0x8000, np.uint16)])


def test_quantizer_every_finite_bf16_pattern_bit_exact(ops):
    w = all_finite_bf16_rows()
    q, s = ops.lm_head_quantize_fp8(P.to_dev_bf16(w))
    qr, sr = OH.quantize_fp8(w)
    assert np.array_equal(P.np_(s).view(np.uint32), sr.view(np.uint32))
    assert np.array_equal(P.np_(q), qr)


@pytest.mark.parametrize("V,K", [(1, 32), (7, 96), (33, 2560), (5, 16384)])
def test_quantizer_ragged_shapes(ops, V, K):
    w = inputs.normal_bf16((5, V, K), (V, K), 0.02)
    w[0, :] = 0
    q, s = ops.lm_head_quantize_fp8(P.to_dev_bf16(w))
    qr, sr = OH.quantize_fp8(w)
    assert np.array_equal(P.np_(q), qr) and np.array_equal(P.np_(s), sr)


@pytest.fixture(scope="module")
def full_head(ops):
    wl = configs.LM_HEAD
    w = inputs.head_weights(wl)
    wd = P.to_dev_bf16(w)
    q, s = ops.lm_head_quantize_fp8(wd)
    torch.cuda.synchronize()
    return dict(w=w, wd=wd, q=q, s=s, qh=P.np_(q), sh=P.np_(s))


def test_quantizer_full_head_sampled_rows(full_head):
    V = full_head["w"].shape[0]
    rows = np.unique(np.concatenate([np.arange(64), np.arange(V - 64, V),
                                     np.random.default_rng(1).integers(0, V, 3000)]))
    qr, sr = OH.quantize_fp8(full_head["w"][rows])
    assert np.array_equal(full_head["qh"][rows], qr)
    assert np.array_equal(full_head["sh"][rows], sr)
    assert full_head["qh"].nbytes * 2 == full_head["w"].nbytes


@pytest.mark.parametrize("T", [1, 2, 4])
def test_fp8_head_full_size(ops, full_head, T):
    wl = configs.LM_HEAD
    x = inputs.normal_bf16((wl.seed, inputs.T_X, 1000 + T), (T, 2560), 1.0)
    logits, am = ops.lm_head_gemv_fp8_argmax(full_head["q"], full_head["s"], P.to_dev_bf16(x))
    P.check_head(full_head["qh"], full_head["sh"], x, P.np_(logits), P.np_(am))


@pytest.mark.parametrize("T", [1, 4])
def test_bf16_head_full_size(ops, full_head, T):
    x = inputs.normal_bf16((77, T), (T, 2560), 1.0)
    logits, am = ops.lm_head_gemv_bf16_argmax(full_head["wd"], P.to_dev_bf16(x))
    P.check_head(None, None, x, P.np_(logits), P.np_(am), bf16_w=full_head["w"])


@pytest.mark.parametrize("V,K", [(1, 32), (5, 96), (17, 256), (4099, 256), (3, 2560), (1000, 2560), (300, 4096)])
@pytest.mark.parametrize("T", [1, 2, 3, 4])
def test_heads_ragged_shapes(ops, V, K, T):
    w = inputs.normal_bf16((9, V, K), (V, K), 0.02)
    x = inputs.normal_bf16((10, T, K), (T, K), 1.0)
    wd, xd = P.to_dev_bf16(w), P.to_dev_bf16(x)
    q, s = ops.lm_head_quantize_fp8(wd)
    logits, am = ops.lm_head_gemv_fp8_argmax(q, s, xd)
    P.check_head(P.np_(q), P.np_(s), x, P.np_(logits), P.np_(am))
    logits, am = ops.lm_head_gemv_bf16_argmax(wd, xd)
    P.check_head(None, None, x, P.np_(logits), P.np_(am), bf16_w=w)
    _, am2 = ops.lm_head_gemv_fp8_argmax(q, s, xd, want_logits=False)
    assert np.array_equal(P.np_(am2), P.np_(ops.lm_head_gemv_fp8_argmax(q, s, xd)[1]))


@pytest.mark.parametrize("T", [1, 4])
def test_fp8_head_exact_small_integers(ops, T):
    g = np.random.default_rng(3)
    V, K = 3001, 2560
    q = g.integers(0, 256, size=(V, K)).astype(np.uint8)
    big = ((q >> 3) & 0xF) > 7
    q[big] = (q[big] & 0x87) | 0x38          # |value| < 2: every partial sum is an exact binary32
    s = (2.0 ** g.integers(-3, 4, size=V)).astype(np.float32)
    xi = g.integers(-3, 4, size=(T, K))
    x = torch.from_numpy(xi.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    m = np.round(F.decode_e4m3fn(q) * 512).astype(np.int64)     # every E4M3 value is an integer / 512
    exact = (xi @ m.T).astype(np.float64) / 512.0 * s.astype(np.float64)[None, :]
    logits, am = ops.lm_head_gemv_fp8_argmax(P.to_dev(q), P.to_dev(s), P.to_dev_bf16(x))
    assert np.array_equal(P.np_(logits).astype(np.float64), exact)
    assert np.array_equal(P.np_(am), np.argmax(exact, axis=1))


@pytest.mark.parametrize("T", [1, 2])
def test_head_ties_go_to_lowest_index(ops, T):
    """Rows 777, 5001 and 19000 tie for the top logit; they are read by
    different workgroups, and the argmax takes the lowest row."""
    V, K = 20000, 2560
    w = inputs.normal_bf16((12,), (V, K), 0.02)
    w[[777, 5001, 19000]] = 0x3D4D                        # bf16 0.05 in every element
    x = np.full((T, K), 0x3F80, dtype=np.uint16)          # all ones: rows 777, 5001, 19000 tie for the top
    wd = P.to_dev_bf16(w)
    q, s = ops.lm_head_quantize_fp8(wd)
    logits, am = ops.lm_head_gemv_fp8_argmax(q, s, P.to_dev_bf16(x))
    lg = P.np_(logits)
    assert lg[0, 777] == lg[0, 5001] == lg[0, 19000] == lg[0].max()
    assert list(P.np_(am)) == [777] * T
    _, amb = ops.lm_head_gemv_bf16_argmax(wd, P.to_dev_bf16(x))
    assert list(P.np_(amb)) == [777] * T


def test_head_is_deterministic(ops, full_head):
    x = P.to_dev_bf16(inputs.normal_bf16((13,), (4, 2560), 1.0))
    a = ops.lm_head_gemv_fp8_argmax(full_head["q"], full_head["s"], x)
    for _ in range(5):
        b = ops.lm_head_gemv_fp8_argmax(full_head["q"], full_head["s"], x)
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("T", [2, 3, 4])
def test_fp8_multi_row_head_equals_one_row_head(ops, full_head, T):
    """At 2..4 rows each row's products are added in the 1-token head's order,
    so its logits and argmax equal the 1-token head's on that row, bit for
    bit; one workspace serves the calls one after another (its counter and
    maxima return to zero)."""
    dev = torch.device("cuda:0")
    ws = ops.workspace(ops.lm_head_workspace_bytes(T, full_head["q"].shape[0], 2560), dev)
    for rep in range(2):
        x = inputs.normal_bf16((21, T, rep), (T, 2560), 1.0)
        xd = P.to_dev_bf16(x)
        lg, am = ops.lm_head_gemv_fp8_argmax(full_head["q"], full_head["s"], xd, ws=ws)
        lg, am = P.np_(lg), P.np_(am)
        for t in range(T):
            l1, a1 = ops.lm_head_gemv_fp8_argmax(full_head["q"], full_head["s"], xd[t:t + 1].contiguous())
            assert np.array_equal(lg[t], P.np_(l1)[0]), (T, t)
            assert int(am[t]) == int(P.np_(a1)[0]), (T, t)
