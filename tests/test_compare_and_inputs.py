"""Host-side checks of the comparison rules and the seeded input recipes."""

import numpy as np

from oracle import compare as C
from oracle import formats as F
from weight_streaming_expert_amd import configs, inputs


def test_fp_close_rule():
    ref = np.array([[1.0, -1.0, 1.0, -1.0]])
    ok, r = C.fp_close(ref + 1.9e-3, ref)
    assert ok and abs(r - 1.9e-3) < 1e-12
    assert not C.fp_close(ref + 2.1e-3, ref)[0]


def test_argmax_near_tie_rule():
    l = np.array([[10.0, 9.9995, 3.0], [1.0, 5.0, 2.0]])
    ok, ties = C.check_argmax([1, 1], l)
    assert ok and ties == 1
    assert not C.check_argmax([2, 1], l)[0]
    assert not C.check_argmax([0, 0], l)[0]


def test_topk_near_tie_rule():
    l = np.array([[5.0, 4.0, 3.0, 2.0, 1.0]])
    assert C.check_topk([[0, 1]], l, 2) == (True, 0)
    assert not C.check_topk([[1, 0]], l, 2)[0]
    l2 = np.array([[5.0, 4.0, 3.9999, 2.0, 1.0]])
    assert C.check_topk([[0, 2]], l2, 2) == (True, 1)
    assert not C.check_topk([[0, 3]], l2, 2)[0]
    assert not C.check_topk([[0, 0]], l2, 2)[0]


def test_inputs_are_deterministic_and_keyed():
    wl = configs.TINY
    a = inputs.expert_weights(wl, 0, 3)
    b = inputs.expert_weights(wl, 0, 3)
    c = inputs.expert_weights(wl, 0, 4)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    assert not np.array_equal(a[0], c[0])
    bulk = inputs.layer_weights(wl, 0, threads=2)
    assert np.array_equal(bulk["w13c"][3], a[0]) and np.array_equal(bulk["w2s"][3], a[3])


def test_input_distributions():
    wl = configs.TINY
    c13, s13, c2, s2 = inputs.expert_weights(wl, 0, 0)
    e = s13.astype(int) - 127
    assert e.min() >= -4 and e.max() <= 2 and set(np.unique(e)) == set(range(-4, 3))
    big = inputs.scale_bytes((1, 2, 3), (200000,), ("normal", -6.0, 1.0)).astype(int) - 127
    assert abs(big.mean() + 6.0) < 0.02 and abs(big.std() - np.sqrt(1 + 1 / 12)) < 0.02
    nib = np.concatenate([c13 & 15, c13 >> 4]).ravel()
    counts = np.bincount(nib, minlength=16)
    assert counts.min() > 0.8 * counts.mean()
    x = F.bf16_to_f64(inputs.activations(configs.MOE_LAYER, 0))
    assert x.shape == (1, 2560) and abs(x.std() - 1.0) < 0.05
    r = F.bf16_to_f64(inputs.router_weights(configs.MOE_LAYER, 0))
    assert r.shape == (512, 2560) and abs(r.std() - 0.02) < 0.001
