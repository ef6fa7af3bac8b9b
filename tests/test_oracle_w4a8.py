"""Pins of the W4A8 oracle (oracle/w4a8.py) against things other than itself:
a brute-force search for the block exponent, torch's float8_e4m3fn
conversion, round-trip bounds of the format, exact rational arithmetic, and
the bf16-activation layer of oracle/moe.py on inputs the 8-bit format holds
exactly."""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import moe as OM
from oracle import w4a8 as W

RNG = np.random.default_rng(1234)


def brute_exponent(amax):
    """The X in [-127, 127] with 2^(X+8) <= amax < 2^(X+9), found by trying
    every X (clamped at the ends); -127 for amax = 0."""
    if amax == 0:
        return -127
    for X in range(127, -128, -1):
        if amax >= 2.0 ** (X + 8):
            return X
    return -127


def test_block_exponent_against_brute_force():
    vals = [0.0, 1.0, 255.9, 256.0, 256.1, 447.0, 448.0, 511.9, 512.0, 2.0 ** -130, 2.0 ** 140, 3e38, 1e-3]
    vals += list(np.ldexp(1.0, np.arange(-140, 140, 7)))
    vals += list(np.ldexp(1.0, np.arange(-140, 140, 7)) * (1 - 2.0 ** -20))
    vals += list(np.abs(RNG.standard_normal(200)) * 10.0 ** RNG.integers(-20, 20, 200))
    got = W.mx_exponent(np.array(vals))
    want = np.array([brute_exponent(v) for v in vals])
    assert np.array_equal(got, want)


def random_blocks(n, scale_pow):
    """n blocks of 32 float32 values with varied magnitudes and signs."""
    v = RNG.standard_normal((n, 32)).astype(np.float32)
    v *= np.float32(2.0) ** RNG.integers(-scale_pow, scale_pow + 1, (n, 1)).astype(np.float32)
    v *= (RNG.random((n, 32)) < 0.9)                                   # some exact zeros
    v[::7, 3] *= 1e-4                                                   # small members of large blocks
    return v.astype(np.float32)


def test_codes_against_torch_float8():
    v = random_blocks(400, 30).reshape(10, 40 * 32)
    q, s = W.quantize_mxfp8(v)
    X = s.astype(np.int64) - 127
    scaled = v.reshape(10, 40, 32).astype(np.float64) * np.ldexp(1.0, -X)[..., None]
    scaled32 = np.clip(scaled, -448, 448).astype(np.float32)                       # exact
    assert np.array_equal(scaled32.astype(np.float64), np.clip(scaled, -448, 448))
    ref = torch.from_numpy(scaled32).to(torch.float8_e4m3fn).view(torch.uint8).numpy().reshape(10, -1)
    assert np.array_equal(q, ref)


def test_round_trip_bounds_and_top_binade():
    v = random_blocks(2000, 40).astype(np.float64)
    q, s = W.quantize_mxfp8(v)
    d = W.dequant_mxfp8(q, s)
    X = (s.astype(np.int64) - 127)[:, 0]
    sc = np.ldexp(1.0, X)[:, None]
    a = np.abs(v) / sc
    normal = (a >= 2.0 ** -6) & (a <= 448)
    assert np.all(np.abs(d - v)[normal] <= 2.0 ** -4 * np.abs(v)[normal])
    sub = a < 2.0 ** -6
    assert np.all(np.abs(d - v)[sub] <= (2.0 ** -10 * sc * np.ones_like(v))[sub])
    sat = a > 448
    assert np.all(np.abs(d)[sat] == (448 * sc * np.ones_like(v))[sat])
    nz = np.max(np.abs(v), axis=1) > 0
    top = np.max(np.abs(d), axis=1)[nz] / sc[nz, 0]
    assert np.all((top >= 256) & (top <= 448))


def test_zero_and_saturating_blocks():
    z = np.zeros((1, 64))
    q, s = W.quantize_mxfp8(z)
    assert np.all(q == 0) and np.all(s == 0)
    b = np.zeros((1, 32))
    b[0, 5] = 1.875 * 2.0 ** 3          # scaled to 480: saturates to 448
    b[0, 6] = -1.0
    q, s = W.quantize_mxfp8(b)
    assert int(s[0, 0]) == 127 + 3 - 8
    # -1.0 / 2^-5 = -32 = -(1.0 * 2^5): sign, exponent field 5 + 7 = 12, mantissa 0
    assert q[0, 5] == 0x7E and q[0, 6] == 0x80 | (12 << 3)
    assert F.decode_e4m3fn(np.array([0x80 | (12 << 3)]))[0] == -32.0


def fr_e2m1(c):
    s = -1 if c & 8 else 1
    e, m = (c >> 1) & 3, c & 1
    return s * (Fraction(m, 2) if e == 0 else Fraction(2) ** (e - 1) * (1 + Fraction(m, 2)))


def fr_e4m3(c):
    s = -1 if c & 0x80 else 1
    e, m = (c >> 3) & 15, c & 7
    return s * (Fraction(m, 8) * Fraction(1, 64) if e == 0 else Fraction(2) ** (e - 7) * (1 + Fraction(m, 8)))


def test_gate_up_against_exact_rationals():
    """The whole W4A8 gate/up of one expert, recomputed in exact rational
    arithmetic from the bit fields (E2M1, E4M3 and E8M0 written out again
    here); silu is applied to the exact g."""
    H, I = 64, 32
    x = F.f64_to_bf16_rne(RNG.standard_normal((2, H)))
    c13 = RNG.integers(0, 256, (2 * I, H // 2), dtype=np.uint8)
    s13 = (127 + RNG.integers(-3, 4, (2 * I, H // 32))).astype(np.uint8)
    a = W.gate_up_w4a8(x, c13, s13, I)
    q, s = W.quantize_bf16_rows(x)
    for t in range(2):
        xq = [fr_e4m3(int(q[t, h])) * Fraction(2) ** (int(s[t, h // 32]) - 127) for h in range(H)]
        for i in range(0, I, 5):
            def row(r):
                tot = Fraction(0)
                for h in range(H):
                    byte = int(c13[r, h // 2])
                    code = (byte >> 4) if h % 2 else (byte & 15)
                    tot += fr_e2m1(code) * Fraction(2) ** (int(s13[r, h // 32]) - 127) * xq[h]
                return tot
            g, u = float(row(i)), float(row(I + i))
            assert a[t, i] == pytest.approx(g / (1 + np.exp(-g)) * u, rel=1e-12, abs=1e-300)


def test_exact_on_small_integer_blocks_equals_bf16_layer():
    """Blocks whose values are in {0, +-1, +-2, +-3, +-4} with a +-4 in each
    are held exactly by MXFP8, so the W4A8 gate/up equals the bf16-activation
    gate/up of moe.py, and so does the whole layer when the SwiGLU outputs are
    also held exactly."""
    H, I = 256, 64
    x = RNG.integers(-4, 5, (3, H)).astype(np.float64)
    x[:, ::32] = 4.0
    xb = F.f64_to_bf16_rne(x)
    q, s = W.quantize_bf16_rows(xb)
    assert np.array_equal(W.dequant_mxfp8(q, s), x)
    c13 = RNG.integers(0, 256, (2 * I, H // 2), dtype=np.uint8)
    s13 = (127 + RNG.integers(-2, 3, (2 * I, H // 32))).astype(np.uint8)
    assert np.array_equal(W.gate_up_w4a8(xb, c13, s13, I), OM.gate_up(xb, c13, s13, I))
    a = RNG.integers(-3, 4, (3, I)).astype(np.float64)
    a[:, ::32] = 4.0
    c2 = RNG.integers(0, 256, (H, I // 2), dtype=np.uint8)
    s2 = (127 + RNG.integers(-2, 3, (H, I // 32))).astype(np.uint8)
    assert np.array_equal(W.down_w4a8(a, c2, s2), OM.down(a, c2, s2))


def test_layer_combines_like_the_bf16_layer():
    """With activations the format holds exactly (one routed expert whose
    gate/up is fed the layer input, the activations given explicitly), the
    W4A8 layer's combine, shared expert and residual equal moe.py's."""
    H, I, E = 64, 32, 4
    ex = {e: (RNG.integers(0, 256, (2 * I, H // 2), dtype=np.uint8),
              (127 + RNG.integers(-2, 3, (2 * I, H // 32))).astype(np.uint8),
              RNG.integers(0, 256, (H, I // 2), dtype=np.uint8),
              (127 + RNG.integers(-2, 3, (H, I // 32))).astype(np.uint8)) for e in range(E + 1)}
    x = F.f64_to_bf16_rne(RNG.standard_normal((2, H)))
    ids = np.array([1, 3])
    sw = np.array([[0.25, 0.0], [0.75, 1.0]])
    acts = RNG.integers(-4, 5, (3, 2, I)).astype(np.float64)
    acts[:, :, 0] = 4.0
    y = W.moe_y_w4a8(x, ids, sw, ex.__getitem__, ex[E], I, acts=acts)
    d = np.stack([OM.down(acts[s], ex[int(e)][2], ex[int(e)][3]) for s, e in enumerate(ids)])
    want = OM.combine(d, sw, OM.down(acts[2], ex[E][2], ex[E][3]))
    assert np.array_equal(y, want)
