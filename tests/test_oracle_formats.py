"""Pins for the oracle's number formats, each against a route other than the
oracle's own bit-field formula (torch's float8 conversion, IEEE binary32 bit
patterns, the E2M1 value table, torch's bfloat16 rounding)."""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F


def torch_e4m3_decode(codes):
    t = torch.from_numpy(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = F.decode_e4m3fn(codes)
    ref = torch_e4m3_decode(codes)
    assert np.array_equal(ours, ref, equal_nan=True)
    assert np.isnan(ours[0x7F]) and np.isnan(ours[0xFF])
    assert ours[0x7E] == 448.0 and ours[0xFE] == -448.0
    assert ours[0x01] == 2.0 ** -9          # smallest subnormal


def _e4m3_inputs():
    vals = []
    bits = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    vals.append(bits)
    vals.append(((np.arange(65536, dtype=np.uint32) << 16) | 0x8000).view(np.float32))  # bf16 midpoints
    g = np.random.default_rng(5)
    vals.append((g.uniform(-448, 448, 200000) * 2.0 ** g.integers(-20, 1, 200000)).astype(np.float32))
    v = np.concatenate(vals)
    v = v[np.isfinite(v) & (np.abs(v) <= 448)]
    return v


def test_e4m3_encode_matches_torch_rne():
    v = _e4m3_inputs()
    ours = F.encode_e4m3fn_rne(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_encode_ties_go_to_even():
    # 1 + 1/16 lies halfway between 1 (code 0x38, mantissa 0) and 1.125 (0x39, mantissa 1)
    assert F.encode_e4m3fn_rne(np.array([1.0625]))[0] == 0x38
    # 1.1875 lies halfway between 1.125 (0x39) and 1.25 (0x3A): even mantissa is 0x3A
    assert F.encode_e4m3fn_rne(np.array([1.1875]))[0] == 0x3A
    # halfway between the two smallest subnormals 2^-9 and 2^-8
    assert F.encode_e4m3fn_rne(np.array([1.5 * 2.0 ** -9]))[0] == 0x02
    assert F.encode_e4m3fn_rne(np.array([-0.5 * 2.0 ** -9]))[0] == 0x80   # rounds to -0
    with pytest.raises(ValueError):
        F.encode_e4m3fn_rne(np.array([449.0]))


# The E2M1 magnitudes for codes 0..7 (OCP MX v1.0 FP4 E2M1 value table).
E2M1_TABLE = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4), Fraction(6)]


def test_e2m1_decode_matches_value_table():
    ours = F.decode_e2m1(np.arange(16))
    for c in range(16):
        ref = float(E2M1_TABLE[c & 7]) * (-1.0 if c & 8 else 1.0)
        assert ours[c] == ref, c
    assert np.signbit(ours[8])            # code 8 is -0


def test_e2m1_decode_matches_torch_via_e4m3_repacking():
    """Re-express each E2M1 code as the E4M3 code of the same value by moving
    its fields (exponent bias 1 -> 7, mantissa 1 bit -> 3 bits) and decode that
    with torch."""
    out = []
    for c in range(16):
        s, e, m = (c >> 3) & 1, (c >> 1) & 3, c & 1
        if e == 0 and m == 0:
            code8 = 0
        elif e == 0:                 # subnormal 0.5 = 2^-1 -> E4M3 exponent field 6
            code8 = 6 << 3
        else:
            code8 = ((e - 1 + 7) << 3) | (m << 2)
        out.append(code8 | (s << 7))
    ref = torch_e4m3_decode(np.array(out, dtype=np.uint8))
    assert np.array_equal(F.decode_e2m1(np.arange(16)), ref)


def test_e8m0_matches_binary32_bit_patterns():
    b = np.arange(255)
    # 2^(b-127) as an IEEE binary32: exponent field b for b >= 1, subnormal 2^-127 for b = 0
    bits = np.where(b >= 1, b.astype(np.uint32) << 23, np.uint32(1 << 22)).astype(np.uint32)
    ref = bits.view(np.float32).astype(np.float64)
    assert np.array_equal(F.decode_e8m0(b), ref)
    assert np.isnan(F.decode_e8m0(np.array([255]))[0])


def test_dequant_mxfp4_planted_layout():
    """Plant known E2M1 values and scales, pack them nibble by nibble with plain
    integer operations (element 2j low nibble, 2j+1 high nibble; one scale per
    32 elements), and check the oracle returns the planted matrix."""
    g = np.random.default_rng(1)
    N, K = 5, 96
    codes4 = g.integers(0, 16, size=(N, K))
    sexp = g.integers(-8, 5, size=(N, K // 32))
    packed = np.zeros((N, K // 2), dtype=np.uint8)
    for n in range(N):
        for j in range(K // 2):
            packed[n, j] = int(codes4[n, 2 * j]) | (int(codes4[n, 2 * j + 1]) << 4)
    sbytes = (sexp + 127).astype(np.uint8)
    expect = np.zeros((N, K))
    for n in range(N):
        for kk in range(K):
            c = int(codes4[n, kk])
            v = float(E2M1_TABLE[c & 7]) * (-1.0 if c & 8 else 1.0)
            expect[n, kk] = v * 2.0 ** int(sexp[n, kk // 32])
    assert np.array_equal(F.dequant_mxfp4(packed, sbytes, K), expect)


def test_bf16_rounding_matches_torch_on_binary32_inputs():
    g = np.random.default_rng(2)
    x = np.concatenate([
        (g.standard_normal(200000) * 10.0 ** g.integers(-30, 30, 200000)).astype(np.float32),
        ((np.arange(65536, dtype=np.uint32) << 16) | 0x8000).view(np.float32),   # exact bf16 midpoints
        ((np.arange(65536, dtype=np.uint32) << 16) | 0x7FFF).view(np.float32),
        ((np.arange(65536, dtype=np.uint32) << 16) | 0x8001).view(np.float32),
        np.array([1e-40, -1e-40, 3.3e38, -3.3e38, 0.0, -0.0], dtype=np.float32),
    ])
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ours = F.f64_to_bf16_rne(x.astype(np.float64))
    assert np.array_equal(ours, ref)


def test_bf16_rounding_of_float64_is_direct_not_double():
    # 1 + 2^-8 + 2^-30 is above the midpoint between 1 and 1 + 2^-7: must round up,
    # although rounding through binary32 first would drop the 2^-30 and tie to 1.
    x = 1.0 + 2.0 ** -8 + 2.0 ** -30
    assert F.bf16_to_f64(F.f64_to_bf16_rne(np.array([x])))[0] == 1.0 + 2.0 ** -7
    assert F.bf16_to_f64(F.f64_to_bf16_rne(np.array([1.0 + 2.0 ** -8])))[0] == 1.0
    assert F.bf16_to_f64(F.f64_to_bf16_rne(np.array([1.0 + 3 * 2.0 ** -8])))[0] == 1.0 + 2.0 ** -6
    assert np.isinf(F.bf16_to_f64(F.f64_to_bf16_rne(np.array([3.5e38])))[0])
