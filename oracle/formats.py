"""Number formats used on the decode path, decoded from their bit-field definitions.

TEST INFRASTRUCTURE ONLY (see the package docstring).

* MXFP4 routed-expert weights: [saipien] "Why one user waits on weights" names
  the checkpoint's MXFP4 expert kernels; [genai] "DGX Spark Can Hold the Whole
  Model" names the MXFP4 checkpoint.  An MXFP4 tensor is E2M1 4-bit elements
  sharing one E8M0 power-of-two scale per 32 consecutive elements along K.
* FP8 LM head: [saipien] "Stop hauling the vocabulary in full precision" and
  [genai] "2. Compressing the Output Head": the BF16 head is quantized to FP8
  when the layer is built.  The FP8 flavour is OCP E4M3FN.
* bf16: the upper 16 bits of an IEEE binary32.

Pins (tests/test_oracle_formats.py): E4M3 decode and encode against torch's
float8_e4m3fn conversion (a library routine, exhaustive over all codes and a
dense input sweep); E2M1 decode against torch's float8_e4m3fn decode of the
re-packed bit fields plus the value-set invariants; E8M0 against exact powers
of two; bf16 rounding against torch's float32->bfloat16 conversion.
"""

import numpy as np

# ----------------------------------------------------------------------------- E2M1


def decode_e2m1(code):
    """E2M1 (sign, 2-bit exponent with bias 1, 1-bit mantissa) -> float64.

    Exponent field 0 is subnormal: m * 0.5.  Otherwise 2**(e-1) * (1 + m/2).
    No inf/NaN encodings exist.
    """
    c = np.asarray(code, dtype=np.int64) & 0xF
    s = (c >> 3) & 1
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, m * 0.5, np.ldexp(1.0 + m / 2.0, (e - 1).astype(np.int64)))
    return np.where(s == 1, -mag, mag).astype(np.float64)


def decode_e8m0(b):
    """E8M0 block scale -> float64: 2**(b-127); the byte 0xFF encodes NaN."""
    b = np.asarray(b, dtype=np.int64)
    out = np.ldexp(np.ones(b.shape, dtype=np.float64), b - 127)
    return np.where(b == 255, np.nan, out)


def dequant_mxfp4(codes, scales, K):
    """Dequantize an MXFP4 matrix stored row-major along K.

    codes:  uint8 [..., N, K/2]; element 2j of a row sits in the LOW nibble of
            byte j and element 2j+1 in the HIGH nibble.
    scales: uint8 [..., N, K/32]; byte b scales elements 32b .. 32b+31.
    Returns float64 [..., N, K], exact (every value is E2M1 * 2**e).
    """
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    assert codes.shape[-1] * 2 == K and scales.shape[-1] * 32 == K
    lo = decode_e2m1(codes & 0xF)
    hi = decode_e2m1(codes >> 4)
    vals = np.empty(codes.shape[:-1] + (K,), dtype=np.float64)
    vals[..., 0::2] = lo
    vals[..., 1::2] = hi
    sc = np.repeat(decode_e8m0(scales), 32, axis=-1)
    return vals * sc


# ----------------------------------------------------------------------------- E4M3FN


def decode_e4m3fn(code):
    """OCP E4M3FN (sign, 4-bit exponent with bias 7, 3-bit mantissa) -> float64.

    Exponent field 0: (m/8) * 2**-6.  Otherwise (1 + m/8) * 2**(e-7).
    S.1111.111 is NaN; there is no infinity; the largest finite value is 448.
    """
    c = np.asarray(code, dtype=np.int64) & 0xFF
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 7
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64)))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag).astype(np.float64)


E4M3_MAX = 448.0

# All non-negative finite E4M3FN magnitudes, indexed by code 0..126.  They are
# strictly increasing with the code, which is what the encoder relies on.
_E4M3_POS = decode_e4m3fn(np.arange(127))


def encode_e4m3fn_rne(v):
    """Round float values to the nearest E4M3FN code, ties to the even code.

    The input must already lie in [-448, 448] (callers saturate first).  The
    sign bit is kept, so negative values that round to zero give 0x80.
    Written from the definition: pick the nearer of the two representable
    neighbours of |v|; on an exact tie pick the one whose mantissa LSB is 0.
    """
    v = np.asarray(v, dtype=np.float64)
    if np.any(np.abs(v) > E4M3_MAX) or np.any(np.isnan(v)):
        raise ValueError("encode_e4m3fn_rne expects finite values within +-448")
    a = np.abs(v)
    hi = np.searchsorted(_E4M3_POS, a, side="left")          # first value >= a
    hi = np.minimum(hi, 126)
    lo = np.maximum(hi - 1, 0)
    exact = _E4M3_POS[hi] == a
    d_lo = a - _E4M3_POS[lo]
    d_hi = _E4M3_POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(exact, hi, np.where(pick_hi, hi, lo)).astype(np.int64)
    sign = np.signbit(v).astype(np.int64)
    return (code | (sign << 7)).astype(np.uint8)


# ----------------------------------------------------------------------------- bf16


def bf16_to_f64(bits):
    """bf16 bit patterns (uint16) -> float64 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16_rne(x):
    """Round float64 values straight to bf16 (8 significant bits), ties to even.

    Returns uint16 bit patterns.  Values beyond the bf16 range become +-inf.
    The unit in the last place of x in [2**(e-1), 2**e) is 2**(e-8), floored at
    the subnormal quantum 2**-133.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    ulp = np.ldexp(1.0, np.maximum(e, -125) - 8)
    r = np.rint(x / ulp) * ulp
    r32 = r.astype(np.float32)  # exact: r has at most 8 significant bits (or overflows to inf)
    with np.errstate(over="ignore"):
        r32 = np.where(np.abs(r) > float(np.finfo(np.float32).max), np.copysign(np.inf, r), r32).astype(np.float32)
    return (r32.view(np.uint32) >> 16).astype(np.uint16)
