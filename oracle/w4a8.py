"""W4A8 variant of the MoE layer: MXFP4 weights with 8-bit activations, in fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[saipien] "Why one user waits on weights": the official baseline of the DGX
Spark runs was the "W4A8" recipe, with MXFP4 kernels for the experts; the page
notes that NVIDIA leaves W4A8 undefined and that the term usually means 4-bit
weights and 8-bit activations.  [ncij] "Why is MoE decoding on DGX Spark
memory-bound?" gives the same baseline.

Readings taken (the pages define neither the 8-bit format nor where it
applies):
  * 8-bit activations are MXFP8 with E4M3 elements (the OCP microscaling
    format that pairs with the MXFP4 weights): each block of 32 consecutive
    elements along the contraction dimension shares one E8M0 scale 2^X with
    X = floor(log2(max |v|)) - 8, 8 being the exponent of E4M3's largest power
    of two; X is clamped to [-127, 127] and an all-zero block takes X = -127.
    Each element is v / 2^X rounded to the nearest E4M3 value (ties to even)
    after saturating to +-448.  The top of a block can saturate (a block
    maximum of 1.875 * 2^e maps to 480 and is stored as 448): that is the
    format's rule, kept as is.
  * Both activations that enter an expert contraction are quantized: the
    layer input u before gate/up (from its bf16 values) and the SwiGLU output
    a before down (from its binary32 values, the precision the device holds
    it in, so both sides take the same rounding decisions when given the same
    a).
  * Weights, routing, the silu, the weighted combine, the shared expert and
    the residual are as in moe.py.  Products and sums are exact here (fp64).

Pins (tests/test_oracle_w4a8.py): the block exponent against a brute-force
search over powers of two; element codes against torch's float8_e4m3fn
conversion of the same scaled values; round-trip error bounds; the largest
element of every nonzero block landing in [256, 448]; zero and saturating
blocks; exactness on blocks of small integers, where the W4A8 layer must
equal the bf16-activation layer of moe.py; the contraction against exact
rational arithmetic on tiny inputs.
"""

import numpy as np

from .formats import E4M3_MAX, bf16_to_f64, decode_e4m3fn, decode_e8m0, dequant_mxfp4, encode_e4m3fn_rne
from .moe import combine, residual_bf16, silu

MX_BLOCK = 32
E4M3_EMAX = 8        # exponent of the largest power of two in E4M3 (256)


def mx_exponent(amax):
    """Shared block exponent X = floor(log2(amax)) - 8, clamped to [-127, 127];
    amax = 0 gives -127."""
    amax = np.asarray(amax, dtype=np.float64)
    _, e = np.frexp(np.where(amax > 0, amax, 1.0))       # amax = f * 2^e, f in [0.5, 1)
    X = (e - 1) - E4M3_EMAX
    X = np.where(amax > 0, X, -127)
    return np.clip(X, -127, 127).astype(np.int64)


def quantize_mxfp8(v):
    """Values [..., K] (K a multiple of 32) -> (E4M3 codes uint8 [..., K],
    E8M0 scale bytes uint8 [..., K/32])."""
    v = np.asarray(v, dtype=np.float64)
    K = v.shape[-1]
    assert K % MX_BLOCK == 0
    blocks = v.reshape(v.shape[:-1] + (K // MX_BLOCK, MX_BLOCK))
    X = mx_exponent(np.max(np.abs(blocks), axis=-1))
    scaled = blocks * np.ldexp(1.0, -X)[..., None]              # exact: a power of two
    scaled = np.clip(scaled, -E4M3_MAX, E4M3_MAX)
    codes = encode_e4m3fn_rne(scaled).reshape(v.shape)
    return codes, (X + 127).astype(np.uint8)


def dequant_mxfp8(codes, scales):
    """E4M3 codes [..., K] with E8M0 bytes [..., K/32] -> float64 [..., K] (exact)."""
    codes = np.asarray(codes, dtype=np.uint8)
    vals = decode_e4m3fn(codes)
    return vals * np.repeat(decode_e8m0(scales), MX_BLOCK, axis=-1)


def quantize_bf16_rows(x_bits):
    """The layer input: bf16 rows [T][H] -> MXFP8 codes and scales."""
    return quantize_mxfp8(bf16_to_f64(np.atleast_2d(x_bits)))


def gate_up_w4a8(x_bits, w13_codes, w13_scales, I):
    """a = silu(Wg xq) * (Wu xq) for one expert, xq the MXFP8 form of the bf16
    input rows [T][H]; returns a [T][I] in fp64."""
    q, s = quantize_bf16_rows(x_bits)
    xq = dequant_mxfp8(q, s)
    H = xq.shape[1]
    W = dequant_mxfp4(w13_codes, w13_scales, H)
    return silu(xq @ W[:I].T) * (xq @ W[I:2 * I].T)


def down_w4a8(a, w2_codes, w2_scales):
    """d = Wd aq for one expert, aq the MXFP8 form of a [T][I] taken from its
    binary32 values."""
    a32 = np.atleast_2d(np.asarray(a, dtype=np.float64)).astype(np.float32).astype(np.float64)
    q, s = quantize_mxfp8(a32)
    aq = dequant_mxfp8(q, s)
    W = dequant_mxfp4(w2_codes, w2_scales, aq.shape[1])
    return aq @ W.T


def moe_y_w4a8(x_bits, expert_ids, slot_w, experts, shared, I, acts=None):
    """y [T][H] of the W4A8 layer for given routing: expert_ids ascending
    [n_active], slot_w [n_active][T].  experts: e -> (w13c, w13s, w2c, w2s).

    acts: optional activations [n_slots][T][I] to use as the down stage's
    input (the slots in list order, then the shared expert): the device's own
    binary32 a, so that the down stage's quantization decisions are taken on
    the same values on both sides.  None: this module's own a."""
    d = []
    for s, e in enumerate(expert_ids):
        c13, s13, c2, s2 = experts(int(e))
        a = gate_up_w4a8(x_bits, c13, s13, I) if acts is None else acts[s]
        d.append(down_w4a8(a, c2, s2))
    d_sh = None
    if shared is not None:
        a = gate_up_w4a8(x_bits, shared[0], shared[1], I) if acts is None else acts[len(expert_ids)]
        d_sh = down_w4a8(a, shared[2], shared[3])
    return combine(np.stack(d), slot_w, d_sh)


def moe_layer_w4a8(x_bits, expert_ids, slot_w, experts, shared, I, residual_bits=None):
    """The W4A8 layer's outputs for given routing: y and, with a residual,
    h' = RNE_bf16(h + y)."""
    y = moe_y_w4a8(x_bits, expert_ids, slot_w, experts, shared, I)
    out = dict(y=y)
    if residual_bits is not None:
        out["h"] = residual_bf16(residual_bits, y)
    return out
