"""LM head: load-time FP8 quantization and the per-token GEMV + greedy argmax.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[saipien] "Stop hauling the vocabulary in full precision", [ncij] "What are the
3 optimizations?" and [genai] "2. Compressing the Output Head": only the
2,560 -> 157,184 BF16 language-model head is quantized to FP8, once, when the
layer is built; every decode step then reads half the bytes.  [ncij] "What
happens on a real workload?": the synthetic run decodes greedily, i.e. the next
token is the argmax of the logits.

Readings taken (the pages name FP8 only): OCP E4M3FN codes with one fp32 scale
per vocabulary row, s = absmax(row) / 448 computed as an IEEE binary32
division, each element w / s (binary32 division) saturated to +-448 and rounded
to nearest-even; an all-zero row gets s = 0 and all codes 0.  Because the
quotients are binary32 operations, each code has exactly one correct value.

Pins (tests/test_oracle_head.py): codes against torch's float8_e4m3fn
conversion of the same binary32 quotients over every finite bf16 pattern;
round-trip error bounds; the +-448 code in every nonzero row; the zero row;
the byte count halving; logits against torch's fp64 matmul over torch-decoded
codes; exact small-integer cases; argmax ties to the lowest index.
"""

import numpy as np

from .formats import E4M3_MAX, bf16_to_f64, decode_e4m3fn, encode_e4m3fn_rne


def quantize_row_scales(w_bits):
    """Per-row scale s = fl32(absmax / 448) for bf16 rows [V][K] -> float32 [V]."""
    w = bf16_to_f64(w_bits).astype(np.float32)        # exact
    amax = np.max(np.abs(w), axis=-1)
    return (amax / np.float32(E4M3_MAX)).astype(np.float32)


def quantize_fp8(w_bits):
    """BF16 [V][K] -> (E4M3FN codes uint8 [V][K], fp32 row scales [V])."""
    w = bf16_to_f64(np.atleast_2d(w_bits)).astype(np.float32)
    s = quantize_row_scales(w_bits).reshape(-1)
    q = np.zeros(w.shape, dtype=np.uint8)
    nz = s > 0
    if np.any(nz):
        v = (w[nz] / s[nz][:, None]).astype(np.float32)        # binary32 division
        v = np.clip(v, -E4M3_MAX, E4M3_MAX)
        q[nz] = encode_e4m3fn_rne(v)
    return q, s


def head_logits(q, s, x_bits, chunk=8192):
    """logit[t][v] = s[v] * sum_k E4M3(q[v][k]) * x[t][k], fp64.  Rows are decoded
    in chunks so the full 157,184 x 2,560 head never exists in fp64 at once."""
    x = bf16_to_f64(np.atleast_2d(x_bits))
    V = q.shape[0]
    out = np.empty((x.shape[0], V), dtype=np.float64)
    lut = decode_e4m3fn(np.arange(256))
    for r0 in range(0, V, chunk):
        r1 = min(V, r0 + chunk)
        W = lut[q[r0:r1]]
        out[:, r0:r1] = (x @ W.T) * np.asarray(s[r0:r1], dtype=np.float64)[None, :]
    return out


def head_logits_bf16(w_bits, x_bits, chunk=8192):
    """Unquantized BF16 head (the 2x-bytes comparison): logit = W x, fp64."""
    x = bf16_to_f64(np.atleast_2d(x_bits))
    V = w_bits.shape[0]
    out = np.empty((x.shape[0], V), dtype=np.float64)
    for r0 in range(0, V, chunk):
        r1 = min(V, r0 + chunk)
        out[:, r0:r1] = x @ bf16_to_f64(w_bits[r0:r1]).T
    return out


def greedy_argmax(logits):
    """Per token, the index of the largest logit; ties go to the lowest index."""
    logits = np.atleast_2d(logits)
    return np.argmax(logits, axis=-1).astype(np.int32)
