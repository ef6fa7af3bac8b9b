"""Ling-style MoE layer at batch 1 (and the 4-token verify variant), in fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the layer computes, per token t with input row x[t] (H values):
  1. Router logits  l[e] = sum_h Wr[e][h] * x[h]  for every routed expert e.
     [saipien] "Why one user waits on weights": a router sends each token to
     8 of 512 routed experts plus one shared expert that always runs; [ncij]
     "What is Ling 3.0, and why does it suit DGX Spark?" repeats the counts.
  2. Top-k: order experts by (logit descending, id ascending), keep k.  The
     routing weights are the softmax of the k kept logits (reading taken: the
     pages give only the 8-of-512 count; no bias, no group limit, scale 1).
  3. Each selected expert and the shared expert is a SwiGLU FFN with a narrow
     intermediate size ([saipien] "Kernels built for the shape you actually
     have": intermediate 768): g = Wg x, u = Wu x, a = silu(g) * u, d = Wd a.
     gate rows are rows 0..I-1 and up rows are rows I..2I-1 of one [2I][H]
     MXFP4 matrix (reading taken; the pages do not give the storage).
  4. y = sum_i w_i d_{e_i} + d_shared (shared weight 1), then the bf16
     residual h' = RNE_bf16(h + y).
  5. The 4-token MTP-verify pass ([saipien] "Draft three tokens, verify four";
     [genai] "3. Predicting Several Tokens at Once") scores 4 positions in one
     pass, so up to 4*8 = 32 distinct routed experts plus the shared one are
     read.  Its result is by definition 4 independent 1-token evaluations.
  6. Decode-step composition (reading taken; the pages give no norm): each
     layer's input is the unit-gain RMS norm of the bf16 residual stream,
     rounded to bf16; the LM head reads the same norm of the last stream.
     Without a norm the synthetic stack overflows within a few layers.

Intermediates stay unrounded (fp64 here); a GPU keeps them in fp32.

Pins (tests/test_oracle_moe.py): top-k against a brute-force full sort and all
orderings of small inputs, ties to the lowest id; softmax sums and special
cases; silu against scipy's expit; the dequantized contraction against exact
rational arithmetic on tiny inputs (fractions.Fraction, written from the bit
layout independently of formats.py); one-hot inputs returning a planted
column; the identical-experts invariant; the RMS norm against torch's
rms_norm; the verify pass against per-token runs.
"""

import numpy as np

from .formats import bf16_to_f64, dequant_mxfp4, f64_to_bf16_rne

# ----------------------------------------------------------------------------- router


def router_logits(x_bits, w_router):
    """Router GEMV in fp64.  x_bits: bf16 bits [T][H]; w_router: float array [E][H]
    holding the exact router weights (fp32 values, or bf16 values decoded)."""
    x = bf16_to_f64(x_bits)
    return x @ np.asarray(w_router, dtype=np.float64).T   # [T][E]


def topk_order(logits_row, k):
    """Indices of the k largest logits, ordered by (logit desc, id asc)."""
    l = np.asarray(logits_row, dtype=np.float64)
    ids = np.arange(l.shape[0])
    order = np.lexsort((ids, -l))          # primary key -l, secondary key id
    return order[:k].astype(np.int32)


def softmax_selected(sel_logits):
    """w_i = exp(l_i - l_max) / sum_j exp(l_j - l_max) over the selected logits."""
    l = np.asarray(sel_logits, dtype=np.float64)
    z = np.exp(l - l.max())
    return z / z.sum()


def route(logits, k):
    """Per-token top-k ids (rank order) and softmax weights. logits: [T][E]."""
    logits = np.atleast_2d(np.asarray(logits, dtype=np.float64))
    T = logits.shape[0]
    ids = np.zeros((T, k), dtype=np.int32)
    w = np.zeros((T, k), dtype=np.float64)
    for t in range(T):
        ids[t] = topk_order(logits[t], k)
        w[t] = softmax_selected(logits[t][ids[t]])
    return ids, w


def expert_list(topk_ids, topk_w):
    """Union of the routed ids of all tokens, ascending, and the slot weight table.

    Returns (ids [n_active] int32 ascending, slot_w [n_active][T] with the
    routing weight of token t for that expert, 0 where t did not pick it)."""
    topk_ids = np.atleast_2d(topk_ids)
    topk_w = np.atleast_2d(topk_w)
    T = topk_ids.shape[0]
    ids = np.unique(topk_ids).astype(np.int32)
    slot_w = np.zeros((ids.shape[0], T), dtype=np.float64)
    for t in range(T):
        for j in range(topk_ids.shape[1]):
            s = int(np.searchsorted(ids, topk_ids[t, j]))
            slot_w[s, t] = topk_w[t, j]
    return ids, slot_w


# ----------------------------------------------------------------------------- experts


def silu(g):
    """silu(g) = g / (1 + exp(-g)); for very negative g exp overflows and the
    quotient is -0, never NaN."""
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def gate_up(x_bits, w13_codes, w13_scales, I):
    """a = silu(Wg x) * (Wu x) for one expert; x_bits bf16 [T][H] -> a [T][I] fp64."""
    x = bf16_to_f64(np.atleast_2d(x_bits))
    H = x.shape[1]
    W = dequant_mxfp4(w13_codes, w13_scales, H)      # [2I][H]
    g = x @ W[:I].T
    u = x @ W[I:2 * I].T
    return silu(g) * u


def down(a, w2_codes, w2_scales):
    """d = Wd a for one expert; a [T][I] (fp64 or fp32 values) -> d [T][H] fp64."""
    a = np.atleast_2d(np.asarray(a, dtype=np.float64))
    I = a.shape[1]
    W = dequant_mxfp4(w2_codes, w2_scales, I)        # [H][I]
    return a @ W.T


def combine(d_routed, slot_w, d_shared=None):
    """y[t] = sum_s slot_w[s][t] * d_routed[s][t] (+ d_shared[t]).

    d_routed: [S][T][H]; slot_w: [S][T]."""
    d_routed = np.asarray(d_routed, dtype=np.float64)
    slot_w = np.asarray(slot_w, dtype=np.float64)
    y = np.einsum("st,sth->th", slot_w, d_routed)
    if d_shared is not None:
        y = y + np.asarray(d_shared, dtype=np.float64)
    return y


def residual_bf16(h_bits, y):
    """h' = RNE_bf16(h + y), the sum taken exactly in fp64."""
    return f64_to_bf16_rne(bf16_to_f64(h_bits) + np.asarray(y, dtype=np.float64))


def rmsnorm_f64(h_bits, eps=1e-6):
    """h / sqrt(mean(h^2) + eps), unit gain, per token row, unrounded fp64."""
    h = bf16_to_f64(np.atleast_2d(h_bits))
    r = 1.0 / np.sqrt(np.mean(h * h, axis=-1, keepdims=True) + eps)
    return h * r


def rmsnorm_bf16(h_bits, eps=1e-6):
    """u = RNE_bf16(h / sqrt(mean(h^2) + eps)): the next layer's (or the head's) input."""
    return f64_to_bf16_rne(rmsnorm_f64(h_bits, eps))


# ----------------------------------------------------------------------------- whole layer


def moe_layer(x_bits, w_router, k, experts, shared=None, residual_bits=None, I=None):
    """One MoE layer for T tokens, every stage in fp64.

    experts: callable e -> (w13_codes, w13_scales, w2_codes, w2_scales) so a
    caller can regenerate single experts instead of holding all of them.
    shared:  the same 4-tuple for the shared expert, or None.
    Returns a dict with logits, topk ids/weights, expert list, slot weights,
    y and (when residual_bits is given) the bf16 residual h'.
    """
    x_bits = np.atleast_2d(x_bits)
    logits = router_logits(x_bits, w_router)
    ids, w = route(logits, k)
    elist, slot_w = expert_list(ids, w)
    d = []
    for e in elist:
        c13, s13, c2, s2 = experts(int(e))
        a = gate_up(x_bits, c13, s13, I)
        d.append(down(a, c2, s2))
    d_sh = None
    if shared is not None:
        c13, s13, c2, s2 = shared
        d_sh = down(gate_up(x_bits, c13, s13, I), c2, s2)
    y = combine(np.stack(d), slot_w, d_sh)
    out = dict(logits=logits, topk_ids=ids, topk_w=w, expert_list=elist, slot_w=slot_w, y=y)
    if residual_bits is not None:
        out["h"] = residual_bf16(residual_bits, y)
    return out
