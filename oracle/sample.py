"""Seeded temperature / top-k / top-p sampling of one token from the LM-head
logits: the sampling epilogue of the head.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[ncij] "What happens on a real workload?": the GSM8K run samples with
temperature 0.6, top_p 0.95 and top_k 29 instead of decoding greedily.  The
pages name the three settings and nothing else, so the steps below are a
reading, the usual one for these three knobs:

  1. order the vocabulary by (logit descending, id ascending) and keep the
     first top_k entries: z_0 >= z_1 >= ... >= z_{k-1};
  2. e_i = exp((z_i - z_0) / temperature), the softmax numerators over the k
     kept logits (subtracting z_0 changes nothing but the range);
  3. c_i = e_0 + ... + e_i (added in rank order), Z = c_{k-1};
  4. top-p: keep ranks 0..m, m the smallest index with c_m >= top_p * Z
     (so at least one token survives, and top_p = 1 keeps all k);
  5. the probabilities are p_i = e_i / c_m for i <= m, 0 beyond;
  6. with one uniform u in [0, 1) per token (passed in, not drawn here), the
     token is rank j, the first j <= m with c_j > u * c_m (j = m if rounding
     leaves none).

The arithmetic of steps 2-6 is binary32 in exactly this order: the sampled
token is an integer decided by floating-point comparisons, and the HIP kernel
takes those decisions in binary32, so this oracle does too.  The logits it is
given are binary32 (a head oracle's fp64 logits rounded once).

Pins (tests/test_oracle_sample.py): top_k = 1 and tiny top_p give the argmax;
with top_k = V and top_p = 1 the interval widths are scipy's softmax of
logits / temperature; the kept set is the smallest high-probability set of
mass >= top_p, by brute force over all subsets of a tiny vocabulary, and so
are cumulative_bounds' kept ranks at top_p < 1 after a top-k cut, with widths
from an fp64 softmax renormalised over the kept set; a worked
example by hand (tests/golden/sampling_example.json); u -> 0 gives rank 0 and
u -> 1 the last kept rank; a constant added to every logit changes nothing;
sampling frequencies over a fine grid of u match the probabilities.
"""

import numpy as np


def ranked_topk(logits_row, k):
    """Step 1: ids of the k largest logits, by (value desc, id asc)."""
    z = np.asarray(logits_row, dtype=np.float32)
    order = np.lexsort((np.arange(z.size), -z.astype(np.float64)))
    return order[:k].astype(np.int64)


def sample_row(logits_row, temperature, top_k, top_p, u):
    """Steps 1-6 for one token.  Returns (token id, kept ids [top_k] in rank
    order, probabilities [top_k] float32 with zeros past the top-p cut)."""
    z = np.asarray(logits_row, dtype=np.float32)
    ids = ranked_topk(z, top_k)
    zk = z[ids]
    t = np.float32(temperature)
    e = np.empty(top_k, dtype=np.float32)
    for i in range(top_k):
        d = np.float32(zk[i] - zk[0])
        e[i] = np.exp(np.float32(d / t), dtype=np.float32)
    c = np.empty(top_k, dtype=np.float32)
    acc = np.float32(0.0)
    for i in range(top_k):
        acc = np.float32(acc + e[i])
        c[i] = acc
    thr = np.float32(np.float32(top_p) * c[top_k - 1])
    m = top_k - 1
    for i in range(top_k):
        if c[i] >= thr:
            m = i
            break
    mass = c[m]
    p = np.zeros(top_k, dtype=np.float32)
    for i in range(m + 1):
        p[i] = np.float32(e[i] / mass)
    target = np.float32(np.float32(u) * mass)
    j = m
    for i in range(m + 1):
        if c[i] > target:
            j = i
            break
    return int(ids[j]), ids, p


def cumulative_bounds(logits_row, temperature, top_k, top_p):
    """The interval [lo_j, hi_j) of u that selects each kept rank j, in fp64
    (for tolerance checks of a sampler whose logits differ by rounding)."""
    z = np.asarray(logits_row, dtype=np.float64)
    ids = ranked_topk(np.asarray(logits_row, dtype=np.float32), top_k)
    e = np.exp((z[ids] - z[ids[0]]) / temperature)
    c = np.cumsum(e)
    m = int(np.argmax(c >= top_p * c[-1]))
    hi = c[:m + 1] / c[m]
    lo = np.concatenate(([0.0], hi[:-1]))
    return ids[:m + 1], lo, hi
