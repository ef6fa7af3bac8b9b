"""Comparison rules between a device result and the oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring).

* Floating-point outputs: max |gpu - ref| <= 2e-3 * RMS(ref), RMS taken per
  token over the output vector.
* Argmax and top-k ids: bit-exact, except where the oracle's logits hold a
  near tie, i.e. two candidates within 1e-3 * |top logit| of each other.
  There the device may pick either member; the check then verifies that what
  it picked is still a valid answer within that band.
"""

import numpy as np

FP_REL_TOL = 2e-3
NEAR_TIE_REL = 1e-3


def rms(a, axis=-1):
    a = np.asarray(a, dtype=np.float64)
    return np.sqrt(np.mean(a * a, axis=axis))


def fp_error_ratio(gpu, ref):
    """Per row: max |gpu - ref| / RMS(ref).  Rows are the leading axes."""
    gpu = np.atleast_2d(np.asarray(gpu, dtype=np.float64))
    ref = np.atleast_2d(np.asarray(ref, dtype=np.float64))
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    err = np.max(np.abs(gpu - ref), axis=-1)
    scale = rms(ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        return np.where(scale > 0, err / scale, np.where(err == 0, 0.0, np.inf))


def fp_close(gpu, ref, rel=FP_REL_TOL):
    r = fp_error_ratio(gpu, ref)
    return bool(np.all(r <= rel)), float(np.max(r))


def near_tie_set(logits_row, rel=NEAR_TIE_REL):
    """Ids whose logit is within rel*|top| of the top logit."""
    l = np.asarray(logits_row, dtype=np.float64)
    top = l.max()
    return np.nonzero(top - l <= rel * abs(top))[0]


def check_argmax(gpu_idx, ref_logits, rel=NEAR_TIE_REL):
    """Returns (ok, n_near_tie_tokens).  Exact where the near-tie set has one
    member; otherwise the device's pick must lie in the near-tie set."""
    ref_logits = np.atleast_2d(ref_logits)
    gpu_idx = np.atleast_1d(gpu_idx)
    ok, ties = True, 0
    for t in range(ref_logits.shape[0]):
        s = near_tie_set(ref_logits[t], rel)
        if s.size == 1:
            ok &= int(gpu_idx[t]) == int(s[0])
        else:
            ties += 1
            ok &= int(gpu_idx[t]) in set(int(v) for v in s)
    return bool(ok), ties


def check_topk(gpu_ids, ref_logits, k, rel=NEAR_TIE_REL):
    """Top-k ids in rank order.  Returns (ok, n_tokens_with_a_near_tie).

    With delta = rel * |largest logit| of the token:
      * no unselected expert may beat a selected one by more than delta, and
      * the rank order may invert only pairs within delta;
    where every gap among the k+1 best logits exceeds delta this forces the
    oracle's exact ordered list, which is then required bit for bit."""
    gpu_ids = np.atleast_2d(gpu_ids)
    ref_logits = np.atleast_2d(np.asarray(ref_logits, dtype=np.float64))
    ok, ties = True, 0
    from .moe import topk_order
    for t in range(ref_logits.shape[0]):
        l = ref_logits[t]
        g = gpu_ids[t].astype(np.int64)
        E = l.shape[0]
        if len(set(g.tolist())) != k or g.min() < 0 or g.max() >= E:
            return False, ties
        delta = rel * abs(l.max())
        ref = topk_order(l, min(k + 1, E))
        srt = l[ref]
        gaps = -np.diff(srt)
        if np.all(gaps > delta):
            ok &= bool(np.array_equal(g, ref[:k]))
            continue
        ties += 1
        sel = np.zeros(E, dtype=bool)
        sel[g] = True
        if (~sel).any():
            ok &= bool(l[sel].min() >= l[~sel].max() - delta)
        ok &= bool(np.all(l[g][:-1] >= l[g][1:] - delta))
    return bool(ok), ties
