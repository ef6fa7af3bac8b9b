"""Seeded synthetic inputs, shared by the tests, the benchmark and the oracle checks.

This module only draws random numbers: it holds none of the decode path's
arithmetic.  Every tensor is keyed by (workload seed, tensor id, layer,
expert, token) through numpy's SeedSequence, so any single expert of any layer
can be regenerated on the host without generating the rest.

Recipes:
  * MXFP4 codes: uniform random bytes, i.e. each 4-bit E2M1 code uniform over
    its 16 values.
  * E8M0 scale bytes: 127 + e with e uniform on an integer range, or
    e = rint(N(mean, std)) (half-even) clamped to [-127, 127].
  * Router weights: N(0, 0.02) as fp32 or rounded to bf16.
  * Activations: N(0, 1) rounded to bf16.
  * LM head: N(0, 0.02) rounded to bf16, generated in 8192-row chunks.
Rounding to bf16 uses torch's float32 -> bfloat16 conversion.
"""

from concurrent.futures import ThreadPoolExecutor
import os

import numpy as np

T_ROUTER, T_W13C, T_W13S, T_W2C, T_W2S, T_X, T_HEAD, T_XPERT = 1, 2, 3, 4, 5, 6, 7, 8
SHARED = -1
HEAD_CHUNK = 8192


def rng(*key):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) + 2**31 for k in key])))


def _to_bf16_bits(f32):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def uniform_bytes(key, shape):
    n = int(np.prod(shape))
    raw = rng(*key).bit_generator.random_raw((n + 7) // 8)
    return raw.view(np.uint8)[:n].reshape(shape)


def scale_bytes(key, shape, dist):
    g = rng(*key)
    if dist[0] == "uniform":
        e = g.integers(int(dist[1]), int(dist[2]) + 1, size=shape)
    elif dist[0] == "normal":
        z = g.standard_normal(size=shape, dtype=np.float32)
        e = np.rint(np.float32(dist[1]) + np.float32(dist[2]) * z)
        e = np.clip(e, -127, 127)
    else:
        raise ValueError(dist)
    return (e.astype(np.int64) + 127).astype(np.uint8)


def normal_f32(key, shape, std):
    return (rng(*key).standard_normal(size=shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def normal_bf16(key, shape, std):
    return _to_bf16_bits(normal_f32(key, shape, std))


def uniform_f32(key, shape):
    """Draws in [0, 1) as float32 (the sampler's per-token uniforms)."""
    u = rng(*key).random(size=shape, dtype=np.float32)
    return np.minimum(u, np.nextafter(np.float32(1), np.float32(0))).astype(np.float32)


# ----------------------------------------------------------------------------- MoE weights


def expert_weights(wl, layer, expert):
    """(w13_codes [2I][H/2], w13_scales [2I][H/32], w2_codes [H][I/2], w2_scales [H][I/32])
    of routed expert `expert`, or of the shared expert when expert == SHARED."""
    m = wl.moe
    e = expert + 1
    s = wl.seed
    return (uniform_bytes((s, T_W13C, layer, e), (2 * m.I, m.H // 2)),
            scale_bytes((s, T_W13S, layer, e), (2 * m.I, m.H // 32), m.scale_dist),
            uniform_bytes((s, T_W2C, layer, e), (m.H, m.I // 2)),
            scale_bytes((s, T_W2S, layer, e), (m.H, m.I // 32), m.scale_dist))


def router_weights(wl, layer):
    """Router [E][H]: float32 values, or bf16 bits (uint16) when the router is bf16."""
    m = wl.moe
    if m.router_dtype == "f32":
        return normal_f32((wl.seed, T_ROUTER, layer), (m.E, m.H), m.router_std)
    return normal_bf16((wl.seed, T_ROUTER, layer), (m.E, m.H), m.router_std)


def layer_weights(wl, layer, out=None, threads=None):
    """All routed experts of one layer, stacked: dict of arrays with a leading
    [E] axis (w13c, w13s, w2c, w2s), plus 'router' and 'shared' (4-tuple).
    `out` may supply preallocated arrays (e.g. pinned host buffers) to fill."""
    m = wl.moe
    shapes = dict(w13c=(m.E, 2 * m.I, m.H // 2), w13s=(m.E, 2 * m.I, m.H // 32),
                  w2c=(m.E, m.H, m.I // 2), w2s=(m.E, m.H, m.I // 32))
    if out is None:
        out = {k: np.empty(v, dtype=np.uint8) for k, v in shapes.items()}

    def fill(e):
        c13, s13, c2, s2 = expert_weights(wl, layer, e)
        out["w13c"][e] = c13
        out["w13s"][e] = s13
        out["w2c"][e] = c2
        out["w2s"][e] = s2

    nthreads = threads or min(16, os.cpu_count() or 1)
    with ThreadPoolExecutor(nthreads) as ex:
        list(ex.map(fill, range(m.E)))
    out["router"] = router_weights(wl, layer)
    out["shared"] = expert_weights(wl, layer, SHARED) if m.shared else None
    return out


# ----------------------------------------------------------------------------- activations / head


def activations(wl, step):
    """Input rows [T][H] (bf16 bits) for pass `step`: T independent N(0,1) tokens."""
    return normal_bf16((wl.seed, T_X, step), (wl.T, wl.moe.H), 1.0)


def overlapping_activations(wl, step, spread=0.05):
    """Verify-pass input whose tokens 1..T-1 are small perturbations of token 0,
    so several tokens share routed experts."""
    base = normal_f32((wl.seed, T_XPERT, step, 0), (1, wl.moe.H), 1.0)
    rows = [base[0]]
    for t in range(1, wl.T):
        rows.append(base[0] + normal_f32((wl.seed, T_XPERT, step, t), (wl.moe.H,), spread))
    return _to_bf16_bits(np.stack(rows))


def head_weights(wl, K=None, threads=None, out=None):
    """BF16 head [V][K] (uint16 bits), N(0, head_std), generated per 8192-row chunk."""
    K = K or wl.moe.H
    V = wl.V
    if out is None:
        out = np.empty((V, K), dtype=np.uint16)

    def fill(c):
        r0 = c * HEAD_CHUNK
        r1 = min(V, r0 + HEAD_CHUNK)
        out[r0:r1] = normal_bf16((wl.seed, T_HEAD, c), (r1 - r0, K), wl.head_std)

    nthreads = threads or min(16, os.cpu_count() or 1)
    with ThreadPoolExecutor(nthreads) as ex:
        list(ex.map(fill, range((V + HEAD_CHUNK - 1) // HEAD_CHUNK)))
    return out
