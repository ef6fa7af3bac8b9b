"""Workload shapes and synthetic-input recipes for the decode path.

Shapes come from the pages: [saipien] "Why one user waits on weights"
(8 of 512 routed experts plus one shared expert; the 2,560 x 157,184 BF16
head) and "Kernels built for the shape you actually have" (expert
intermediate size 768).  The distributions define the synthetic stand-ins
for the trained checkpoint, which is not available.
"""

from dataclasses import dataclass, field


@dataclass(frozen=True)
class MoEShape:
    H: int            # hidden size
    I: int            # expert intermediate size
    E: int            # routed experts
    k: int            # experts chosen per token
    router_dtype: str  # "f32" or "bf16"
    router_std: float = 0.02
    # E8M0 scale exponent distribution: ("uniform", lo, hi) inclusive, or ("normal", mean, std) rounded half-even
    scale_dist: tuple = ("normal", -6.0, 1.0)
    shared: bool = True


@dataclass(frozen=True)
class Workload:
    name: str
    T: int                         # tokens scored per pass (1 = decode, 4 = MTP verify)
    moe: MoEShape = None
    layers: int = 0                # stacked MoE layers (0 = none)
    V: int = 0                     # vocabulary rows of the LM head (0 = no head)
    head_std: float = 0.02
    steps: int = 1                 # seeded tokens / passes the workload runs
    seed: int = 0
    notes: str = ""


LING_MOE = MoEShape(H=2560, I=768, E=512, k=8, router_dtype="bf16", scale_dist=("normal", -6.0, 1.0))
TINY_MOE = MoEShape(H=256, I=64, E=16, k=2, router_dtype="f32", scale_dist=("uniform", -4, 2))

# Tiny decode: one MoE layer (16 experts top-2 + shared, H=256, I=64) then a 4096 x 256 FP8 head.
TINY = Workload("tiny_moe_fp8_head", T=1, moe=TINY_MOE, layers=1, V=4096, steps=8, seed=11,
                notes="MoE on the raw N(0,1) input, head on RNE_bf16(x + y)")
# One Ling-shaped MoE layer, 1 token, 100 seeded tokens, each measured with a cold cache.
MOE_LAYER = Workload("moe_layer_h2560_e512_top8_i768", T=1, moe=LING_MOE, layers=1, steps=100, seed=21)
# The 157,184 x 2,560 LM head quantized to FP8 at load, 1 token.
LM_HEAD = Workload("lm_head_157184x2560_fp8", T=1, V=157184, moe=MoEShape(H=2560, I=768, E=512, k=8, router_dtype="bf16"),
                   steps=100, seed=31)
# MTP verify: the MoE layer on 4 tokens with independent top-8 routing, then the head on 4 rows.
VERIFY = Workload("mtp_verify_t4", T=4, moe=LING_MOE, layers=1, V=157184, steps=100, seed=41)
# A small batch or a longer draft: the MoE layer on 16 tokens with independent top-8 routing.
GROUPED16 = Workload("moe_layer_grouped_t16", T=16, moe=LING_MOE, layers=1, steps=20, seed=61)
# Stacks of shapes the one-launch step is not compiled for ahead of time (compiled at run time).
RTC_A = Workload("rtc_stack_h512_e64_top4_i128", T=1, layers=2, V=2048, seed=71,
                 moe=MoEShape(H=512, I=128, E=64, k=4, router_dtype="bf16"))
RTC_B = Workload("rtc_stack_h384_e40_top3_i96", T=1, layers=3, V=1000, seed=72,
                 moe=MoEShape(H=384, I=96, E=40, k=3, router_dtype="f32", scale_dist=("uniform", -4, 2)))
# Full decode step: 32 stacked MoE layers (512 experts each) then the FP8 head, 2000 seeded tokens.
DECODE_STEP = Workload("decode_step_32x_moe_fp8_head", T=1, moe=LING_MOE, layers=32, V=157184, steps=2000, seed=51)

ALL = {w.name: w for w in (TINY, MOE_LAYER, LM_HEAD, VERIFY, GROUPED16, DECODE_STEP)}


def mxfp4_bytes(N, K):
    """Bytes of an MXFP4 [N][K] matrix: K/2 code bytes + K/32 scale bytes per row."""
    return N * K // 2 + N * K // 32


def expert_bytes(m: MoEShape):
    return mxfp4_bytes(2 * m.I, m.H) + mxfp4_bytes(m.H, m.I)


def router_bytes(m: MoEShape):
    return m.E * m.H * (4 if m.router_dtype == "f32" else 2)


def moe_layer_bytes(m: MoEShape, n_active):
    """Algorithmic bytes of one MoE layer pass: router + every active routed expert
    + the shared expert (weights only)."""
    return router_bytes(m) + (n_active + (1 if m.shared else 0)) * expert_bytes(m)


def head_bytes(V, K, T=1, fp8=True):
    """Algorithmic bytes of one head pass: weights (+ fp32 row scales for FP8)
    plus the fp32 logits written."""
    w = V * K * (1 if fp8 else 2) + (V * 4 if fp8 else 0)
    return w + T * V * 4
