"""The one-launch decode step compiled at run time (hipRTC) for stack shapes
that are not compiled ahead of time, checked layer by layer against the
oracle with teacher forcing, as the precompiled shapes are; and consecutive
calls, which reuse the compiled kernel."""

import numpy as np
import pytest
import torch

from weight_streaming_expert_amd import configs, inputs
import parity as P
from test_gpu_decode import build_stack, check_step

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from weight_streaming_expert_amd import ops as _ops
    return _ops


@pytest.mark.parametrize("name", ["rtc_stack_h512_e64_top4_i128", "rtc_stack_h384_e40_top3_i96"])
def test_runtime_compiled_step_matches_the_oracle(ops, name):
    wl = configs.ALL[name] if name in configs.ALL else {w.name: w for w in (configs.RTC_A, configs.RTC_B)}[name]
    layers, stack = build_stack(ops, wl, wl.layers)
    assert ops.decode_step_path(1, stack) == 2
    head = ops.Fp8LmHead.quantize(P.to_dev_bf16(inputs.head_weights(wl, K=wl.moe.H)))
    qh, sh = P.np_(head.q), P.np_(head.s)
    ws = ops.workspace(ops.decode_step_workspace_bytes(1, wl.moe.H, wl.moe.I, wl.moe.E, wl.moe.k, head.V), "cuda")
    first = None
    for step in range(3):
        h0 = inputs.normal_bf16((wl.seed, inputs.T_X, step), (1, wl.moe.H), 1.0)
        out = ops.moe_decode_step(P.to_dev_bf16(h0), stack, head, trace=True, ws=ws)
        check_step(wl, layers, out, qh, sh, h0)
        assert int(out["argmax"][0]) >= 0
        if first is None:
            first = (h0, {k: v.clone() for k, v in out.items()})
    again = ops.moe_decode_step(P.to_dev_bf16(first[0]), stack, head, ws=ws)
    assert torch.equal(again["h"], first[1]["h"]) and torch.equal(again["logits"], first[1]["logits"])


def test_tiny_shape_with_a_bf16_router_is_compiled_at_run_time(ops):
    """The tiny shape is compiled ahead of time with an fp32 router only; with
    its router in bf16 the step is compiled at run time."""
    wl = configs.TINY
    layers, stack = build_stack(ops, wl, 2)
    router = stack.w_router.to(torch.bfloat16).contiguous()
    st = ops.MoeStackTensors(router, stack.w13_codes, stack.w13_scales, stack.w2_codes, stack.w2_scales,
                             shared=stack.shared, k=stack.k)
    assert ops.decode_step_path(1, st) == 2
    layers_b = [dict(lw, router=P.bits(router[l])) for l, lw in enumerate(layers)]
    head = ops.Fp8LmHead.quantize(P.to_dev_bf16(inputs.head_weights(wl, K=wl.moe.H)))
    h0 = inputs.normal_bf16((wl.seed, 93), (1, wl.moe.H), 1.0)
    out = ops.moe_decode_step(P.to_dev_bf16(h0), st, head, trace=True)
    check_step(wl, layers_b, out, P.np_(head.q), P.np_(head.s), h0)
