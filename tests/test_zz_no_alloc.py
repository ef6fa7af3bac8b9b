"""The allocation-free decode step (moe_decode_step_noalloc) against the
allocating one (moe_decode_step), both called through the C ABI on the same
inputs: outputs and traces must be identical bit for bit.  The calls come in
a row on the one device array the library keeps: the Ling shape at T = 4 (the
per-phase kernels) and then at T = 1 (the one-launch step, a smaller input),
then the tiny shape (a change of stack shape, which clears the array), then
the Ling shape again."""

import ctypes

import numpy as np
import pytest
import torch

from weight_streaming_expert_amd import configs, inputs
import parity as P

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from weight_streaming_expert_amd import ops as _ops
    return _ops


def stack_and_head(ops, wl, L, head_wl):
    layers = [inputs.layer_weights(wl, l) for l in range(L)]
    st = lambda key: P.to_dev(np.stack([lw[key] for lw in layers]))
    r = np.stack([lw["router"] for lw in layers])
    router = P.to_dev(r) if r.dtype == np.float32 else P.to_dev_bf16(r)
    shared = tuple(P.to_dev(np.stack([lw["shared"][i] for lw in layers])) for i in range(4))
    stack = ops.MoeStackTensors(router, st("w13c"), st("w13s"), st("w2c"), st("w2s"), shared=shared, k=wl.moe.k)
    head = ops.Fp8LmHead.quantize(P.to_dev_bf16(inputs.head_weights(head_wl, K=wl.moe.H)))
    return stack, head


def outputs(stack, head, T):
    H, L, k = stack.H, stack.L, stack.k
    return dict(h=torch.empty((T, H), dtype=torch.bfloat16, device="cuda"),
                logits=torch.empty((T, head.V), dtype=torch.float32, device="cuda"),
                argmax=torch.empty((T,), dtype=torch.int32, device="cuda"),
                h_trace=torch.empty((L + 1, T, H), dtype=torch.bfloat16, device="cuda"),
                u_trace=torch.empty((L + 1, T, H), dtype=torch.bfloat16, device="cuda"),
                ids_trace=torch.empty((L, T, k), dtype=torch.int32, device="cuda"),
                w_trace=torch.empty((L, T, k), dtype=torch.float32, device="cuda"))


def call_noalloc(ops, x, stack, head, out):
    cs = stack.cstruct()
    ops._lib.call("moe_decode_step_noalloc", ops._p(x), x.shape[0], ctypes.byref(cs), ops._p(head.q),
                  ops._p(head.s), head.V, ops._p(out["h"]), ops._p(out["logits"]), ops._p(out["argmax"]),
                  ops._p(out["h_trace"]), ops._p(out["u_trace"]), ops._p(out["ids_trace"]),
                  ops._p(out["w_trace"]), ops._stream())


def test_noalloc_step_matches_the_allocating_step(ops):
    ling = stack_and_head(ops, configs.DECODE_STEP, 2, configs.LM_HEAD)
    tiny = stack_and_head(ops, configs.TINY, 3, configs.TINY)
    plan = [("ling", 4, 0), ("ling", 1, 1), ("tiny", 4, 2), ("tiny", 1, 3), ("ling", 1, 4)]
    for name, T, seed in plan:
        stack, head = ling if name == "ling" else tiny
        x = P.to_dev_bf16(inputs.normal_bf16((97, seed, T), (T, stack.H), 1.0))
        want = ops.moe_decode_step(x, stack, head, trace=True)
        got = outputs(stack, head, T)
        call_noalloc(ops, x, stack, head, got)
        torch.cuda.synchronize()
        assert int(want["argmax"].min()) >= 0
        for key in ("h", "logits", "argmax", "h_trace", "u_trace", "ids_trace", "w_trace"):
            assert torch.equal(got[key], want[key]), (name, T, key)
