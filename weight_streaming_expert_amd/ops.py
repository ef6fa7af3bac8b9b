"""Thin Python binding of libwsx.so over torch device tensors.

Argument marshalling only: each function checks dtypes/devices, allocates the
outputs as torch tensors and calls the C entry point of the same name on
torch's current stream.  Every step of the computation runs in the HIP
kernels.  Importing this module loads the library and raises if it is absent.
"""

import ctypes

import numpy as np
import torch

from . import _lib
from ._lib import DTYPE_BF16, DTYPE_F32, MoeStack, WsxError  # noqa: F401

_lib.load()

MAX_T, MAX_K, MAX_E = 4, 8, 1024


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev=None):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _chk(t, dtype, name):
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise TypeError(f"{name}: expected a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous tensor")


def bf16_from_bits(bits, device):
    """numpy uint16 bf16 bit patterns -> device torch.bfloat16 tensor."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def bits_from_bf16(t):
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def workspace(nbytes, device):
    """Zero-filled device workspace (the C ABI requires zeros before first use)."""
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def moe_workspace_bytes(T, H, I, E, k):
    return int(_lib.load().wsx_moe_workspace_bytes(T, H, I, E, k))


def lm_head_workspace_bytes(T, V, K):
    return int(_lib.load().wsx_lm_head_workspace_bytes(T, V, K))


def decode_step_workspace_bytes(T, H, I, E, k, V):
    return int(_lib.load().wsx_decode_step_workspace_bytes(T, H, I, E, k, V))


def decode_step_path(T, stack):
    """0: per-phase launches, 1: one launch compiled ahead of time, 2: one launch
    compiled at run time (hipRTC) for this stack's shape."""
    dt = DTYPE_F32 if stack.w_router.dtype == torch.float32 else DTYPE_BF16
    return int(_lib.load().wsx_decode_step_path(T, dt, int(stack.shared is not None), stack.H, stack.I, stack.E,
                                                stack.k))


def build_info():
    return _lib.load().wsx_build_info().decode()


# ----------------------------------------------------------------------------- MoE


def moe_route_topk(x, w_router, k, ws=None, want_logits=True):
    """Router + top-k.  x: bf16 [T][H]; w_router: bf16 or float32 [E][H].
    Returns dict(topk_ids, topk_w, expert_list, slot_w, logits)."""
    _chk(x, torch.bfloat16, "x")
    T, H = x.shape
    E = w_router.shape[0]
    if w_router.dtype == torch.bfloat16:
        dt = DTYPE_BF16
    elif w_router.dtype == torch.float32:
        dt = DTYPE_F32
    else:
        raise TypeError("w_router must be bfloat16 or float32")
    _chk(w_router, w_router.dtype, "w_router")
    dev = x.device
    out = dict(topk_ids=torch.empty((T, k), dtype=torch.int32, device=dev),
               topk_w=torch.empty((T, k), dtype=torch.float32, device=dev),
               expert_list=torch.empty((1 + T * k,), dtype=torch.int32, device=dev),
               slot_w=torch.empty((T * k, T), dtype=torch.float32, device=dev),
               logits=torch.empty((T, E), dtype=torch.float32, device=dev) if want_logits else None)
    if ws is None:
        ws = workspace(moe_workspace_bytes(T, H, 0, E, k), dev)
    _lib.call("moe_route_topk", _p(x), _p(w_router), dt, T, H, E, k,
              _p(out["topk_ids"]), _p(out["topk_w"]), _p(out["expert_list"]), _p(out["slot_w"]),
              _p(out["logits"]), _p(ws), ws.numel(), _stream(dev))
    return out


def moe_expert_gemv_mxfp4(x, w13_codes, w13_scales, w2_codes, w2_scales, expert_list, slot_w, k,
                          shared=None, residual=None, want_y=True, want_h=True, ws=None):
    """Routed + shared SwiGLU experts.  Weights uint8 as in include/wsx.h,
    shared = (sh13_codes, sh13_scales, sh2_codes, sh2_scales) or None.
    Returns (y float32 [T][H] or None, h bf16 [T][H] or None)."""
    _chk(x, torch.bfloat16, "x")
    T, H = x.shape
    E = w13_codes.shape[0]
    I = w13_codes.shape[1] // 2
    for name, t in (("w13_codes", w13_codes), ("w13_scales", w13_scales), ("w2_codes", w2_codes), ("w2_scales", w2_scales)):
        _chk(t, torch.uint8, name)
    _chk(expert_list, torch.int32, "expert_list")
    _chk(slot_w, torch.float32, "slot_w")
    sh = [None] * 4 if shared is None else list(shared)
    dev = x.device
    y = torch.empty((T, H), dtype=torch.float32, device=dev) if want_y else None
    h = torch.empty((T, H), dtype=torch.bfloat16, device=dev) if (want_h and residual is not None) else None
    if ws is None:
        ws = workspace(moe_workspace_bytes(T, H, I, E, k), dev)
    _lib.call("moe_expert_gemv_mxfp4", _p(x), _p(w13_codes), _p(w13_scales), _p(w2_codes), _p(w2_scales),
              *[_p(t) for t in sh], _p(expert_list), _p(slot_w), T, H, I, E, k,
              _p(residual), _p(y), _p(h), _p(ws), ws.numel(), _stream(dev))
    return y, h


def act_quantize_mxfp8(x):
    """bf16 [T][K] -> (E4M3 codes uint8 [T][K], E8M0 scale bytes uint8 [T][K/32])."""
    _chk(x, torch.bfloat16, "x")
    T, K = x.shape
    codes = torch.empty((T, K), dtype=torch.uint8, device=x.device)
    scales = torch.empty((T, K // 32), dtype=torch.uint8, device=x.device)
    _lib.call("act_quantize_mxfp8", _p(x), T, K, _p(codes), _p(scales), _stream(x.device))
    return codes, scales


def moe_expert_gemv_w4a8(x, w13_codes, w13_scales, w2_codes, w2_scales, expert_list, slot_w, k,
                         shared=None, residual=None, want_y=True, want_h=True, want_act=False, ws=None):
    """W4A8 routed + shared SwiGLU experts (MXFP8 activations).  Returns
    (y float32 [T][H] or None, h bf16 [T][H] or None, act float32 [T*k+1][T][I] or None)."""
    _chk(x, torch.bfloat16, "x")
    T, H = x.shape
    E = w13_codes.shape[0]
    I = w13_codes.shape[1] // 2
    for name, t in (("w13_codes", w13_codes), ("w13_scales", w13_scales), ("w2_codes", w2_codes), ("w2_scales", w2_scales)):
        _chk(t, torch.uint8, name)
    _chk(expert_list, torch.int32, "expert_list")
    _chk(slot_w, torch.float32, "slot_w")
    sh = [None] * 4 if shared is None else list(shared)
    dev = x.device
    y = torch.empty((T, H), dtype=torch.float32, device=dev) if want_y else None
    h = torch.empty((T, H), dtype=torch.bfloat16, device=dev) if (want_h and residual is not None) else None
    act = torch.zeros((T * k + 1, T, I), dtype=torch.float32, device=dev) if want_act else None
    if ws is None:
        ws = workspace(moe_workspace_bytes(T, H, I, E, k), dev)
    _lib.call("moe_expert_gemv_w4a8", _p(x), _p(w13_codes), _p(w13_scales), _p(w2_codes), _p(w2_scales),
              *[_p(t) for t in sh], _p(expert_list), _p(slot_w), T, H, I, E, k,
              _p(residual), _p(y), _p(h), _p(act), _p(ws), ws.numel(), _stream(dev))
    return y, h, act


# ----------------------------------------------------------------------------- LM head


def lm_head_quantize_fp8(w):
    """BF16 [V][K] -> (codes uint8 [V][K], row scales float32 [V])."""
    _chk(w, torch.bfloat16, "w")
    V, K = w.shape
    q = torch.empty((V, K), dtype=torch.uint8, device=w.device)
    s = torch.empty((V,), dtype=torch.float32, device=w.device)
    _lib.call("lm_head_quantize_fp8", _p(w), V, K, _p(q), _p(s), _stream(w.device))
    return q, s


def lm_head_gemv_fp8_argmax(q, row_scale, x, want_logits=True, ws=None):
    _chk(q, torch.uint8, "q")
    _chk(row_scale, torch.float32, "row_scale")
    _chk(x, torch.bfloat16, "x")
    V, K = q.shape
    T = x.shape[0]
    dev = x.device
    logits = torch.empty((T, V), dtype=torch.float32, device=dev) if want_logits else None
    am = torch.empty((T,), dtype=torch.int32, device=dev)
    if ws is None:
        ws = workspace(lm_head_workspace_bytes(T, V, K), dev)
    _lib.call("lm_head_gemv_fp8_argmax", _p(q), _p(row_scale), V, K, _p(x), T, _p(logits), _p(am),
              _p(ws), ws.numel(), _stream(dev))
    return logits, am


def lm_head_gemv_bf16_argmax(w, x, want_logits=True, ws=None):
    _chk(w, torch.bfloat16, "w")
    _chk(x, torch.bfloat16, "x")
    V, K = w.shape
    T = x.shape[0]
    dev = x.device
    logits = torch.empty((T, V), dtype=torch.float32, device=dev) if want_logits else None
    am = torch.empty((T,), dtype=torch.int32, device=dev)
    if ws is None:
        ws = workspace(lm_head_workspace_bytes(T, V, K), dev)
    _lib.call("lm_head_gemv_bf16_argmax", _p(w), V, K, _p(x), T, _p(logits), _p(am), _p(ws), ws.numel(), _stream(dev))
    return logits, am


def _sample_args(T, k, uniforms, dev):
    _chk(uniforms, torch.float32, "uniforms")
    if uniforms.numel() != T:
        raise ValueError("uniforms must hold one value per row")
    tok = torch.empty((T,), dtype=torch.int32, device=dev)
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    probs = torch.empty((T, k), dtype=torch.float32, device=dev)
    return tok, ids, probs


def lm_sample_topk_topp(logits, temperature, top_k, top_p, uniforms, ws=None):
    """One token per row of logits float32 [T][V]: temperature, top-k, top-p,
    inverse-CDF draw with uniforms float32 [T].  Returns (token int32 [T],
    ranked top-k ids int32 [T][k], kept probabilities float32 [T][k])."""
    _chk(logits, torch.float32, "logits")
    T, V = logits.shape
    dev = logits.device
    tok, ids, probs = _sample_args(T, top_k, uniforms, dev)
    if ws is None:
        ws = workspace(max(int(_lib.load().wsx_sample_workspace_bytes(T, V, top_k)), 256), dev)
    _lib.call("lm_sample_topk_topp", _p(logits), V, T, float(temperature), int(top_k), float(top_p), _p(uniforms),
              _p(tok), _p(ids), _p(probs), _p(ws), ws.numel(), _stream(dev))
    return tok, ids, probs


def lm_head_sample_path(T, V, K, top_k):
    """1: lm_head_gemv_fp8_sample is one launch (the sampler in the head's
    tail) on the current device; 0: three launches; -1: unsupported sizes."""
    return int(_lib.load().wsx_lm_head_sample_path(T, V, K, top_k))


def lm_head_gemv_fp8_sample(q, row_scale, x, temperature, top_k, top_p, uniforms, ws=None):
    """FP8 head with the sampler on its logits (fused into the head's tail for
    one token where lm_head_sample_path says so).  Returns (logits, token, ids,
    probs)."""
    _chk(q, torch.uint8, "q")
    _chk(row_scale, torch.float32, "row_scale")
    _chk(x, torch.bfloat16, "x")
    V, K = q.shape
    T = x.shape[0]
    dev = x.device
    logits = torch.empty((T, V), dtype=torch.float32, device=dev)
    tok, ids, probs = _sample_args(T, top_k, uniforms, dev)
    if ws is None:
        ws = workspace(max(int(_lib.load().wsx_lm_head_sample_workspace_bytes(T, V, K, top_k)), 256), dev)
    _lib.call("lm_head_gemv_fp8_sample", _p(q), _p(row_scale), V, K, _p(x), T, float(temperature), int(top_k),
              float(top_p), _p(uniforms), _p(logits), _p(tok), _p(ids), _p(probs), _p(ws), ws.numel(), _stream(dev))
    return logits, tok, ids, probs


class Fp8LmHead:
    """The FP8 head as one object: codes, row scales and shape travel together,
    so FP8 bytes can only ever reach the FP8 GEMV entry point."""

    def __init__(self, q, s):
        _chk(q, torch.uint8, "q")
        _chk(s, torch.float32, "s")
        self.q, self.s = q, s
        self.V, self.K = q.shape

    @classmethod
    def quantize(cls, w_bf16):
        return cls(*lm_head_quantize_fp8(w_bf16))

    def gemv_argmax(self, x, want_logits=True, ws=None):
        return lm_head_gemv_fp8_argmax(self.q, self.s, x, want_logits, ws)


# ----------------------------------------------------------------------------- decode step


class MoeStackTensors:
    """Device tensors of L stacked MoE layers (leading [L] axis on each)."""

    def __init__(self, w_router, w13_codes, w13_scales, w2_codes, w2_scales, shared=None, k=8):
        self.w_router, self.w13_codes, self.w13_scales = w_router, w13_codes, w13_scales
        self.w2_codes, self.w2_scales = w2_codes, w2_scales
        self.shared = shared
        self.L, self.E = w_router.shape[0], w_router.shape[1]
        self.H = w_router.shape[2]
        self.I = w13_codes.shape[2] // 2
        self.k = k

    def cstruct(self):
        sh = [None] * 4 if self.shared is None else list(self.shared)
        dt = DTYPE_F32 if self.w_router.dtype == torch.float32 else DTYPE_BF16
        return MoeStack(self.w_router.data_ptr(), dt, self.w13_codes.data_ptr(), self.w13_scales.data_ptr(),
                        self.w2_codes.data_ptr(), self.w2_scales.data_ptr(),
                        *[None if t is None else t.data_ptr() for t in sh],
                        self.L, self.H, self.I, self.E, self.k)


def moe_decode_step(h_in, stack, head, want_logits=True, trace=False, ws=None, out=None):
    """One pass through the stacked MoE layers and the FP8 head.
    Returns dict(h, logits, argmax[, h_trace, u_trace, ids_trace, w_trace])."""
    _chk(h_in, torch.bfloat16, "h_in")
    T, H = h_in.shape
    dev = h_in.device
    L, k = stack.L, stack.k
    if out is None:
        out = dict(h=torch.empty((T, H), dtype=torch.bfloat16, device=dev),
                   logits=torch.empty((T, head.V), dtype=torch.float32, device=dev) if want_logits else None,
                   argmax=torch.empty((T,), dtype=torch.int32, device=dev))
        if trace:
            out.update(h_trace=torch.empty((L + 1, T, H), dtype=torch.bfloat16, device=dev),
                       u_trace=torch.empty((L + 1, T, H), dtype=torch.bfloat16, device=dev),
                       ids_trace=torch.empty((L, T, k), dtype=torch.int32, device=dev),
                       w_trace=torch.empty((L, T, k), dtype=torch.float32, device=dev))
    if ws is None:
        ws = workspace(decode_step_workspace_bytes(T, H, stack.I, stack.E, k, head.V), dev)
    cs = stack.cstruct()
    _lib.call("moe_decode_step", _p(h_in), T, ctypes.byref(cs), _p(head.q), _p(head.s), head.V,
              _p(out["h"]), _p(out.get("logits")), _p(out["argmax"]),
              _p(out.get("h_trace")), _p(out.get("u_trace")), _p(out.get("ids_trace")), _p(out.get("w_trace")),
              _p(ws), ws.numel(), _stream(dev))
    return out
