"""ctypes declarations of libwsx.so (the C ABI in include/wsx.h).

Loading fails loudly if the library has not been built: there is no fallback
path.  Build it with `python -m weight_streaming_expert_amd.build`.
"""

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libwsx.so")

c_void_p, c_int, c_size_t, c_char_p, c_float = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_char_p, ctypes.c_float

STATUS = {0: "WSX_OK", 1: "WSX_ERR_NULL", 2: "WSX_ERR_SHAPE", 3: "WSX_ERR_ALIGN", 4: "WSX_ERR_UNSUPPORTED",
          5: "WSX_ERR_WORKSPACE", 6: "WSX_ERR_DTYPE", 7: "WSX_ERR_HIP"}
DTYPE_BF16, DTYPE_F32 = 0, 1


class WsxError(RuntimeError):
    def __init__(self, fn, status, text):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} ({text})")
        self.status = status


class MoeStack(ctypes.Structure):
    _fields_ = [("w_router", c_void_p), ("router_dtype", c_int),
                ("w13_codes", c_void_p), ("w13_scales", c_void_p),
                ("w2_codes", c_void_p), ("w2_scales", c_void_p),
                ("sh13_codes", c_void_p), ("sh13_scales", c_void_p),
                ("sh2_codes", c_void_p), ("sh2_scales", c_void_p),
                ("L", c_int), ("H", c_int), ("I", c_int), ("E", c_int), ("k", c_int)]


# name -> argtypes (every entry point returns wsx_status as int unless listed in _RESTYPES)
_PROTOS = {
    "moe_route_topk": [c_void_p, c_void_p, c_int, c_int, c_int, c_int, c_int,
                       c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p],
    "moe_expert_gemv_mxfp4": [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                              c_void_p, c_void_p, c_int, c_int, c_int, c_int, c_int,
                              c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p],
    "act_quantize_mxfp8": [c_void_p, c_int, c_int, c_void_p, c_void_p, c_void_p],
    "moe_expert_gemv_w4a8": [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                             c_void_p, c_void_p, c_int, c_int, c_int, c_int, c_int,
                             c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p],
    "lm_head_quantize_fp8": [c_void_p, c_int, c_int, c_void_p, c_void_p, c_void_p],
    "lm_head_gemv_fp8_argmax": [c_void_p, c_void_p, c_int, c_int, c_void_p, c_int, c_void_p, c_void_p,
                                c_void_p, c_size_t, c_void_p],
    "lm_head_gemv_bf16_argmax": [c_void_p, c_int, c_int, c_void_p, c_int, c_void_p, c_void_p,
                                 c_void_p, c_size_t, c_void_p],
    "lm_sample_topk_topp": [c_void_p, c_int, c_int, c_float, c_int, c_float, c_void_p, c_void_p, c_void_p, c_void_p,
                            c_void_p, c_size_t, c_void_p],
    "lm_head_gemv_fp8_sample": [c_void_p, c_void_p, c_int, c_int, c_void_p, c_int, c_float, c_int, c_float, c_void_p,
                                c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p],
    "moe_decode_step": [c_void_p, c_int, ctypes.POINTER(MoeStack), c_void_p, c_void_p, c_int,
                        c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                        c_void_p, c_size_t, c_void_p],
    "moe_decode_step_noalloc": [c_void_p, c_int, ctypes.POINTER(MoeStack), c_void_p, c_void_p, c_int,
                                c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p],
    "wsx_read_probe": [c_void_p, c_size_t, c_void_p, c_void_p],
    "wsx_decode_step_path": [c_int, c_int, c_int, c_int, c_int, c_int, c_int],
    "wsx_moe_workspace_bytes": [c_int, c_int, c_int, c_int, c_int],
    "wsx_lm_head_workspace_bytes": [c_int, c_int, c_int],
    "wsx_decode_step_workspace_bytes": [c_int, c_int, c_int, c_int, c_int, c_int],
    "wsx_sample_workspace_bytes": [c_int, c_int, c_int],
    "wsx_lm_head_sample_workspace_bytes": [c_int, c_int, c_int, c_int],
    "wsx_lm_head_sample_path": [c_int, c_int, c_int, c_int],
    "wsx_status_string": [c_int],
    "wsx_build_info": [],
}
_RESTYPES = {"wsx_moe_workspace_bytes": c_size_t, "wsx_lm_head_workspace_bytes": c_size_t,
             "wsx_decode_step_workspace_bytes": c_size_t, "wsx_sample_workspace_bytes": c_size_t,
             "wsx_lm_head_sample_workspace_bytes": c_size_t, "wsx_status_string": c_char_p,
             "wsx_build_info": c_char_p, "wsx_decode_step_path": c_int, "wsx_lm_head_sample_path": c_int}
EXPORTS = tuple(_PROTOS)

_lib = None


def load():
    """Load libwsx.so and declare its prototypes (cached)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m weight_streaming_expert_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    for name, argtypes in _PROTOS.items():
        fn = getattr(lib, name)
        fn.argtypes = argtypes
        fn.restype = _RESTYPES.get(name, c_int)
    _lib = lib
    return lib


def call(name, *args):
    """Call a status-returning entry point; raise WsxError on any non-OK status."""
    lib = load()
    st = getattr(lib, name)(*args)
    if st != 0:
        raise WsxError(name, st, lib.wsx_status_string(st).decode())
    return st
