"""C-ABI checks that need no GPU: the library loads, exports every function
include/wsx.h declares, and rejects bad arguments on the host before anything
is enqueued (no HIP call is reached on these paths)."""

import ctypes
import os
import re

import pytest

from weight_streaming_expert_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wsx.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="libwsx.so not built")

FAKE = 0x7F0000000000          # 256-byte aligned fake device address, never dereferenced on these paths
MIS = FAKE + 8                 # misaligned


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[\w]+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "for", "while", "sizeof")))


def test_header_functions_are_exported_and_declared():
    lib = _lib.load()
    names = header_functions()
    assert "moe_route_topk" in names and "moe_decode_step" in names and len(names) >= 11
    for n in names:
        assert hasattr(lib, n), n
        assert n in _lib.EXPORTS, n


def test_build_info_names_the_target():
    info = _lib.load().wsx_build_info().decode()
    assert "gfx950" in info and "lm_head" in info and "moe_gateup" in info


def test_status_strings():
    lib = _lib.load()
    for s in range(8):
        assert lib.wsx_status_string(s)


def route(x=FAKE, w=FAKE, dt=0, T=1, H=2560, E=512, k=8, ids=FAKE, tw=FAKE, el=FAKE, sw=FAKE, lo=None, ws=FAKE,
          wsb=1 << 20):
    return _lib.load().moe_route_topk(x, w, dt, T, H, E, k, ids, tw, el, sw, lo, ws, wsb, None)


def test_route_argument_errors():
    assert route(x=None) == 1
    assert route(ids=None) == 1
    assert route(dt=7) == 6
    assert route(T=0) == 2
    assert route(T=17) == 4                      # MoE layers take up to 16 tokens
    assert route(k=9) == 4
    assert route(k=0) == 2
    assert route(E=4, k=8) == 2
    assert route(E=2048) == 4
    assert route(H=100) == 2
    assert route(x=MIS) == 3
    assert route(ws=None) == 5
    assert route(wsb=16) == 5
    assert route(ws=FAKE + 16) == 3


def experts(x=FAKE, c13=FAKE, s13=FAKE, c2=FAKE, s2=FAKE, sh=(None, None, None, None), el=FAKE, sw=FAKE, T=1,
            H=2560, I=768, E=512, k=8, res=None, y=FAKE, h=None, ws=FAKE, wsb=1 << 24):
    return _lib.load().moe_expert_gemv_mxfp4(x, c13, s13, c2, s2, *sh, el, sw, T, H, I, E, k, res, y, h, ws, wsb, None)


def test_expert_argument_errors():
    assert experts(c13=None) == 1
    assert experts(el=None) == 1
    assert experts(sh=(FAKE, None, None, None)) == 1
    assert experts(h=FAKE, res=None) == 1
    assert experts(I=100) == 2
    assert experts(H=0) == 2
    assert experts(T=17) == 4
    assert experts(I=32 * 1000) == 4
    assert experts(c2=MIS) == 3
    assert experts(s13=MIS) == 3 and experts(s2=MIS) == 3
    assert experts(sh=(FAKE, MIS, FAKE, FAKE)) == 3
    assert experts(wsb=100) == 5
    lib = _lib.load()
    need = lib.wsx_moe_workspace_bytes(1, 2560, 768, 512, 8)
    assert need >= 9 * 768 * 4 and experts(wsb=need - 1) == 5


def test_head_argument_errors():
    lib = _lib.load()
    assert lib.lm_head_quantize_fp8(None, 10, 256, FAKE, FAKE, None) == 1
    assert lib.lm_head_quantize_fp8(FAKE, 0, 256, FAKE, FAKE, None) == 2
    assert lib.lm_head_quantize_fp8(FAKE, 10, 250, FAKE, FAKE, None) == 2
    assert lib.lm_head_quantize_fp8(FAKE, 10, 32768, FAKE, FAKE, None) == 4
    assert lib.lm_head_quantize_fp8(MIS, 10, 256, FAKE, FAKE, None) == 3
    f = lib.lm_head_gemv_fp8_argmax
    assert f(FAKE, None, 10, 256, FAKE, 1, None, FAKE, FAKE, 1 << 20, None) == 1
    assert f(FAKE, FAKE, 10, 256, FAKE, 0, None, FAKE, FAKE, 1 << 20, None) == 2
    assert f(FAKE, FAKE, 10, 256, FAKE, 5, None, FAKE, FAKE, 1 << 20, None) == 4
    assert f(FAKE, FAKE, 10, 256, FAKE, 1, None, FAKE, FAKE, 10, None) == 5
    assert f(FAKE, FAKE, 10, 256 * 100, FAKE, 1, None, FAKE, FAKE, 1 << 20, None) == 4
    g = lib.lm_head_gemv_bf16_argmax
    assert g(FAKE, 10, 256, None, 1, None, FAKE, FAKE, 1 << 20, None) == 1
    assert g(FAKE, 10, 256, FAKE, 1, None, FAKE, FAKE + 4, 1 << 20, None) == 3


def test_decode_step_argument_errors():
    lib = _lib.load()
    st = _lib.MoeStack(FAKE, 0, FAKE, FAKE, FAKE, FAKE, None, None, None, None, 2, 2560, 768, 512, 8)
    f = lib.moe_decode_step
    args = lambda **kw: [kw.get("h", FAKE), kw.get("T", 1), ctypes.byref(kw.get("st", st)), FAKE, FAKE,
                         kw.get("V", 157184), FAKE, None, FAKE, None, None, None, None, kw.get("ws", FAKE),
                         kw.get("wsb", 1 << 26), None]
    assert f(*args(h=None)) == 1
    assert f(*args(V=0)) == 2
    assert f(*args(T=6)) == 4
    assert f(*args(wsb=1000)) == 5
    bad = _lib.MoeStack(FAKE, 0, FAKE, FAKE, FAKE, FAKE, None, None, None, None, 0, 2560, 768, 512, 8)
    assert f(*args(st=bad)) == 2
    need = lib.wsx_decode_step_workspace_bytes(1, 2560, 768, 512, 8, 157184)
    assert need > lib.wsx_moe_workspace_bytes(1, 2560, 768, 512, 8)


def sample(lo=FAKE, V=157184, T=1, temp=0.6, k=29, p=0.95, u=FAKE, tok=FAKE, ws=FAKE, wsb=1 << 24):
    return _lib.load().lm_sample_topk_topp(lo, V, T, temp, k, p, u, tok, None, None, ws, wsb, None)


def test_sample_argument_errors():
    lib = _lib.load()
    assert sample(lo=None) == 1 and sample(u=None) == 1 and sample(tok=None) == 1
    assert sample(T=0) == 2 and sample(T=5) == 4
    assert sample(k=0) == 2 and sample(k=65) == 4 and sample(V=10, k=11) == 2
    assert sample(temp=0.0) == 2 and sample(temp=-1.0) == 2 and sample(temp=float("inf")) == 2
    assert sample(temp=float("nan")) == 2
    assert sample(p=0.0) == 2 and sample(p=1.5) == 2 and sample(p=float("nan")) == 2
    assert sample(V=8191 * 64 + 1) == 4 and sample(V=8191 * 64, k=64, wsb=0) == 5   # largest V passes the shape checks
    assert sample(ws=None) == 5 and sample(ws=MIS) == 3
    need = lib.wsx_sample_workspace_bytes(1, 157184, 29)
    assert need == 2456 * (29 + 1) * 8      # 64-logit chunks: k candidates and the maximum each
    assert sample(wsb=need - 1) == 5
    assert lib.wsx_sample_workspace_bytes(1, 10, 11) == 0
    head_need = lib.wsx_lm_head_sample_workspace_bytes(4, 157184, 2560, 29)
    assert head_need == lib.wsx_lm_head_workspace_bytes(4, 157184, 2560) + 256 + 4 * 2456 * 30 * 8
    # one row: room for the one-launch form's published maxima as well (up to 512 workgroups: 16 chunk
    # maxima and the workgroup's maximum each)
    head = lib.wsx_lm_head_workspace_bytes(1, 157184, 2560) + 256
    assert lib.wsx_lm_head_sample_workspace_bytes(1, 157184, 2560, 29) == head + 2456 * 30 * 8
    assert lib.wsx_lm_head_sample_workspace_bytes(1, 1000, 2560, 29) == head + 512 * 17 * 8
    assert lib.wsx_lm_head_sample_path(2, 157184, 2560, 29) == 0
    assert lib.wsx_lm_head_sample_path(5, 157184, 2560, 29) == -1
    assert lib.wsx_lm_head_sample_path(1, 157184, 2560, 65) == -1
    assert lib.wsx_lm_head_sample_path(1, 157184, 100, 29) == -1
    f = lib.lm_head_gemv_fp8_sample
    assert f(None, FAKE, 157184, 2560, FAKE, 1, 0.6, 29, 0.95, FAKE, FAKE, FAKE, None, None, FAKE, head_need, None) == 1
    assert f(FAKE, FAKE, 157184, 2560, FAKE, 1, 0.6, 29, 0.95, FAKE, None, FAKE, None, None, FAKE, head_need, None) == 1
    assert f(FAKE, FAKE, 157184, 100, FAKE, 1, 0.6, 29, 0.95, FAKE, FAKE, FAKE, None, None, FAKE, head_need, None) == 2
    assert f(FAKE, FAKE, 157184, 2560, FAKE, 1, 0.6, 29, 0.95, FAKE, FAKE, FAKE, None, None, FAKE, 1000, None) == 5


def test_noalloc_decode_step_rejects_on_the_host():
    """The allocation-free step checks everything on the host first: a shape
    whose workspace exceeds the device array is refused, and so are the
    allocating step's argument errors, before the device is touched."""
    lib = _lib.load()
    f = lib.moe_decode_step_noalloc
    big = _lib.MoeStack(FAKE, 0, FAKE, FAKE, FAKE, FAKE, None, None, None, None, 2, 8192, 2048, 1024, 8)
    st = _lib.MoeStack(FAKE, 0, FAKE, FAKE, FAKE, FAKE, None, None, None, None, 2, 2560, 768, 512, 8)
    args = lambda **kw: [kw.get("h", FAKE), kw.get("T", 1), ctypes.byref(kw.get("st", st)), FAKE, FAKE,
                         kw.get("V", 157184), FAKE, None, FAKE, None, None, None, None, None]
    assert lib.wsx_decode_step_workspace_bytes(4, 8192, 2048, 1024, 8, 157184) > (2 << 20)
    assert f(*args(st=big, T=4)) == 5
    assert f(*args(h=None)) == 1
    assert f(*args(T=6)) == 4
    assert f(*args(V=0)) == 2
    assert f(FAKE, 1, None, FAKE, FAKE, 157184, FAKE, None, FAKE, None, None, None, None, None) == 1


def test_w4a8_argument_errors():
    lib = _lib.load()
    q = lib.act_quantize_mxfp8
    assert q(None, 1, 64, FAKE, FAKE, None) == 1
    assert q(FAKE, 0, 64, FAKE, FAKE, None) == 2
    assert q(FAKE, 1, 48, FAKE, FAKE, None) == 2
    assert q(MIS, 1, 64, FAKE, FAKE, None) == 3
    f = lib.moe_expert_gemv_w4a8
    args = lambda **kw: [kw.get("x", FAKE), FAKE, FAKE, FAKE, FAKE, None, None, None, None, FAKE, FAKE,
                         kw.get("T", 1), kw.get("H", 2560), kw.get("I", 768), 512, 8, None, FAKE, None,
                         kw.get("act", None), kw.get("ws", FAKE), kw.get("wsb", 1 << 26), None]
    assert f(*args(x=None)) == 1
    assert f(*args(H=4096)) == 4                 # beyond the W4A8 kernels' 2560
    assert f(*args(T=17)) == 4
    assert f(*args(act=MIS)) == 3
    assert f(*args(wsb=100)) == 5


def test_decode_step_path_query():
    """Which path a stack shape takes: the two shapes compiled ahead of time,
    run-time compiled shapes inside the one-launch layout, per-phase otherwise."""
    q = _lib.load().wsx_decode_step_path
    assert q(1, 0, 1, 2560, 768, 512, 8) == 1            # Ling shape, bf16 router
    assert q(1, 1, 1, 256, 64, 16, 2) == 1               # tiny shape, fp32 router
    assert q(1, 0, 1, 512, 128, 64, 4) == 2              # compiled at run time
    assert q(1, 1, 1, 384, 96, 40, 3) == 2
    assert q(1, 0, 1, 256, 64, 16, 2) == 2               # the tiny shape with a bf16 router
    assert q(4, 0, 1, 2560, 768, 512, 8) == 0            # several tokens: per-phase
    assert q(1, 0, 0, 2560, 768, 512, 8) == 0            # no shared expert
    assert q(1, 0, 1, 2560, 768, 1024, 8) == 0           # more experts than one routing workgroup ranks
    assert q(1, 0, 1, 8192, 768, 512, 8) == 0            # beyond the kernel's register arrays
    assert q(1, 7, 1, 2560, 768, 512, 8) == 0
