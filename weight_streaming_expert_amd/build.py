"""Build libwsx.so for gfx950 with hipcc, in-tree (next to this file).

    python -m weight_streaming_expert_amd.build [--jobs N]

Every HIP source is compiled for gfx950 only.  Packed fp32 VALU instructions
are disabled for all device code; IEEE-correct fp32 division and square root
(hipcc's default) are kept because the FP8 head scale is defined by them.
"""

import argparse
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libwsx.so")
BUILD = os.path.join(HERE, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["gemv_rows.hip", "moe_experts.hip", "moe_w4a8.hip", "lm_head_quant.hip", "decode_step.hip", "sample.hip", "probe.hip", "api.cpp"]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-x", "hip",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable", "-Wno-unused-but-set-variable",
    "-I", os.path.join(ROOT, "include"),
]

# The one-launch decode step is also compiled at run time (hipRTC) for shapes
# not built here: its kernel header and the headers it includes travel inside
# the library as text.  hipRTC supplies no standard headers, so those names get
# stand-ins (the fixed-width integer types live in hipRTC's own namespace).
RTC_HEADERS = [("decode_step_kernel.h", "csrc/decode_step_kernel.h"), ("wsx_device.h", "csrc/wsx_device.h"),
               ("../../include/wsx.h", "../include/wsx.h")]
RTC_STANDINS = [
    ("hip/hip_runtime.h", "#pragma once\n"),
    ("stddef.h", "#pragma once\n"),
    ("stdint.h", "#pragma once\nusing __hip_internal::int8_t; using __hip_internal::uint8_t;\n"
                 "using __hip_internal::int16_t; using __hip_internal::uint16_t;\n"
                 "using __hip_internal::int32_t; using __hip_internal::uint32_t;\n"
                 "using __hip_internal::int64_t; using __hip_internal::uint64_t;\n"),
]


def write_rtc_sources(path):
    """rtc_sources.inc: kRtcHeaders[] = {name, text} for hipRTC."""
    parts = []
    for name, rel in RTC_HEADERS:
        text = open(os.path.join(HERE, rel)).read()
        assert ")WSXRTC" not in text
        parts.append(f'  {{"{name}", R"WSXRTC({text})WSXRTC"}},')
    for name, text in RTC_STANDINS:
        parts.append(f'  {{"{name}", R"WSXRTC({text})WSXRTC"}},')
    body = "\n".join(parts)
    out = ("// Written by build.py: the one-launch step's kernel header and its includes, for hipRTC.\n"
           "struct RtcHeader { const char* name; const char* text; };\n"
           f"static const RtcHeader kRtcHeaders[] = {{\n{body}\n}};\n"
           "static const int kRtcNumHeaders = (int)(sizeof(kRtcHeaders) / sizeof(kRtcHeaders[0]));\n")
    tmp = path + ".tmp"
    with open(tmp, "w") as f:
        f.write(out)
    os.replace(tmp, path)


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-I", CSRC, "-I", BUILD, "-c", os.path.join(CSRC, src), "-o", obj]
    p = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 target feature; that warning is harmless
    err = "\n".join(l for l in p.stderr.splitlines() if "packed-fp32-ops" not in l and "is not a recognized feature" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(jobs=None, verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    write_rtc_sources(os.path.join(BUILD, "rtc_sources.inc"))
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1)
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp, "-L/opt/rocm/lib", "-lhiprtc"]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError("link failed:\n" + p.stderr)
    os.replace(tmp, OUT)
    if verbose:
        print("built", OUT)
    return OUT


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    a = ap.parse_args()
    build(a.jobs, verbose=True)
