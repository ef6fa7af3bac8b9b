// One decode step (T = 1) of the stacked MoE layers plus the FP8 LM head in a
// single launch: host side.  The kernel is in decode_step_kernel.h; it is
// instantiated here for the shapes compiled ahead of time, and compiled at run
// time through hipRTC for any other shape the kernel's layout supports.
#include "decode_step_kernel.h"
#include "wsx_internal.h"

#include <hip/hiprtc.h>

#include <mutex>
#include <string>
#include <vector>

// kRtcHeaders: the kernel header and the headers it includes, as text (written
// by the build next to the objects), with stand-ins for the standard headers,
// which hipRTC does not provide.
#include "rtc_sources.inc"

namespace wsx {

// ---------------------------------------------------------------- host side

namespace {

struct Shape {
  int NJ, NJD, RJ, HJ, QPT, QA;
};

Shape fused_shape(int H, int I, int router_bytes) {
  Shape s;
  s.NJ = (H / 32 + 15) / 16;
  s.NJD = (I / 32 + 7) / 8;
  s.RJ = (H * router_bytes / 16 + 31) / 32;
  s.HJ = (H / 16 + 15) / 16;
  s.QPT = (H / 4 + NT - 1) / NT;
  s.QA = (I / 2 + 63) / 64;
  return s;
}

bool is_ling(const Shape& s) {
  return s.NJ == 5 && s.NJD == 3 && s.RJ == 10 && s.HJ == 10 && s.QPT == 3 && s.QA == 6;
}
bool is_tiny(const Shape& s) {
  return s.NJ == 1 && s.NJD == 1 && s.RJ == 2 && s.HJ == 1 && s.QPT == 1 && s.QA == 1;
}

inline size_t al(size_t n) { return (n + 255) & ~(size_t)255; }

struct FusedLayout {
  size_t ctl, hx, lg, a, total;
  int n_head;
};

int fused_head_blocks(int V) {
  const int NG = (V + 3) / 4;
  const int n = (NG + 4 * 8 - 1) / (4 * 8);   // about 8 row groups per wavefront
  return n < 1 ? 1 : (n > 1024 ? 1024 : n);
}

FusedLayout fused_layout(int H, int I, int E, int k, int V) {
  FusedLayout f;
  const int nslot = k + 1;
  f.n_head = fused_head_blocks(V);
  f.ctl = 0;
  f.hx = al(f.ctl + sizeof(Ctl));
  f.lg = al(f.hx + (size_t)kCopiesH * 2 * (H / 2) * 8);
  f.a = al(f.lg + (size_t)kCopiesLg * E * 8);
  f.total = al(f.a + (size_t)kCopiesA * nslot * I * 8);
  return f;
}

size_t fused_lds_bytes(int H, int I, int k) {
  size_t m = (size_t)(k + 1) * (I / 32) * 144;   // expert activations, 144-byte blocks
  const size_t u[3] = {(size_t)LayPlain::bytes(H), (size_t)LayMX::bytes(H), (size_t)LayHead::bytes(H)};
  for (size_t v : u) m = v > m ? v : m;
  return m;
}

// ---------------------------------------------------------------- run-time specialization

// [saipien] "Kernels built for the shape you actually have": the pages' MoE
// kernels are compiled at run time for the model's shapes.  Here the one-launch
// step is compiled ahead of time for the Ling shape (bf16 router) and the tiny
// shape (fp32 router); any other shape its layout supports is compiled on
// first use with hipRTC from the same kernel text, once per (device, shape),
// and kept for the life of the process.

bool same_shape(const Shape& a, const Shape& b) {
  return a.NJ == b.NJ && a.NJD == b.NJD && a.RJ == b.RJ && a.HJ == b.HJ && a.QPT == b.QPT && a.QA == b.QA;
}

struct RtcKernel {
  int dev, rb;
  Shape s;
  hipModule_t mod;
  hipFunction_t fn;
};
std::mutex g_rtc_mu;
std::vector<RtcKernel> g_rtc;

// Compiles (or finds) decode_step_kernel<s..., rb> for the current device.
hipError_t rtc_kernel(const Shape& s, int rb, hipFunction_t* fn) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(g_rtc_mu);
  for (const RtcKernel& r : g_rtc)
    if (r.dev == dev && r.rb == rb && same_shape(r.s, s)) {
      *fn = r.fn;
      return hipSuccess;
    }
  const std::string inst = "wsx::decode_step_kernel<" + std::to_string(s.NJ) + ", " + std::to_string(s.NJD) + ", " +
                           std::to_string(s.RJ) + ", " + std::to_string(s.HJ) + ", " + std::to_string(s.QPT) + ", " +
                           std::to_string(s.QA) + ", " + std::to_string(rb) + ">";
  const std::string src = "#include \"decode_step_kernel.h\"\ntemplate __global__ void " + inst + "(wsx::FusedStepArgs);\n";
  const char* texts[kRtcNumHeaders];
  const char* names[kRtcNumHeaders];
  for (int i = 0; i < kRtcNumHeaders; ++i) {
    names[i] = kRtcHeaders[i].name;
    texts[i] = kRtcHeaders[i].text;
  }
  hiprtcProgram prog;
  if (hiprtcCreateProgram(&prog, src.c_str(), "decode_step_rtc.hip", kRtcNumHeaders, texts, names) != HIPRTC_SUCCESS)
    return hipErrorInvalidValue;
  // the same code generation as the ahead-of-time build (no packed fp32)
  const char* opts[] = {"--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
                        "-packed-fp32-ops"};
  std::string lowered;
  std::vector<char> code;
  bool ok = hiprtcAddNameExpression(prog, inst.c_str()) == HIPRTC_SUCCESS &&
            hiprtcCompileProgram(prog, (int)(sizeof(opts) / sizeof(opts[0])), opts) == HIPRTC_SUCCESS;
  if (ok) {
    const char* ln = nullptr;
    size_t n = 0;
    ok = hiprtcGetLoweredName(prog, inst.c_str(), &ln) == HIPRTC_SUCCESS && ln && hiprtcGetCodeSize(prog, &n) == HIPRTC_SUCCESS && n > 0;
    if (ok) {
      lowered = ln;
      code.resize(n);
      ok = hiprtcGetCode(prog, code.data()) == HIPRTC_SUCCESS;
    }
  }
  hiprtcDestroyProgram(&prog);
  if (!ok) return hipErrorInvalidValue;
  RtcKernel r;
  r.dev = dev;
  r.rb = rb;
  r.s = s;
  if ((e = hipModuleLoadData(&r.mod, code.data())) != hipSuccess) return e;
  if ((e = hipModuleGetFunction(&r.fn, r.mod, lowered.c_str())) != hipSuccess) return e;
  g_rtc.push_back(r);
  *fn = r.fn;
  return hipSuccess;
}

// Shapes the kernel's layout supports: the routing ranks at most 2 NT logits,
// tiles of 8 router rows, 16 intermediate values and 8 output rows, MX blocks
// of 32, and bounded per-lane register arrays (H <= 4096, I <= 2048; the
// down stage keeps 2 QA <= 32 chunk bits per lane).
bool layout_supported(int H, int I, int E, int k, int rb) {
  if (E % kRRows || E > 2 * NT || I % kGRows || H % kDRows || H % 32 || I % 32 || k < 1 || k > WSX_MAX_K || k > E)
    return false;
  const Shape s = fused_shape(H, I, rb);
  if (s.NJ > 8 || s.NJD > 8 || s.RJ > 32 || s.HJ > 16 || s.QPT > 8 || s.QA > 16) return false;
  return fused_lds_bytes(H, I, k) <= 64 * 1024;
}

int fused_path(int T, int router_dtype, bool has_shared, int H, int I, int E, int k) {
  if (T != 1 || !has_shared) return 0;
  const int rb = router_dtype == WSX_DTYPE_F32 ? 4 : 2;
  if (!layout_supported(H, I, E, k, rb)) return 0;
  const Shape s = fused_shape(H, I, rb);
  if ((is_ling(s) && rb == 2) || (is_tiny(s) && rb == 4)) return 1;
  return 2;
}

}  // namespace

int fused_step_path(int T, int router_dtype, bool has_shared, int H, int I, int E, int k) {
  return fused_path(T, router_dtype, has_shared, H, I, E, k);
}

bool fused_step_supported(int T, int router_dtype, bool has_shared, int H, int I, int E, int k) {
  return fused_path(T, router_dtype, has_shared, H, I, E, k) != 0;
}

size_t fused_step_workspace_bytes(int H, int I, int E, int k, int V) { return fused_layout(H, I, E, k, V).total; }

hipError_t launch_fused_step(const wsx_moe_stack* sk, const uint16_t* h_in, const uint8_t* hq, const float* hs, int V,
                             uint16_t* h_out, float* logits, int32_t* argmax, uint16_t* h_trace, uint16_t* u_trace,
                             int32_t* ids_trace, float* w_trace, void* ws, hipStream_t st, int segments) {
  const int L = sk->L, H = sk->H, I = sk->I, E = sk->E, k = sk->k;
  const FusedLayout f = fused_layout(H, I, E, k, V);
  char* base = reinterpret_cast<char*>(ws);
  FusedStepArgs A;
  A.router = sk->w_router;
  A.w13c = sk->w13_codes; A.w13s = sk->w13_scales; A.w2c = sk->w2_codes; A.w2s = sk->w2_scales;
  A.sh13c = sk->sh13_codes; A.sh13s = sk->sh13_scales; A.sh2c = sk->sh2_codes; A.sh2s = sk->sh2_scales;
  A.hq = hq; A.hs = hs; A.h_in = h_in; A.h_out = h_out; A.logits = logits; A.argmax = argmax;
  A.h_trace = h_trace; A.u_trace = u_trace; A.ids_trace = ids_trace; A.w_trace = w_trace;
  A.b.ctl = base + f.ctl;
  A.b.hx = reinterpret_cast<uint2*>(base + f.hx);
  A.b.lg = reinterpret_cast<uint2*>(base + f.lg);
  A.b.a = reinterpret_cast<uint2*>(base + f.a);
  A.L = L; A.H = H; A.I = I; A.E = E; A.k = k; A.V = V;
  A.nslot = k + 1;
  A.nR = E / kRRows;
  A.nS = I / kGRows;
  A.nG = k * (I / kGRows);
  A.nD = H / kDRows;
  A.per_layer = A.nR + A.nS + A.nG + A.nD;
  A.n_head = f.n_head;
  const size_t lds = fused_lds_bytes(H, I, k);
  const int total = L * A.per_layer + A.n_head;
  const int rb = sk->router_dtype == WSX_DTYPE_F32 ? 4 : 2;
  const Shape s = fused_shape(H, I, rb);
  const bool aot = (is_ling(s) && rb == 2) || (is_tiny(s) && rb == 4);
  hipFunction_t rtc = nullptr;
  if (!aot) {
    const hipError_t e = rtc_kernel(s, rb, &rtc);
    if (e != hipSuccess) return e;
  }
  // The workgroups run in one launch (segments = 0), one launch per layer
  // plus one for the head (1), or one per phase (2); every split respects the
  // dependency order, so the waits inside simply find their data ready.
  int cuts[4 * WSX_MAX_LAYERS + 2];
  int nc = 0;
  cuts[nc++] = 0;
  if (segments > 0) {
    for (int l = 0; l < L; ++l) {
      const int b = l * A.per_layer;
      if (segments == 2) {
        cuts[nc++] = b + A.nR;
        cuts[nc++] = b + A.nR + A.nS + A.nG;
      }
      cuts[nc++] = b + A.per_layer;
    }
  }
  cuts[nc++] = total;
  for (int c = 0; c + 1 < nc; ++c) {
    A.block0 = cuts[c];
    const int grid = cuts[c + 1] - cuts[c];
    if (grid <= 0) continue;
    if (is_ling(s) && rb == 2) {
      decode_step_kernel<5, 3, 10, 10, 3, 6, 2><<<grid, NT, lds, st>>>(A);
    } else if (is_tiny(s) && rb == 4) {
      decode_step_kernel<1, 1, 2, 1, 1, 1, 4><<<grid, NT, lds, st>>>(A);
    } else {
      void* args[] = {&A};
      const hipError_t e = hipModuleLaunchKernel(rtc, (unsigned)grid, 1, 1, NT, 1, 1, (unsigned)lds, st, args, nullptr);
      if (e != hipSuccess) return e;
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace wsx
