// C ABI of libwsx.so: host-side argument validation, workspace layout and
// launch sequencing.  Every check runs before anything is enqueued; on an
// error no work is enqueued and outputs are untouched.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "wsx_internal.h"

// Device scratch of the allocation-free decode step (moe_decode_step_noalloc):
// one copy per GPU, held until the process ends.  Host code never uses this
// name as an address: each device's copy is located once with
// hipGetSymbolAddress and only that pointer is passed to kernels.
static __device__ __align__(256) uint8_t scratch[WSX_NOALLOC_SCRATCH_BYTES];

namespace {

using namespace wsx;

inline size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }
inline bool a16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
inline hipStream_t S(void* s) { return reinterpret_cast<hipStream_t>(s); }
inline wsx_status hip_status(hipError_t e) { return e == hipSuccess ? WSX_OK : WSX_ERR_HIP; }

struct MoeWs {
  size_t counter, dcnt, logits, a, part, total;
};
// The counters first, at offsets that depend on H only, so one workspace
// serves calls with any T (every counter is back at zero after a call): the
// router's counter, the grouped down kernel's per-row-tile counters (64-byte
// stride); then the router logits, the expert activations and the grouped
// down kernel's partial sums, all overwritten before they are read.
MoeWs moe_ws(int T, int H, int I, int E, int k) {
  MoeWs w;
  w.counter = 0;
  w.dcnt = 256;
  w.logits = align256(w.dcnt + (size_t)(H / 32 + 1) * 64);
  w.a = align256(w.logits + (size_t)T * E * 4);
  w.part = align256(w.a + (size_t)(T * k + 1) * T * I * 4);
  const int ng = down_groups(T * k + 1) > down_sparse_groups(T, k) ? down_groups(T * k + 1) : down_sparse_groups(T, k);
  w.total = align256(w.part + (size_t)ng * T * H * 4);
  return w;
}
size_t head_ws_bytes() { return 256 + (size_t)2 * kHeadMaxGrid * WSX_MAX_T * 4; }

// The per-phase region of the decode step: the head's region (its counter
// first) and the MoE region at fixed offsets, then the T-dependent buffers.
struct StepWs {
  MoeWs moe;
  size_t moe_base, head, u, h0, h1, ids, w, el, sw, total;
};
StepWs step_ws(int T, int H, int I, int E, int k) {
  StepWs s;
  s.moe = moe_ws(T, H, I, E, k);
  s.head = 0;
  s.moe_base = align256(head_ws_bytes());
  s.u = align256(s.moe_base + s.moe.total);
  s.h0 = align256(s.u + (size_t)T * H * 2);
  s.h1 = align256(s.h0 + (size_t)T * H * 2);
  s.ids = align256(s.h1 + (size_t)T * H * 2);
  s.w = align256(s.ids + (size_t)T * k * 4);
  s.el = align256(s.w + (size_t)T * k * 4);
  s.sw = align256(s.el + (size_t)(1 + T * k) * 4);
  s.total = align256(s.sw + (size_t)T * k * T * 4);
  return s;
}

// maxT: WSX_MAX_T_MOE for the MoE layer's entry points, WSX_MAX_T where the
// head or the decode step is involved
wsx_status check_tk(int T, int k, int E, int maxT) {
  if (T < 1 || k < 1 || E < 1 || k > E) return WSX_ERR_SHAPE;
  if (T > maxT || k > WSX_MAX_K || E > WSX_MAX_E) return WSX_ERR_UNSUPPORTED;
  return WSX_OK;
}

wsx_status check_ws(const void* ws, size_t have, size_t need) {
  if (!ws) return WSX_ERR_WORKSPACE;
  if (((uintptr_t)ws & 255u) != 0) return WSX_ERR_ALIGN;
  if (have < need) return WSX_ERR_WORKSPACE;
  return WSX_OK;
}

wsx_status check_router(const uint16_t* x, const void* w_router, int router_dtype, int T, int H, int E, int k,
                        int maxT) {
  if (!x || !w_router) return WSX_ERR_NULL;
  if (router_dtype != WSX_DTYPE_BF16 && router_dtype != WSX_DTYPE_F32) return WSX_ERR_DTYPE;
  wsx_status st = check_tk(T, k, E, maxT);
  if (st != WSX_OK) return st;
  if (H < 32 || H % 32) return WSX_ERR_SHAPE;
  if (!router_shape_supported(router_dtype, H)) return WSX_ERR_UNSUPPORTED;
  if (!a16(x) || !a16(w_router)) return WSX_ERR_ALIGN;
  return WSX_OK;
}

// Weights and shapes of the expert stage (the expert list is checked by the caller).
wsx_status check_experts(const uint16_t* x, const uint8_t* w13c, const uint8_t* w13s, const uint8_t* w2c,
                         const uint8_t* w2s, const uint8_t* sh13c, const uint8_t* sh13s, const uint8_t* sh2c,
                         const uint8_t* sh2s, int T, int H, int I, int E, int k, int maxT) {
  if (!x || !w13c || !w13s || !w2c || !w2s) return WSX_ERR_NULL;
  const int nsh = (sh13c != nullptr) + (sh13s != nullptr) + (sh2c != nullptr) + (sh2s != nullptr);
  if (nsh != 0 && nsh != 4) return WSX_ERR_NULL;
  wsx_status st = check_tk(T, k, E, maxT);
  if (st != WSX_OK) return st;
  if (H < 32 || I < 32 || H % 32 || I % 32) return WSX_ERR_SHAPE;
  if (!experts_shape_supported(H, I)) return WSX_ERR_UNSUPPORTED;
  if (!a16(x) || !a16(w13c) || !a16(w2c) || !a16(w13s) || !a16(w2s)) return WSX_ERR_ALIGN;
  if (sh13c && (!a16(sh13c) || !a16(sh2c) || !a16(sh13s) || !a16(sh2s))) return WSX_ERR_ALIGN;
  return WSX_OK;
}

// The host-side checks of moe_decode_step that do not involve the workspace.
wsx_status moe_decode_step_check(const uint16_t* h_in, int T, const wsx_moe_stack* sk, const uint8_t* head_q,
                                 const float* head_scale, int V, const uint16_t* h_out, const int32_t* argmax,
                                 const uint16_t* h_trace, const uint16_t* u_trace) {
  if (!sk || !h_in || !head_q || !head_scale || !h_out || !argmax) return WSX_ERR_NULL;
  if (sk->L < 1) return WSX_ERR_SHAPE;
  if (sk->L > WSX_MAX_LAYERS - 1) return WSX_ERR_UNSUPPORTED;
  const int H = sk->H, I = sk->I, E = sk->E, k = sk->k;
  wsx_status st = check_router(h_in, sk->w_router, sk->router_dtype, T, H, E, k, WSX_MAX_T);
  if (st != WSX_OK) return st;
  st = check_experts(h_in, sk->w13_codes, sk->w13_scales, sk->w2_codes, sk->w2_scales, sk->sh13_codes,
                     sk->sh13_scales, sk->sh2_codes, sk->sh2_scales, T, H, I, E, k, WSX_MAX_T);
  if (st != WSX_OK) return st;
  if (V < 1) return WSX_ERR_SHAPE;
  if (!head_shape_supported(0, H)) return WSX_ERR_UNSUPPORTED;
  if (!a16(head_q) || !a16(h_out)) return WSX_ERR_ALIGN;
  if ((h_trace && !a16(h_trace)) || (u_trace && !a16(u_trace))) return WSX_ERR_ALIGN;
  return WSX_OK;
}

}  // namespace

extern "C" {

size_t wsx_moe_workspace_bytes(int T, int H, int I, int E, int k) {
  (void)H;
  if (T < 1 || T > WSX_MAX_T_MOE || k < 1 || k > WSX_MAX_K || E < 1 || E > WSX_MAX_E || I < 0) return 0;
  return moe_ws(T, H, I, E, k).total;
}

size_t wsx_lm_head_workspace_bytes(int T, int V, int K) {
  (void)T; (void)V; (void)K;
  return head_ws_bytes();
}

size_t wsx_decode_step_workspace_bytes(int T, int H, int I, int E, int k, int V) {
  if (T < 1 || T > WSX_MAX_T || k < 1 || k > WSX_MAX_K || E < 1 || E > WSX_MAX_E || I < 0 || H < 0 || V < 0) return 0;
  // the single-launch step's exchange buffers, then the per-phase region
  return fused_step_workspace_bytes(H, I, E, k, V) + step_ws(T, H, I, E, k).total;
}

wsx_status moe_route_topk(const uint16_t* x, const void* w_router, int router_dtype, int T, int H, int E, int k,
                          int32_t* topk_ids, float* topk_w, int32_t* expert_list, float* slot_w, float* logits_out,
                          void* ws, size_t ws_bytes, void* stream) {
  wsx_status st = check_router(x, w_router, router_dtype, T, H, E, k, WSX_MAX_T_MOE);
  if (st != WSX_OK) return st;
  if (!topk_ids || !topk_w || !expert_list || !slot_w) return WSX_ERR_NULL;
  if ((st = check_ws(ws, ws_bytes, moe_ws(T, H, 32, E, k).a)) != WSX_OK) return st;   // counters + logits
  const MoeWs L = moe_ws(T, H, 32, E, k);
  float* logits = logits_out ? logits_out : reinterpret_cast<float*>((char*)ws + L.logits);
  return hip_status(launch_router(router_dtype, w_router, E, H, k, x, T, 0, nullptr, logits, topk_ids, topk_w,
                                  expert_list, slot_w, reinterpret_cast<unsigned*>((char*)ws + L.counter), S(stream)));
}

wsx_status moe_expert_gemv_mxfp4(const uint16_t* x, const uint8_t* w13_codes, const uint8_t* w13_scales,
                                 const uint8_t* w2_codes, const uint8_t* w2_scales, const uint8_t* sh13_codes,
                                 const uint8_t* sh13_scales, const uint8_t* sh2_codes, const uint8_t* sh2_scales,
                                 const int32_t* expert_list, const float* slot_w, int T, int H, int I, int E, int k,
                                 const uint16_t* residual, float* out_y, uint16_t* out_h, void* ws, size_t ws_bytes,
                                 void* stream) {
  if (!expert_list || !slot_w) return WSX_ERR_NULL;
  wsx_status st = check_experts(x, w13_codes, w13_scales, w2_codes, w2_scales, sh13_codes, sh13_scales, sh2_codes,
                                sh2_scales, T, H, I, E, k, WSX_MAX_T_MOE);
  if (st != WSX_OK) return st;
  if (out_h && !residual) return WSX_ERR_NULL;
  const MoeWs L = moe_ws(T, H, I, E, k);
  if ((st = check_ws(ws, ws_bytes, L.total)) != WSX_OK) return st;
  float* a = reinterpret_cast<float*>((char*)ws + L.a);
  float* part = reinterpret_cast<float*>((char*)ws + L.part);
  unsigned* dcnt = reinterpret_cast<unsigned*>((char*)ws + L.dcnt);
  hipError_t e = launch_gateup(x, T, H, I, E, k, w13_codes, w13_scales, sh13_codes, sh13_scales, expert_list, slot_w,
                               a, S(stream));
  if (e != hipSuccess) return WSX_ERR_HIP;
  return hip_status(launch_down(T, H, I, E, k, w2_codes, w2_scales, sh2_codes, sh2_scales, expert_list, slot_w, a,
                                residual, out_y, out_h, nullptr, part, dcnt, S(stream)));
}

wsx_status act_quantize_mxfp8(const uint16_t* x, int T, int K, uint8_t* codes, uint8_t* scales, void* stream) {
  if (!x || !codes || !scales) return WSX_ERR_NULL;
  if (T < 1 || K < 32 || K % 32) return WSX_ERR_SHAPE;
  if ((size_t)T * (K / 32) > 0x7FFFFFFF) return WSX_ERR_UNSUPPORTED;
  if (!a16(x) || !a16(codes)) return WSX_ERR_ALIGN;
  return hip_status(launch_act_quant(x, T, K, codes, scales, S(stream)));
}

wsx_status moe_expert_gemv_w4a8(const uint16_t* x, const uint8_t* w13_codes, const uint8_t* w13_scales,
                                const uint8_t* w2_codes, const uint8_t* w2_scales, const uint8_t* sh13_codes,
                                const uint8_t* sh13_scales, const uint8_t* sh2_codes, const uint8_t* sh2_scales,
                                const int32_t* expert_list, const float* slot_w, int T, int H, int I, int E, int k,
                                const uint16_t* residual, float* out_y, uint16_t* out_h, float* act_out, void* ws,
                                size_t ws_bytes, void* stream) {
  if (!expert_list || !slot_w) return WSX_ERR_NULL;
  wsx_status st = check_experts(x, w13_codes, w13_scales, w2_codes, w2_scales, sh13_codes, sh13_scales, sh2_codes,
                                sh2_scales, T, H, I, E, k, WSX_MAX_T_MOE);
  if (st != WSX_OK) return st;
  if (!w4a8_shape_supported(T, H, I)) return WSX_ERR_UNSUPPORTED;
  if (out_h && !residual) return WSX_ERR_NULL;
  if (act_out && !a16(act_out)) return WSX_ERR_ALIGN;
  const MoeWs L = moe_ws(T, H, I, E, k);
  if ((st = check_ws(ws, ws_bytes, L.total)) != WSX_OK) return st;
  return hip_status(launch_w4a8_experts(x, T, H, I, E, k, w13_codes, w13_scales, w2_codes, w2_scales, sh13_codes,
                                        sh13_scales, sh2_codes, sh2_scales, expert_list, slot_w, residual, out_y,
                                        out_h, act_out, (char*)ws + L.a, reinterpret_cast<float*>((char*)ws + L.part),
                                        reinterpret_cast<unsigned*>((char*)ws + L.dcnt), S(stream)));
}

wsx_status lm_head_quantize_fp8(const uint16_t* w, int V, int K, uint8_t* q, float* row_scale, void* stream) {
  if (!w || !q || !row_scale) return WSX_ERR_NULL;
  if (V < 1 || K < 32 || K % 32) return WSX_ERR_SHAPE;
  if (K > 16384) return WSX_ERR_UNSUPPORTED;
  if (!a16(w) || !a16(q)) return WSX_ERR_ALIGN;
  return hip_status(launch_quant_fp8(w, V, K, q, row_scale, S(stream)));
}

static wsx_status head_common(int wt, const void* W, const float* s, int V, int K, const uint16_t* x, int T,
                              float* logits, int32_t* argmax, void* ws, size_t ws_bytes, void* stream) {
  if (!W || !x || !argmax || (wt == 0 && !s)) return WSX_ERR_NULL;
  if (V < 1 || K < 32 || K % 32 || T < 1) return WSX_ERR_SHAPE;
  if (T > WSX_MAX_T || !head_shape_supported(wt, K)) return WSX_ERR_UNSUPPORTED;
  if (!a16(W) || !a16(x)) return WSX_ERR_ALIGN;
  wsx_status st = check_ws(ws, ws_bytes, head_ws_bytes());
  if (st != WSX_OK) return st;
  return hip_status(launch_lm_head(wt, W, s, V, K, x, T, 0, nullptr, logits, argmax, ws, S(stream)));
}

wsx_status lm_head_gemv_fp8_argmax(const uint8_t* q, const float* row_scale, int V, int K, const uint16_t* x, int T,
                                   float* logits, int32_t* argmax, void* ws, size_t ws_bytes, void* stream) {
  return head_common(0, q, row_scale, V, K, x, T, logits, argmax, ws, ws_bytes, stream);
}

wsx_status lm_head_gemv_bf16_argmax(const uint16_t* w, int V, int K, const uint16_t* x, int T, float* logits,
                                    int32_t* argmax, void* ws, size_t ws_bytes, void* stream) {
  return head_common(1, w, nullptr, V, K, x, T, logits, argmax, ws, ws_bytes, stream);
}

static wsx_status check_sample(const float* logits, int V, int T, float temperature, int top_k, float top_p,
                               const float* uniforms, const int32_t* token) {
  if (!logits || !uniforms || !token) return WSX_ERR_NULL;
  if (V < 1 || T < 1 || top_k < 1 || top_k > V) return WSX_ERR_SHAPE;
  if (!(temperature > 0.f) || !(temperature <= 3.0e38f) || !(top_p > 0.f) || !(top_p <= 1.f)) return WSX_ERR_SHAPE;
  if (T > WSX_MAX_T || !sample_shape_supported(V, top_k)) return WSX_ERR_UNSUPPORTED;
  return WSX_OK;
}

size_t wsx_sample_workspace_bytes(int T, int V, int top_k) {
  if (T < 1 || T > WSX_MAX_T || !sample_shape_supported(V, top_k)) return 0;
  return sample_ws_bytes(T, V, top_k);
}

wsx_status lm_sample_topk_topp(const float* logits, int V, int T, float temperature, int top_k, float top_p,
                               const float* uniforms, int32_t* token, int32_t* topk_ids, float* topk_probs, void* ws,
                               size_t ws_bytes, void* stream) {
  wsx_status st = check_sample(logits, V, T, temperature, top_k, top_p, uniforms, token);
  if (st != WSX_OK) return st;
  if ((st = check_ws(ws, ws_bytes, sample_ws_bytes(T, V, top_k))) != WSX_OK) return st;
  return hip_status(launch_sample(logits, V, T, temperature, top_k, top_p, uniforms, token, topk_ids, topk_probs,
                                  ws, S(stream)));
}

static size_t head_sample_region(int T, int V, int top_k) {
  const size_t s = sample_ws_bytes(T, V, top_k), f = head_sample_fused_ws_bytes(top_k);
  return T == 1 && f > s ? f : s;
}

size_t wsx_lm_head_sample_workspace_bytes(int T, int V, int K, int top_k) {
  if (!wsx_sample_workspace_bytes(T, V, top_k)) return 0;
  return align256(head_ws_bytes()) + 256 + head_sample_region(T, V, top_k);
}

int wsx_lm_head_sample_path(int T, int V, int K, int top_k) {
  if (T < 1 || T > WSX_MAX_T || !sample_shape_supported(V, top_k) || !head_shape_supported(0, K)) return -1;
  return T == 1 ? head_sample_fused_path(V, K, top_k) : 0;
}

wsx_status lm_head_gemv_fp8_sample(const uint8_t* q, const float* row_scale, int V, int K, const uint16_t* x, int T,
                                   float temperature, int top_k, float top_p, const float* uniforms, float* logits,
                                   int32_t* token, int32_t* topk_ids, float* topk_probs, void* ws, size_t ws_bytes,
                                   void* stream) {
  if (!q || !row_scale || !x) return WSX_ERR_NULL;
  wsx_status st = check_sample(logits, V, T, temperature, top_k, top_p, uniforms, token);
  if (st != WSX_OK) return st;
  if (K < 32 || K % 32) return WSX_ERR_SHAPE;
  if (!head_shape_supported(0, K)) return WSX_ERR_UNSUPPORTED;
  if (!a16(q) || !a16(x)) return WSX_ERR_ALIGN;
  // workspace: the head's region, 256 bytes for the head's greedy argmax (a
  // by-product of the two-launch form), then the sampler's region
  const size_t head = align256(head_ws_bytes());
  if ((st = check_ws(ws, ws_bytes, head + 256 + head_sample_region(T, V, top_k))) != WSX_OK) return st;
  if (T == 1) {
    // one launch: the head with the selection in its last workgroup
    bool done = false;
    const hipError_t e = launch_lm_head_sample_fused(q, row_scale, V, K, x, temperature, top_k, top_p, uniforms, logits,
                                                     token, topk_ids, topk_probs, ws, (char*)ws + head + 256,
                                                     S(stream), &done);
    if (e != hipSuccess) return WSX_ERR_HIP;
    if (done) return WSX_OK;
  }
  int32_t* argmax = reinterpret_cast<int32_t*>((char*)ws + head);
  hipError_t e = launch_lm_head(0, q, row_scale, V, K, x, T, 0, nullptr, logits, argmax, ws, S(stream));
  if (e != hipSuccess) return WSX_ERR_HIP;
  return hip_status(launch_sample(logits, V, T, temperature, top_k, top_p, uniforms, token, topk_ids, topk_probs,
                                  (char*)ws + head + 256, S(stream)));
}

}  // extern "C"

namespace {

// Zero fill of the scratch at set-up, as a kernel on the caller's stream.
__global__ void zero_scratch_kernel(uint4* p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0, 0, 0, 0);
}

constexpr int kMaxDevices = 64;
struct ScratchShape {
  int H, I, E, k, V;
  bool operator==(const ScratchShape& o) const { return H == o.H && I == o.I && E == o.E && k == o.k && V == o.V; }
};
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];          // this device's copy of `scratch`, once located
ScratchShape g_scratch_shape[kMaxDevices];  // the stack shape its contents belong to

// The current device's scratch pointer for a stack of shape `sh`.  On the
// first call on a device the symbol is located (hipGetSymbolAddress, with that
// device current).  The whole array is cleared by a kernel enqueued on `s`,
// ahead of the step that follows on the same stream, on that first call and
// whenever the stack shape differs from the previous call's (the layout of
// the exchange buffers and counters depends on it).
wsx_status scratch_for_current_device(hipStream_t s, const ScratchShape& sh, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return WSX_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  void* ptr = g_scratch_ptr[dev];
  const bool fresh = ptr == nullptr;
  if (fresh && (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr)) return WSX_ERR_HIP;
  if (fresh || !(g_scratch_shape[dev] == sh)) {
    zero_scratch_kernel<<<256, 256, 0, s>>>(reinterpret_cast<uint4*>(ptr), WSX_NOALLOC_SCRATCH_BYTES / 16);
    if (hipGetLastError() != hipSuccess) return WSX_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
    g_scratch_shape[dev] = sh;
  }
  *out = ptr;
  return WSX_OK;
}

}  // namespace

extern "C" {

wsx_status moe_decode_step_noalloc(const uint16_t* h_in, int T, const wsx_moe_stack* sk, const uint8_t* head_q,
                                   const float* head_scale, int V, uint16_t* h_out, float* logits, int32_t* argmax,
                                   uint16_t* h_trace, uint16_t* u_trace, int32_t* ids_trace, float* w_trace,
                                   void* stream) {
  if (!sk) return WSX_ERR_NULL;
  const size_t need = wsx_decode_step_workspace_bytes(T, sk->H, sk->I, sk->E, sk->k, V);
  if (need == 0) return (T < 1 || sk->k < 1 || sk->E < 1 || V < 0) ? WSX_ERR_SHAPE : WSX_ERR_UNSUPPORTED;
  if (need > WSX_NOALLOC_SCRATCH_BYTES) return WSX_ERR_WORKSPACE;
  // every host-side check of the allocating entry point, with a stand-in
  // workspace, before anything touches the device
  wsx_status st = moe_decode_step_check(h_in, T, sk, head_q, head_scale, V, h_out, argmax, h_trace, u_trace);
  if (st != WSX_OK) return st;
  void* ws = nullptr;
  if ((st = scratch_for_current_device(S(stream), ScratchShape{sk->H, sk->I, sk->E, sk->k, V}, &ws)) != WSX_OK)
    return st;
  return moe_decode_step(h_in, T, sk, head_q, head_scale, V, h_out, logits, argmax, h_trace, u_trace, ids_trace,
                         w_trace, ws, WSX_NOALLOC_SCRATCH_BYTES, stream);
}

wsx_status moe_decode_step(const uint16_t* h_in, int T, const wsx_moe_stack* sk, const uint8_t* head_q,
                           const float* head_scale, int V, uint16_t* h_out, float* logits, int32_t* argmax,
                           uint16_t* h_trace, uint16_t* u_trace, int32_t* ids_trace, float* w_trace, void* ws,
                           size_t ws_bytes, void* stream) {
  wsx_status st = moe_decode_step_check(h_in, T, sk, head_q, head_scale, V, h_out, argmax, h_trace, u_trace);
  if (st != WSX_OK) return st;
  const int H = sk->H, I = sk->I, E = sk->E, k = sk->k, L = sk->L;
  const StepWs W = step_ws(T, H, I, E, k);
  // workspace: the single-launch step's exchange buffers first (their place
  // does not depend on T), then the per-phase region
  const size_t fused_bytes = fused_step_workspace_bytes(H, I, E, k, V);
  if ((st = check_ws(ws, ws_bytes, fused_bytes + W.total)) != WSX_OK) return st;
  if (fused_step_supported(T, sk->router_dtype, sk->sh13_codes != nullptr, H, I, E, k))
    return hip_status(launch_fused_step(sk, h_in, head_q, head_scale, V, h_out, logits, argmax, h_trace, u_trace,
                                        ids_trace, w_trace, ws, S(stream), kStepSegments));

  char* base = reinterpret_cast<char*>(ws) + fused_bytes;
  char* mbase = base + W.moe_base;
  unsigned* counter = reinterpret_cast<unsigned*>(mbase + W.moe.counter);
  float* rlogits = reinterpret_cast<float*>(mbase + W.moe.logits);
  float* a = reinterpret_cast<float*>(mbase + W.moe.a);
  float* part = reinterpret_cast<float*>(mbase + W.moe.part);
  unsigned* dcnt = reinterpret_cast<unsigned*>(mbase + W.moe.dcnt);
  int32_t* el = reinterpret_cast<int32_t*>(base + W.el);
  float* sw = reinterpret_cast<float*>(base + W.sw);
  uint16_t* ping[2] = {reinterpret_cast<uint16_t*>(base + W.h0), reinterpret_cast<uint16_t*>(base + W.h1)};
  const size_t TH = (size_t)T * H;
  const size_t esz = sk->router_dtype == WSX_DTYPE_F32 ? 4 : 2;
  const size_t r_stride = (size_t)E * H * esz;
  const size_t c13 = (size_t)E * 2 * I * (H / 2), s13 = (size_t)E * 2 * I * (H / 32);
  const size_t c2 = (size_t)E * H * (I / 2), s2 = (size_t)E * H * (I / 32);
  const size_t sc13 = (size_t)2 * I * (H / 2), ss13 = (size_t)2 * I * (H / 32);
  const size_t sc2 = (size_t)H * (I / 2), ss2 = (size_t)H * (I / 32);
  const bool sh = sk->sh13_codes != nullptr;
  hipStream_t s = S(stream);

  const uint16_t* h_cur = h_in;
  if (h_trace) {
    // h_0 is the input itself; record it
    if (hipMemcpyAsync(h_trace, h_in, TH * 2, hipMemcpyDeviceToDevice, s) != hipSuccess) return WSX_ERR_HIP;
  }
  for (int l = 0; l < L; ++l) {
    uint16_t* u = u_trace ? u_trace + (size_t)l * TH : reinterpret_cast<uint16_t*>(base + W.u);
    int32_t* ids = ids_trace ? ids_trace + (size_t)l * T * k : reinterpret_cast<int32_t*>(base + W.ids);
    float* tw = w_trace ? w_trace + (size_t)l * T * k : reinterpret_cast<float*>(base + W.w);
    uint16_t* h_next = h_trace ? h_trace + (size_t)(l + 1) * TH : (l == L - 1 ? h_out : ping[l & 1]);
    uint16_t* h_next2 = (h_trace && l == L - 1) ? h_out : nullptr;
    const char* wr = reinterpret_cast<const char*>(sk->w_router) + (size_t)l * r_stride;
    hipError_t e = launch_router(sk->router_dtype, wr, E, H, k, h_cur, T, 1, u, rlogits, ids, tw, el, sw, counter, s);
    if (e != hipSuccess) return WSX_ERR_HIP;
    e = launch_gateup(u, T, H, I, E, k, sk->w13_codes + (size_t)l * c13, sk->w13_scales + (size_t)l * s13,
                      sh ? sk->sh13_codes + (size_t)l * sc13 : nullptr, sh ? sk->sh13_scales + (size_t)l * ss13 : nullptr,
                      el, sw, a, s);
    if (e != hipSuccess) return WSX_ERR_HIP;
    e = launch_down(T, H, I, E, k, sk->w2_codes + (size_t)l * c2, sk->w2_scales + (size_t)l * s2,
                    sh ? sk->sh2_codes + (size_t)l * sc2 : nullptr, sh ? sk->sh2_scales + (size_t)l * ss2 : nullptr,
                    el, sw, a, h_cur, nullptr, h_next, h_next2, part, dcnt, s);
    if (e != hipSuccess) return WSX_ERR_HIP;
    h_cur = h_next;
  }
  uint16_t* u_head = u_trace ? u_trace + (size_t)L * TH : nullptr;
  return hip_status(launch_lm_head(0, head_q, head_scale, V, H, h_cur, T, 1, u_head, logits, argmax,
                                   base + W.head, s));
}

int wsx_decode_step_path(int T, int router_dtype, int has_shared, int H, int I, int E, int k) {
  if (router_dtype != WSX_DTYPE_BF16 && router_dtype != WSX_DTYPE_F32) return 0;
  return fused_step_path(T, router_dtype, has_shared != 0, H, I, E, k);
}

wsx_status wsx_read_probe(const void* buf, size_t bytes, uint32_t* out, void* stream) {
  if (!buf || !out) return WSX_ERR_NULL;
  if (bytes == 0 || bytes % 16) return WSX_ERR_SHAPE;
  if (!a16(buf)) return WSX_ERR_ALIGN;
  return hip_status(launch_read_probe(buf, bytes, out, S(stream)));
}

const char* wsx_status_string(wsx_status s) {
  switch (s) {
    case WSX_OK: return "ok";
    case WSX_ERR_NULL: return "required pointer is NULL";
    case WSX_ERR_SHAPE: return "size out of range or not a multiple of 32";
    case WSX_ERR_ALIGN: return "pointer not 16-byte aligned (workspace: 256-byte)";
    case WSX_ERR_UNSUPPORTED: return "shape valid but not supported by the compiled kernels";
    case WSX_ERR_WORKSPACE: return "workspace missing or too small";
    case WSX_ERR_DTYPE: return "unknown dtype code";
    case WSX_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

#define WSX_STR2(x) #x
#define WSX_STR(x) WSX_STR2(x)
const char* wsx_build_info(void) {
  return "libwsx arch=gfx950 hip=" WSX_STR(HIP_VERSION_MAJOR) "." WSX_STR(HIP_VERSION_MINOR)
         " kernels=decode_step<T1;one-launch;aot:Ling-bf16,tiny-f32;hiprtc:other-shapes>,"
         "router_topk<bf16|f32,T1-4;rank-count|T5-16;grouped>,moe_gateup<T1;valu-dot2|T2-4;mfma-bf16|T5-16;mfma-4tiles>,"
         "moe_down<T1;valu|T2-16;token-lists>,moe_w4a8<T1-16;mfma-scale-f8f6f4>,"
         "lm_head<fp8|bf16,T1;wide-per-CU>,lm_head<fp8,T2-4;wide-per-CU,norm>,lm_head<bf16,T2-4>,quant_fp8,"
         "sample<topk<=64,topp;fused-into-head-T1>";
}

}  // extern "C"
