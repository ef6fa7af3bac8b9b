// Internal launcher interface between the C ABI (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/wsx.h"

namespace wsx {

constexpr int kHeadMaxGrid = 1024;   // workgroups of the LM-head GEMV (argmax partials)
constexpr int WSX_MAX_LAYERS = 256;   // stacked layers per decode step (tags hold the layer in 8 bits)
// How the single-launch decode step is split into launches: 0 = one launch,
// 1 = one per layer plus the head, 2 = one per phase.
constexpr int kStepSegments = 0;

// gemv_rows.hip
bool head_shape_supported(int wt, int K);           // wt: 0 fp8, 1 bf16
bool router_shape_supported(int router_dtype, int K);
int head_grid(int V);
hipError_t launch_lm_head(int wt, const void* W, const float* s, int V, int K, const uint16_t* x, int T, int norm,
                          uint16_t* u_out, float* logits, int32_t* argmax, void* ws, hipStream_t st);
hipError_t launch_router(int router_dtype, const void* W, int E, int K, int k, const uint16_t* x, int T, int norm,
                         uint16_t* u_out, float* logits, int32_t* ids, float* w, int32_t* el, float* sw,
                         unsigned* counter, hipStream_t st);

// moe_experts.hip
bool experts_shape_supported(int H, int I);
hipError_t launch_gateup(const uint16_t* x, int T, int H, int I, int E, int k, const uint8_t* w13c,
                         const uint8_t* w13s, const uint8_t* sh13c, const uint8_t* sh13s, const int32_t* el,
                         const float* sw, float* a, hipStream_t st);
hipError_t launch_down(int T, int H, int I, int E, int k, const uint8_t* w2c, const uint8_t* w2s,
                       const uint8_t* sh2c, const uint8_t* sh2s, const int32_t* el, const float* sw, const float* a,
                       const uint16_t* res, float* y, uint16_t* h, uint16_t* h2, float* part, unsigned* counters,
                       hipStream_t st);
// The grouped down kernel for several tokens: slot groups per row tile, the
// bytes of its partial sums ([groups][T][H] fp32) and its per-tile counters.
int down_groups(int max_slots);
int down_sparse_groups(int T, int k);   // the same for 5..16 tokens (sparse token lists)
bool down_grouped_ok(int T, int H, int I);

// moe_w4a8.hip: W4A8 experts (MXFP4 weights x MXFP8 activations on the matrix cores)
bool w4a8_shape_supported(int T, int H, int I);
size_t w4a8_act_bytes(int T, int I, int max_slots);
hipError_t launch_act_quant(const uint16_t* x, int T, int K, uint8_t* codes, uint8_t* scales, hipStream_t st);
hipError_t launch_w4a8_experts(const uint16_t* x, int T, int H, int I, int E, int k, const uint8_t* w13c,
                               const uint8_t* w13s, const uint8_t* w2c, const uint8_t* w2s, const uint8_t* sh13c,
                               const uint8_t* sh13s, const uint8_t* sh2c, const uint8_t* sh2s, const int32_t* el,
                               const float* sw, const uint16_t* res, float* y, uint16_t* h, float* act, void* abuf,
                               float* part, unsigned* counters, hipStream_t st);

// decode_step.hip: the whole 1-token decode step in one launch
bool fused_step_supported(int T, int router_dtype, bool has_shared, int H, int I, int E, int k);
// 0: per-phase launches, 1: one launch compiled ahead of time, 2: one launch compiled at run time (hipRTC)
int fused_step_path(int T, int router_dtype, bool has_shared, int H, int I, int E, int k);
size_t fused_step_workspace_bytes(int H, int I, int E, int k, int V);
hipError_t launch_fused_step(const wsx_moe_stack* sk, const uint16_t* h_in, const uint8_t* hq, const float* hs, int V,
                             uint16_t* h_out, float* logits, int32_t* argmax, uint16_t* h_trace, uint16_t* u_trace,
                             int32_t* ids_trace, float* w_trace, void* ws, hipStream_t st, int segments);

// probe.hip: plain streaming read of a buffer (bandwidth reference)
hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* out, hipStream_t st);

// lm_head_quant.hip
hipError_t launch_quant_fp8(const uint16_t* w, int V, int K, uint8_t* q, float* s, hipStream_t st);

// sample.hip: temperature / top-k / top-p sampling of the head's logits
size_t sample_ws_bytes(int T, int V, int k);
bool sample_shape_supported(int V, int k);
hipError_t launch_sample(const float* logits, int V, int T, float temperature, int k, float top_p,
                         const float* uniforms, int32_t* token, int32_t* topk_ids, float* topk_probs, void* ws,
                         hipStream_t st);

// gemv_rows.hip: the 1-token FP8 head with the sampler fused into its tail.
// head_ws: the head's region (its counters first); sample_ws: at least
// head_sample_fused_ws_bytes(top_k).  *done = false (nothing launched) when the
// shape or device does not fit (head_sample_fused_path == 0).
size_t head_sample_fused_ws_bytes(int k);
int head_sample_fused_path(int V, int K, int top_k);
hipError_t launch_lm_head_sample_fused(const void* W, const float* s, int V, int K, const uint16_t* x,
                                       float temperature, int top_k, float top_p, const float* uniforms,
                                       float* logits, int32_t* token, int32_t* topk_ids, float* topk_probs,
                                       void* head_ws, void* sample_ws, hipStream_t st, bool* done);

}  // namespace wsx
