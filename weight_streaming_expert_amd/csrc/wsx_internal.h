// Internal launcher interface between the C ABI (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/wsx.h"

namespace wsx {

constexpr int kHeadMaxGrid = 1024;   // workgroups of the LM-head GEMV (argmax partials)

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
                         float* a, hipStream_t st);
hipError_t launch_down(int T, int H, int I, int E, int k, const uint8_t* w2c, const uint8_t* w2s,
                       const uint8_t* sh2c, const uint8_t* sh2s, const int32_t* el, const float* sw, const float* a,
                       const uint16_t* res, float* y, uint16_t* h, uint16_t* h2, hipStream_t st);

// lm_head_quant.hip
hipError_t launch_quant_fp8(const uint16_t* w, int V, int K, uint8_t* q, float* s, hipStream_t st);

}  // namespace wsx
