// Load-time BF16 -> FP8 E4M3FN quantization of the LM head, one fp32 scale per
// vocabulary row, on gfx950.
//
// [saipien] "Stop hauling the vocabulary in full precision" and [genai] "2.
// Compressing the Output Head": only the LM head is quantized, once, when the
// layer is built, so every decode step reads half the bytes.
//
// One wavefront per row: pass 1 takes the exact absolute maximum, the scale is
// s = absmax / 448 (IEEE binary32 division), pass 2 divides each element by s
// (binary32 division), saturates to +-448 and encodes with the hardware
// converter (round to nearest even, OCP E4M3FN).  An all-zero row gets s = 0
// and all-zero codes.
#include "wsx_device.h"
#include "wsx_internal.h"

namespace wsx {

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ float qdiv(float w, float s) {
  float v = s > 0.f ? w / s : 0.f;
  return fminf(fmaxf(v, -448.0f), 448.0f);
}

__device__ __forceinline__ uint32_t enc4(uint32_t a, uint32_t b, float s) {
  // a, b: four bf16 values -> four E4M3FN codes, element order preserved
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(qdiv(bf16lo(a), s), qdiv(bf16hi(a), s), 0, false);
  int both = __builtin_amdgcn_cvt_pk_fp8_f32(qdiv(bf16lo(b), s), qdiv(bf16hi(b), s), lo, true);
  return (uint32_t)both;
}

__global__ void __launch_bounds__(256) quant_fp8_kernel(const uint16_t* __restrict__ w, int V, int K,
                                                        uint8_t* __restrict__ q, float* __restrict__ row_scale) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= V) return;
  const uint16_t* wr = w + (size_t)row * K;
  const int NC = K / 16;   // 16-element chunks: 32 bytes in, 16 bytes out
  float amax = 0.f;
  for (int ch = lane; ch < NC; ch += 64) {
    const uint4 a = ld16(wr + (size_t)ch * 16), b = ld16(wr + (size_t)ch * 16 + 8);
    const uint32_t v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fmaxf(fabsf(bf16lo(v[i])), fabsf(bf16hi(v[i]))));
  }
  amax = wave_max(amax);
  const float s = amax / 448.0f;
  if (lane == 0) row_scale[row] = s;
  uint8_t* qr = q + (size_t)row * K;
  for (int ch = lane; ch < NC; ch += 64) {
    const uint4 a = ld16(wr + (size_t)ch * 16), b = ld16(wr + (size_t)ch * 16 + 8);
    uint4 o;
    o.x = enc4(a.x, a.y, s);
    o.y = enc4(a.z, a.w, s);
    o.z = enc4(b.x, b.y, s);
    o.w = enc4(b.z, b.w, s);
    *reinterpret_cast<uint4*>(qr + (size_t)ch * 16) = o;
  }
}

hipError_t launch_quant_fp8(const uint16_t* w, int V, int K, uint8_t* q, float* s, hipStream_t st) {
  quant_fp8_kernel<<<(V + 3) / 4, 256, 0, st>>>(w, V, K, q, s);
  return hipGetLastError();
}

}  // namespace wsx
