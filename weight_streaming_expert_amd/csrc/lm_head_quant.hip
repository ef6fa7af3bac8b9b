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

// The row stays in registers between the two passes: each lane issues the
// loads of all its CPL 16-element chunks (lane + 64 i) at once, takes their
// maximum, then encodes them from the same registers.
template <int CPL>
__global__ void __launch_bounds__(256) quant_fp8_kernel(const uint16_t* __restrict__ w, int V, int K,
                                                        uint8_t* __restrict__ q, float* __restrict__ row_scale) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= V) return;
  const uint16_t* wr = w + (size_t)row * K;
  const int NC = K / 16;   // 16-element chunks: 32 bytes in, 16 bytes out
  uint4 a[CPL], b[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int ch = lane + 64 * i;
    a[i] = b[i] = make_uint4(0, 0, 0, 0);   // zeros do not change the maximum
    if (ch < NC) {
      a[i] = ld16(wr + (size_t)ch * 16);
      b[i] = ld16(wr + (size_t)ch * 16 + 8);
    }
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const uint32_t v[8] = {a[i].x, a[i].y, a[i].z, a[i].w, b[i].x, b[i].y, b[i].z, b[i].w};
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fmaxf(fabsf(bf16lo(v[j])), fabsf(bf16hi(v[j]))));
  }
  amax = wave_max(amax);
  const float s = amax / 448.0f;
  if (lane == 0) row_scale[row] = s;
  uint8_t* qr = q + (size_t)row * K;
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int ch = lane + 64 * i;
    if (ch < NC) {
      uint4 o;
      o.x = enc4(a[i].x, a[i].y, s);
      o.y = enc4(a[i].z, a[i].w, s);
      o.z = enc4(b[i].x, b[i].y, s);
      o.w = enc4(b[i].z, b[i].w, s);
      *reinterpret_cast<uint4*>(qr + (size_t)ch * 16) = o;
    }
  }
}

hipError_t launch_quant_fp8(const uint16_t* w, int V, int K, uint8_t* q, float* s, hipStream_t st) {
  const int cpl = (K / 16 + 63) / 64;   // K <= 16384: at most 16 chunks per lane
  const int grid = (V + 3) / 4;
#define WSX_Q_CASE(N)                                                                  \
  if (cpl <= N) {                                                                      \
    quant_fp8_kernel<N><<<grid, 256, 0, st>>>(w, V, K, q, s);                          \
    return hipGetLastError();                                                          \
  }
  WSX_Q_CASE(1) WSX_Q_CASE(2) WSX_Q_CASE(3) WSX_Q_CASE(4) WSX_Q_CASE(8) WSX_Q_CASE(16)
#undef WSX_Q_CASE
  return hipErrorInvalidValue;
}

}  // namespace wsx
