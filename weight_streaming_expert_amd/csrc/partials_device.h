// Device helper shared by the kernels that fold per-group partial sums in a
// last workgroup (the token-list down of moe_experts.hip and the W4A8 down).
#pragma once
#include "wsx_device.h"

namespace wsx {

// Sum, in group order, of the ng partials part[(g T + t) H + n] (written by
// other workgroups with device-coherent stores): the loads go out eight at a
// time, so the tail costs one coherent round trip per eight groups, not one
// per group.
__device__ __forceinline__ float sum_group_partials(const float* part, int ng, int T, int H, int t, int n) {
  float y = 0.f;
  for (int g0 = 0; g0 < ng; g0 += 8) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      v[j] = g0 + j < ng ? __uint_as_float(ld_coh4(part, (uint32_t)(((size_t)(g0 + j) * T + t) * H + n) * 4)) : 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (g0 + j < ng) y += v[j];
  }
  return y;
}

}  // namespace wsx
