// Routed + shared SwiGLU experts with MXFP4 weights for batch-1 decode and the
// 4-token verify pass, on gfx950.
//
// [saipien] "Why one user waits on weights": each token uses 8 of 512 routed
// experts plus one shared expert, and MoE weight reads dominate decode time.
// [saipien] "Kernels built for the shape you actually have": the routed
// experts are narrow (intermediate size 768).
//
// Two launches per layer, both driven by the device-side expert list (the
// host never learns which experts were chosen):
//   gate/up  grid (I/16, T*k+1): workgroup (i-tile, slot) streams 16 gate rows
//            and the 16 matching up rows of that slot's expert, dequantizes the
//            E2M1 nibbles in registers with the hardware converter, applies the
//            E8M0 block scale per 32 elements and writes a = silu(g) * u (fp32).
//            Surplus workgroups (slots past the active count) exit at once.
//   down     one token: grid (H/8), a workgroup owns 8 output rows and loops
//            over every active slot (its 4 wavefronts take slots round-robin),
//            then sums the four wavefront partials in a fixed order, adds the
//            residual and rounds to bf16.  2..16 tokens: (32-row tile, group
//            of four slots) workgroups over expert-sorted token lists, the
//            groups' partials added in group order by the tile's last
//            workgroup.  The order never depends on timing, so the result is
//            bit-reproducible.
#include "wsx_device.h"
#include "partials_device.h"
#include "wsx_internal.h"

namespace wsx {

// MX block (32 E2M1 codes) x 32 fp32 activations, unscaled.
__device__ __forceinline__ float mx_block_dot_f32(uint4 c, const float* a) {
  float s0 = 0.f, s1 = 0.f;
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    f32x2_t p0 = fp4x2_to_f32x2<0>(w[d]);
    f32x2_t p1 = fp4x2_to_f32x2<1>(w[d]);
    f32x2_t p2 = fp4x2_to_f32x2<2>(w[d]);
    f32x2_t p3 = fp4x2_to_f32x2<3>(w[d]);
    s0 = fmaf(p0.x, a[8 * d + 0], s0);
    s1 = fmaf(p0.y, a[8 * d + 1], s1);
    s0 = fmaf(p1.x, a[8 * d + 2], s0);
    s1 = fmaf(p1.y, a[8 * d + 3], s1);
    s0 = fmaf(p2.x, a[8 * d + 4], s0);
    s1 = fmaf(p2.y, a[8 * d + 5], s1);
    s0 = fmaf(p3.x, a[8 * d + 6], s0);
    s1 = fmaf(p3.y, a[8 * d + 7], s1);
  }
  return s0 + s1;
}

// Resolve slot -> (codes, scales) of its expert; false if the slot is inactive
// or its id is out of range (then the slot contributes nothing).
__device__ __forceinline__ bool slot_expert(int slot, int n_active, bool has_sh, int E, const int32_t* expert_list,
                                            const uint8_t* wc, const uint8_t* ws_, const uint8_t* shc,
                                            const uint8_t* shs, size_t c_stride, size_t s_stride,
                                            const uint8_t** C, const uint8_t** S) {
  if (slot < n_active) {
    const int e = expert_list[1 + slot];
    if (e < 0 || e >= E) return false;
    *C = wc + (size_t)e * c_stride;
    *S = ws_ + (size_t)e * s_stride;
    return true;
  }
  if (slot == n_active && has_sh) { *C = shc; *S = shs; return true; }
  return false;
}

// slot_expert with the slot's list entry already loaded (read beside the
// active count, so the two loads share one round trip): e_slot is
// expert_list[1 + slot] for slot < max_slots - 1, anything otherwise.
__device__ __forceinline__ bool slot_expert_pre(int slot, int n_active, bool has_sh, int E, int e_slot,
                                                const uint8_t* wc, const uint8_t* ws_, const uint8_t* shc,
                                                const uint8_t* shs, size_t c_stride, size_t s_stride,
                                                const uint8_t** C, const uint8_t** S) {
  if (slot < n_active) {
    if (e_slot < 0 || e_slot >= E) return false;
    *C = wc + (size_t)e_slot * c_stride;
    *S = ws_ + (size_t)e_slot * s_stride;
    return true;
  }
  if (slot == n_active && has_sh) { *C = shc; *S = shs; return true; }
  return false;
}

// ---------------------------------------------------------------- gate/up + SwiGLU

template <int T, int NJ>
__global__ void __launch_bounds__(256) moe_gateup_kernel(const uint16_t* __restrict__ x, int H, int I, int E, int max_slots,
                                                         const uint8_t* __restrict__ w13c, const uint8_t* __restrict__ w13s,
                                                         const uint8_t* __restrict__ sh13c, const uint8_t* __restrict__ sh13s,
                                                         const int32_t* __restrict__ expert_list, float* __restrict__ a_out) {
  const int slot = blockIdx.y;
  int n_active = expert_list[0];
  n_active = n_active < 0 ? 0 : (n_active > max_slots - 1 ? max_slots - 1 : n_active);
  const bool has_sh = sh13c != nullptr;
  const int i0 = blockIdx.x * 16;
  const uint8_t *C, *S;
  if (!slot_expert(slot, n_active, has_sh, E, expert_list, w13c, w13s, sh13c, sh13s, (size_t)2 * I * (H / 2),
                   (size_t)2 * I * (H / 32), &C, &S)) {
    // inactive slot past the list: nothing to do; bad id: contribute zeros
    if (slot < n_active + (has_sh ? 1 : 0))
      for (int i = threadIdx.x; i < 16 * T; i += 256) a_out[((size_t)slot * T + i / 16) * I + i0 + (i % 16)] = 0.f;
    return;
  }
  extern __shared__ __attribute__((aligned(16))) uint16_t xs[];
  stage_to_lds<256, (T * 320 + 255) / 256>(x, xs, T * H / 8);
  __syncthreads();
  const uint32_t* xs32 = reinterpret_cast<const uint32_t*>(xs);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane >> 4, c = lane & 15;
  const int NB = H / 32;
  const size_t rowc = H / 2, rows = H / 32;

  uint32_t xr[T == 1 ? NJ : 1][16];
  if constexpr (T == 1) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int b = c + 16 * j;
#pragma unroll
      for (int d = 0; d < 16; ++d) xr[j][d] = (b < NB) ? xs32[b * 16 + d] : 0u;
    }
  }
  // two steps of 4 rows: lanes 0-15 gate i, 16-31 gate i+1, 32-47 up i, 48-63 up i+1
  uint4 cw[2][NJ];
  uint32_t sb[2][NJ];
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    const int ri = i0 + 4 * wave + 2 * st + (r & 1);
    const int row = (r < 2) ? ri : I + ri;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int b = c + 16 * j;
      cw[st][j] = (b < NB) ? ld16(C + row * rowc + (size_t)b * 16) : make_uint4(0, 0, 0, 0);
      sb[st][j] = (b < NB) ? (uint32_t)S[row * rows + b] : 127u;
    }
  }
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    float acc[T];
#pragma unroll
    for (int t = 0; t < T; ++t) acc[t] = 0.f;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int b = c + 16 * j;
      if (b >= NB) continue;
      const float scale = e8m0_to_f32(sb[st][j]);
      if constexpr (T == 1) {
        acc[0] = fmaf(mx_block_dot(cw[st][j], xr[j]), scale, acc[0]);
      } else {
#pragma unroll
        for (int t = 0; t < T; ++t) {
          uint32_t xp[16];
          const uint4* src = reinterpret_cast<const uint4*>(xs32 + (size_t)t * (H / 2) + (size_t)b * 16);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            uint4 v = src[q];
            xp[4 * q] = v.x; xp[4 * q + 1] = v.y; xp[4 * q + 2] = v.z; xp[4 * q + 3] = v.w;
          }
          acc[t] = fmaf(mx_block_dot(cw[st][j], xp), scale, acc[t]);
        }
      }
    }
    const int ri = i0 + 4 * wave + 2 * st + (r & 1);
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const float sum = sum16(acc[t]);
      const float up = __shfl_xor(sum, 32);
      if (r < 2 && c == 0) a_out[((size_t)slot * T + t) * I + ri] = silu(sum) * up;
    }
  }
}

// The 1-token gate/up with every load issued before the first wait: the
// slot's list entry, the activations (held in registers) and, once the expert
// is known, all of the workgroup's weights; only then are the activations
// staged in LDS.  The arithmetic is moe_gateup_kernel's for T = 1.
template <int NJ>
__global__ void __launch_bounds__(256) moe_gateup1_kernel(const uint16_t* __restrict__ x, int H, int I, int E,
                                                          int max_slots, const uint8_t* __restrict__ w13c,
                                                          const uint8_t* __restrict__ w13s,
                                                          const uint8_t* __restrict__ sh13c,
                                                          const uint8_t* __restrict__ sh13s,
                                                          const int32_t* __restrict__ expert_list,
                                                          float* __restrict__ a_out) {
  constexpr int XC = 2;   // 16-byte activation chunks per thread: H <= 8 * 256 * XC
  const int slot = blockIdx.y;
  int n_active = expert_list[0];
  const int e_slot = slot < max_slots - 1 ? expert_list[1 + slot] : -1;
  uint4 xv[XC];
#pragma unroll
  for (int q = 0; q < XC; ++q) {
    const int i = threadIdx.x + 256 * q;
    xv[q] = i < H / 8 ? ld16(x + 8 * i) : make_uint4(0, 0, 0, 0);
  }
  n_active = n_active < 0 ? 0 : (n_active > max_slots - 1 ? max_slots - 1 : n_active);
  const bool has_sh = sh13c != nullptr;
  const int i0 = blockIdx.x * 16;
  const uint8_t *C = nullptr, *S = nullptr;
  bool ok = false;
  if (slot < n_active) {
    ok = e_slot >= 0 && e_slot < E;
    if (ok) {
      C = w13c + (size_t)e_slot * ((size_t)2 * I * (H / 2));
      S = w13s + (size_t)e_slot * ((size_t)2 * I * (H / 32));
    }
  } else if (slot == n_active && has_sh) {
    ok = true;
    C = sh13c;
    S = sh13s;
  }
  if (!ok) {
    // inactive slot past the list: nothing to do; bad id: contribute zeros
    if (slot < n_active + (has_sh ? 1 : 0))
      for (int i = threadIdx.x; i < 16; i += 256) a_out[(size_t)slot * I + i0 + i] = 0.f;
    return;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane >> 4, c = lane & 15;
  const int NB = H / 32;
  const size_t rowc = H / 2, rows = H / 32;
  // the tile's scale bytes (16 gate rows, then 16 up rows, each set
  // contiguous) with 16-byte loads into LDS [gate | up][row][block]
  __shared__ __attribute__((aligned(16))) uint8_t lsc[2][16 * 16 * NJ];
  const int t16 = (int)threadIdx.x;
  const uint4 sv = t16 < 2 * NB ? ld16(S + ((size_t)(t16 / NB) * I + i0) * rows + (size_t)(t16 % NB) * 16)
                                : make_uint4(0, 0, 0, 0);
  uint4 cw[2][NJ];
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    const int ri = i0 + 4 * wave + 2 * st + (r & 1);
    const int row = (r < 2) ? ri : I + ri;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int b = c + 16 * j;
      cw[st][j] = (b < NB) ? ld16(C + row * rowc + (size_t)b * 16) : make_uint4(0, 0, 0, 0);
    }
  }
  issue_here();
  extern __shared__ __attribute__((aligned(16))) uint16_t xs[];
#pragma unroll
  for (int q = 0; q < XC; ++q) {
    const int i = threadIdx.x + 256 * q;
    if (i < H / 8) reinterpret_cast<uint4*>(xs)[i] = xv[q];
  }
  if (t16 < 2 * NB) *reinterpret_cast<uint4*>(&lsc[t16 / NB][(t16 % NB) * 16]) = sv;
  lds_barrier();
  const uint32_t* xs32 = reinterpret_cast<const uint32_t*>(xs);
  uint32_t xr[NJ][16];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int b = c + 16 * j;
#pragma unroll
    for (int d = 0; d < 16; ++d) xr[j][d] = (b < NB) ? xs32[b * 16 + d] : 0u;
  }
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    float acc = 0.f;
    const uint8_t* lrow = &lsc[r >> 1][(4 * wave + 2 * st + (r & 1)) * NB];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int b = c + 16 * j;
      if (b >= NB) continue;
      acc = fmaf(mx_block_dot(cw[st][j], xr[j]), e8m0_to_f32(lrow[b]), acc);
    }
    const int ri = i0 + 4 * wave + 2 * st + (r & 1);
    const float sum = sum16(acc);
    const float up = __shfl_xor(sum, 32);
    if (r < 2 && c == 0) a_out[(size_t)slot * I + ri] = silu(sum) * up;
  }
}

// ---------------------------------------------------------------- gate/up on the matrix cores

// Gate/up + SwiGLU for T tokens with v_mfma_f32_16x16x32_bf16: workgroup
// (i-tile, slot) computes the 16 gate rows i0.. and the 16 matching up rows
// as two 16 x 16 tiles (rows x tokens, columns past T are zero), each
// wavefront over a quarter of K.  The MFMA's 32-wide K slice is a
// permutation of K: lane (row, q) supplies 8 consecutive values of MX block
// 4 j + q of its quarter, decoded to bf16 together with the block scale (an
// exact power-of-two product), and the token columns take the same 8
// activations from LDS.  Products are exact; the fp32 sums differ from a
// sequential order only by rounding.  The four quarter sums are added in
// wavefront order.

template <int T, int NQ>   // NQ: groups of 4 MX blocks per wavefront quarter of K
__global__ void __launch_bounds__(256) moe_gateup_mfma_kernel(const uint16_t* __restrict__ x, int H, int I, int E,
                                                              int max_slots, const uint8_t* __restrict__ w13c,
                                                              const uint8_t* __restrict__ w13s,
                                                              const uint8_t* __restrict__ sh13c,
                                                              const uint8_t* __restrict__ sh13s,
                                                              const int32_t* __restrict__ expert_list,
                                                              float* __restrict__ a_out) {
  const int slot = blockIdx.y;
  int n_active = expert_list[0];
  n_active = n_active < 0 ? 0 : (n_active > max_slots - 1 ? max_slots - 1 : n_active);
  const bool has_sh = sh13c != nullptr;
  const int i0 = blockIdx.x * 16;
  const uint8_t *C, *S;
  if (!slot_expert(slot, n_active, has_sh, E, expert_list, w13c, w13s, sh13c, sh13s, (size_t)2 * I * (H / 2),
                   (size_t)2 * I * (H / 32), &C, &S)) {
    if (slot < n_active + (has_sh ? 1 : 0))
      for (int i = threadIdx.x; i < 16 * T; i += 256) a_out[((size_t)slot * T + i / 16) * I + i0 + (i % 16)] = 0.f;
    return;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row = lane & 15, q = lane >> 4;
  const int NB = H / 32;
  const int b0 = wave * 4 * NQ;   // first MX block of this wavefront's quarter
  const size_t rowc = H / 2, rows = H / 32;
  // weights of both tiles first: lane (row, q) owns block b0 + 4 j + q of its row
  // the tile's scale bytes (16 gate rows, then 16 up rows, each set
  // contiguous) with 16-byte loads, staged in LDS with the activations
  __shared__ __attribute__((aligned(16))) uint8_t lsc[2][16 * 16 * NQ];
  const int t16 = (int)threadIdx.x;
  const uint4 sv = t16 < 2 * NB ? ld16(S + ((size_t)(t16 / NB) * I + i0) * rows + (size_t)(t16 % NB) * 16)
                                : make_uint4(0, 0, 0, 0);
  uint4 cw[2][NQ];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = h * I + i0 + row;
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      const int b = b0 + 4 * j + q;
      cw[h][j] = b < NB ? ld16(C + r * rowc + (size_t)b * 16) : make_uint4(0, 0, 0, 0);
    }
  }
  extern __shared__ __attribute__((aligned(16))) uint16_t xs[];
  __shared__ float red[4][2][16][T];
  stage_to_lds<256, (T * 320 + 255) / 256>(x, xs, T * H / 8);
  if (t16 < 2 * NB) *reinterpret_cast<uint4*>(&lsc[t16 / NB][(t16 % NB) * 16]) = sv;
  __syncthreads();
  float sc[2][NQ];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      const int b = b0 + 4 * j + q;
      sc[h][j] = b < NB ? e8m0_to_f32(lsc[h][row * NB + b]) : 0.f;
    }
  f32x4_t dg = {0.f, 0.f, 0.f, 0.f}, du = {0.f, 0.f, 0.f, 0.f};
  const int col = row;   // B operand: lane (col, q)
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    const int b = b0 + 4 * j + q;
    const bool ok = b < NB;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      uint4 xv = make_uint4(0, 0, 0, 0);
      if (col < T && ok) xv = *reinterpret_cast<const uint4*>(xs + (size_t)col * H + b * 32 + m * 8);
      const bf16x8_t bx = __builtin_bit_cast(bf16x8_t, xv);
      const uint32_t wg = m == 0 ? cw[0][j].x : m == 1 ? cw[0][j].y : m == 2 ? cw[0][j].z : cw[0][j].w;
      const uint32_t wu = m == 0 ? cw[1][j].x : m == 1 ? cw[1][j].y : m == 2 ? cw[1][j].z : cw[1][j].w;
      dg = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp4x8_to_bf16x8(wg, sc[0][j]), bx, dg, 0, 0, 0);
      du = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp4x8_to_bf16x8(wu, sc[1][j]), bx, du, 0, 0, 0);
    }
  }
  // D: lane (col, q) holds rows 4 q .. 4 q + 3 of column col
  if (col < T) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      red[wave][0][4 * q + r][col] = dg[r];
      red[wave][1][4 * q + r][col] = du[r];
    }
  }
  __syncthreads();
  if (threadIdx.x < 16 * T) {
    const int rr = threadIdx.x % 16, t = threadIdx.x / 16;
    const float g = ((red[0][0][rr][t] + red[1][0][rr][t]) + red[2][0][rr][t]) + red[3][0][rr][t];
    const float u = ((red[0][1][rr][t] + red[1][1][rr][t]) + red[2][1][rr][t]) + red[3][1][rr][t];
    a_out[((size_t)slot * T + t) * I + i0 + rr] = silu(g) * u;
  }
}

// The same contraction for 5..16 tokens (a small batch or a longer draft),
// with the tokens as the MFMA's columns and four 16-row tiles per workgroup:
// each wavefront keeps its quarter of K of all T token columns in registers
// (loaded once from global memory, with the first tile's weights) and reuses
// it for the workgroup's tiles, whose gate/up rows stream one tile ahead; so
// the activations are read once per 64 rows instead of once per 16, and no
// LDS stage limits T.  The workgroup's scale bytes are staged in LDS once.
// Each tile's four quarter sums meet in LDS (double-buffered, one barrier per
// tile) and are added in wavefront order.
template <int NQ, int NTI>
__global__ void __launch_bounds__(256) moe_gateup_mfma_mt_kernel(const uint16_t* __restrict__ x, int T, int H, int I,
                                                                 int E, int max_slots, const uint8_t* __restrict__ w13c,
                                                                 const uint8_t* __restrict__ w13s,
                                                                 const uint8_t* __restrict__ sh13c,
                                                                 const uint8_t* __restrict__ sh13s,
                                                                 const int32_t* __restrict__ expert_list,
                                                                 const float* __restrict__ slot_w,
                                                                 float* __restrict__ a_out) {
  const int slot = blockIdx.y;
  int n_active = expert_list[0];
  const int e_slot = slot < max_slots - 1 ? expert_list[1 + slot] : -1;
  n_active = n_active < 0 ? 0 : (n_active > max_slots - 1 ? max_slots - 1 : n_active);
  const bool has_sh = sh13c != nullptr;
  const int ibase = blockIdx.x * 16 * NTI;
  // a routed slot serves only the tokens routed to it (nonzero weight in its
  // row of slot_w): the down stage reads no other column, so the others are
  // neither loaded nor meaningful (they come out 0); the shared expert serves all
  const int colw = (int)(threadIdx.x & 15);
  const float wcol = (slot < n_active && colw < T) ? slot_w[(size_t)slot * T + colw] : 1.0f;
  const uint8_t *C, *S;
  if (!slot_expert_pre(slot, n_active, has_sh, E, e_slot, w13c, w13s, sh13c, sh13s, (size_t)2 * I * (H / 2),
                       (size_t)2 * I * (H / 32), &C, &S)) {
    if (slot < n_active + (has_sh ? 1 : 0))
      for (int i = threadIdx.x; i < 16 * NTI * T; i += 256) {
        const int ii = ibase + i % (16 * NTI);
        if (ii < I) a_out[((size_t)slot * T + i / (16 * NTI)) * I + ii] = 0.f;
      }
    return;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row = lane & 15, q = lane >> 4;
  const int NB = H / 32;
  const int b0 = wave * 4 * NQ;
  const size_t rowc = H / 2, rows = H / 32;
  const int col = row;   // B operand: lane (col, q), token col
  // the scale bytes of all of the workgroup's rows, staged in LDS once with
  // 16-byte loads ([gate | up][row][block]; the tiles' rows are contiguous)
  constexpr int kMaxNB = 4 * 4 * NQ;   // blocks per row: H / 32 <= 16 NQ
  __shared__ __attribute__((aligned(16))) uint8_t ss[2][16 * NTI][kMaxNB];
  {
    const int nrow = (I - ibase < 16 * NTI ? I - ibase : 16 * NTI);
    const int n16 = nrow * NB / 16;   // NB % 16 == 0 is not assumed: bytes past n16 * 16 go one at a time
    for (int h = 0; h < 2; ++h) {
      const uint8_t* src = S + ((size_t)h * I + ibase) * rows;
      for (int c = threadIdx.x; c < n16; c += 256) {
        const uint4 v = ld16(src + (size_t)c * 16);
        const uint8_t* vb = reinterpret_cast<const uint8_t*>(&v);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int o = c * 16 + e;
          ss[h][o / NB][o % NB] = vb[e];
        }
      }
      for (int o = n16 * 16 + threadIdx.x; o < nrow * NB; o += 256) ss[h][o / NB][o % NB] = src[o];
    }
  }
  auto load_tile = [&](int i0, uint4 (&cw)[2][NQ]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = h * I + i0 + row;
#pragma unroll
      for (int j = 0; j < NQ; ++j) {
        const int b = b0 + 4 * j + q;
        cw[h][j] = b < NB ? ld16(C + r * rowc + (size_t)b * 16) : make_uint4(0, 0, 0, 0);
      }
    }
  };
  uint4 cw[2][NQ];
  load_tile(ibase, cw);
  const bool col_used = col < T && wcol != 0.f;
  uint4 xa[NQ][4];
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    const int b = b0 + 4 * j + q;
#pragma unroll
    for (int m = 0; m < 4; ++m)
      xa[j][m] = (col_used && b < NB) ? ld16(x + (size_t)col * H + b * 32 + m * 8) : make_uint4(0, 0, 0, 0);
  }
  // rows of 20 floats: the four rows 4q + r that one store touches fall 16
  // banks apart
  __shared__ float red[2][4][2][16][20];
  static_assert(WSX_MAX_T_MOE <= 20, "reduction tile columns");
#pragma unroll 1
  for (int ti = 0; ti < NTI; ++ti) {
    const int i0 = ibase + 16 * ti;
    if (i0 >= I) break;   // the same in every thread
    uint4 nw[2][NQ];
    if (ti + 1 < NTI && i0 + 16 < I) load_tile(i0 + 16, nw);
    issue_here();
    if (ti == 0) lds_barrier();   // the staged scales
    f32x4_t dg = {0.f, 0.f, 0.f, 0.f}, du = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      const int b = b0 + 4 * j + q;
      float sc[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) sc[h] = b < NB ? e8m0_to_f32(ss[h][16 * ti + row][b]) : 0.f;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const bf16x8_t bx = __builtin_bit_cast(bf16x8_t, xa[j][m]);
        const uint32_t wg = m == 0 ? cw[0][j].x : m == 1 ? cw[0][j].y : m == 2 ? cw[0][j].z : cw[0][j].w;
        const uint32_t wu = m == 0 ? cw[1][j].x : m == 1 ? cw[1][j].y : m == 2 ? cw[1][j].z : cw[1][j].w;
        dg = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp4x8_to_bf16x8(wg, sc[0]), bx, dg, 0, 0, 0);
        du = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp4x8_to_bf16x8(wu, sc[1]), bx, du, 0, 0, 0);
      }
    }
    float (*rb)[2][16][20] = red[ti & 1];
    if (col < T) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        rb[wave][0][4 * q + r][col] = dg[r];
        rb[wave][1][4 * q + r][col] = du[r];
      }
    }
    // LDS-only barrier: __syncthreads() would also wait for the next tile's
    // weight loads, which are meant to stay in flight across it
    lds_barrier();
    if ((int)threadIdx.x < 16 * T) {
      const int rr = threadIdx.x % 16, t = threadIdx.x / 16;
      const float g = ((rb[0][0][rr][t] + rb[1][0][rr][t]) + rb[2][0][rr][t]) + rb[3][0][rr][t];
      const float u = ((rb[0][1][rr][t] + rb[1][1][rr][t]) + rb[2][1][rr][t]) + rb[3][1][rr][t];
      a_out[((size_t)slot * T + t) * I + i0 + rr] = silu(g) * u;
    }
    if (ti + 1 < NTI) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int j = 0; j < NQ; ++j) cw[h][j] = nw[h][j];
    }
  }
}

// ---------------------------------------------------------------- down + combine + residual

template <int T, int NJD, bool ALDS>
__global__ void __launch_bounds__(256) moe_down_kernel(int H, int I, int E, int max_slots,
                                                       const uint8_t* __restrict__ w2c, const uint8_t* __restrict__ w2s,
                                                       const uint8_t* __restrict__ sh2c, const uint8_t* __restrict__ sh2s,
                                                       const int32_t* __restrict__ expert_list,
                                                       const float* __restrict__ slot_w, const float* __restrict__ a_in,
                                                       const uint16_t* __restrict__ residual, float* __restrict__ out_y,
                                                       uint16_t* __restrict__ out_h, uint16_t* __restrict__ out_h2) {
  int n_active = expert_list[0];
  n_active = n_active < 0 ? 0 : (n_active > max_slots - 1 ? max_slots - 1 : n_active);
  const bool has_sh = sh2c != nullptr;
  const int nslots = n_active + (has_sh ? 1 : 0);
  extern __shared__ __attribute__((aligned(16))) float as[];
  if constexpr (ALDS) {
    stage_to_lds<256, 7>(a_in, as, nslots * T * I / 4);
    __syncthreads();
  }
  const float* A = ALDS ? as : a_in;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane >> 3, c = lane & 7;
  const int n0 = blockIdx.x * 8;
  const int row = n0 + r;
  const int NBd = I / 32;
  const size_t rowc = I / 2, rows = I / 32;

  float acc[T];
#pragma unroll
  for (int t = 0; t < T; ++t) acc[t] = 0.f;
  for (int s = wave; s < nslots; s += 4) {
    const uint8_t *C, *S;
    if (!slot_expert(s, n_active, has_sh, E, expert_list, w2c, w2s, sh2c, sh2s, (size_t)H * (I / 2),
                     (size_t)H * (I / 32), &C, &S))
      continue;
    uint4 cw[NJD];
    uint32_t sb[NJD];
#pragma unroll
    for (int j = 0; j < NJD; ++j) {
      const int b = c + 8 * j;
      cw[j] = (b < NBd) ? ld16(C + row * rowc + (size_t)b * 16) : make_uint4(0, 0, 0, 0);
      sb[j] = (b < NBd) ? (uint32_t)S[row * rows + b] : 127u;
    }
    float wt[T];
#pragma unroll
    for (int t = 0; t < T; ++t) wt[t] = (s < n_active) ? slot_w[s * T + t] : 1.0f;
#pragma unroll
    for (int j = 0; j < NJD; ++j) {
      const int b = c + 8 * j;
      if (b >= NBd) continue;
      const float scale = e8m0_to_f32(sb[j]);
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const float* ap = A + ((size_t)s * T + t) * I + (size_t)b * 32;
        float av[32];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          float4 v = reinterpret_cast<const float4*>(ap)[q];
          av[4 * q] = v.x; av[4 * q + 1] = v.y; av[4 * q + 2] = v.z; av[4 * q + 3] = v.w;
        }
        acc[t] = fmaf(wt[t] * scale, mx_block_dot_f32(cw[j], av), acc[t]);
      }
    }
  }
  __shared__ float part[4][8][T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const float v = sum8(acc[t]);
    if (c == 0) part[wave][r][t] = v;
  }
  __syncthreads();
  if (threadIdx.x < 8 * T) {
    const int rr = threadIdx.x / T, t = threadIdx.x % T;
    const float y = ((part[0][rr][t] + part[1][rr][t]) + part[2][rr][t]) + part[3][rr][t];
    const size_t o = (size_t)t * H + n0 + rr;
    if (out_y) out_y[o] = y;
    if (residual) {
      const uint16_t h = f32_to_bf16_rne(bf16_bits_to_f32(residual[o]) + y);
      if (out_h) out_h[o] = h;
      if (out_h2) out_h2[o] = h;
    }
  }
}

// The 1-token down + combine + residual with every weight load issued first:
// each wavefront reads the list entries of its slots (s = wave + 4 i, i <
// MAXS) and issues all of those slots' weight loads, and only then are the
// activations staged in LDS.  The arithmetic and the summation order are
// moe_down_kernel's for T = 1.
template <int NJD, int MAXS>
__global__ void __launch_bounds__(256) moe_down1_kernel(int H, int I, int E, int max_slots,
                                                        const uint8_t* __restrict__ w2c, const uint8_t* __restrict__ w2s,
                                                        const uint8_t* __restrict__ sh2c, const uint8_t* __restrict__ sh2s,
                                                        const int32_t* __restrict__ expert_list,
                                                        const float* __restrict__ slot_w, const float* __restrict__ a_in,
                                                        const uint16_t* __restrict__ residual, float* __restrict__ out_y,
                                                        uint16_t* __restrict__ out_h, uint16_t* __restrict__ out_h2) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int n_active = expert_list[0];
  int eid[MAXS];
  float wt[MAXS];
#pragma unroll
  for (int i = 0; i < MAXS; ++i) {
    const int s = wave + 4 * i;
    eid[i] = s < max_slots - 1 ? expert_list[1 + s] : -1;
    wt[i] = s < max_slots - 1 ? slot_w[s] : 1.0f;
  }
  n_active = n_active < 0 ? 0 : (n_active > max_slots - 1 ? max_slots - 1 : n_active);
  const bool has_sh = sh2c != nullptr;
  const int nslots = n_active + (has_sh ? 1 : 0);
  const int r = lane >> 3, c = lane & 7;
  const int n0 = blockIdx.x * 8;
  const int row = n0 + r;
  const int NBd = I / 32;
  const size_t rowc = I / 2, rows = I / 32;
  uint4 cw[MAXS][NJD];
  uint32_t sb[MAXS][NJD];
  bool use[MAXS];
#pragma unroll
  for (int i = 0; i < MAXS; ++i) {
    const int s = wave + 4 * i;
    const uint8_t *C = nullptr, *S = nullptr;
    use[i] = false;
    if (s < n_active) {
      use[i] = eid[i] >= 0 && eid[i] < E;
      if (use[i]) {
        C = w2c + (size_t)eid[i] * ((size_t)H * (I / 2));
        S = w2s + (size_t)eid[i] * ((size_t)H * (I / 32));
      }
    } else if (s == n_active && has_sh) {
      use[i] = true;
      C = sh2c;
      S = sh2s;
      wt[i] = 1.0f;
    }
#pragma unroll
    for (int j = 0; j < NJD; ++j) {
      const int b = c + 8 * j;
      cw[i][j] = (use[i] && b < NBd) ? ld16(C + row * rowc + (size_t)b * 16) : make_uint4(0, 0, 0, 0);
      sb[i][j] = (use[i] && b < NBd) ? (uint32_t)S[row * rows + b] : 127u;
    }
  }
  issue_here();
  extern __shared__ __attribute__((aligned(16))) float as[];
  stage_to_lds<256, 7>(a_in, as, nslots * I / 4);
  __syncthreads();
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < MAXS; ++i) {
    if (!use[i]) continue;
    const int s = wave + 4 * i;
#pragma unroll
    for (int j = 0; j < NJD; ++j) {
      const int b = c + 8 * j;
      if (b >= NBd) continue;
      const float scale = e8m0_to_f32(sb[i][j]);
      const float* ap = as + (size_t)s * I + (size_t)b * 32;
      float av[32];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float4 v = reinterpret_cast<const float4*>(ap)[q];
        av[4 * q] = v.x; av[4 * q + 1] = v.y; av[4 * q + 2] = v.z; av[4 * q + 3] = v.w;
      }
      acc = fmaf(wt[i] * scale, mx_block_dot_f32(cw[i][j], av), acc);
    }
  }
  __shared__ float part[4][8];
  const float v = sum8(acc);
  if (c == 0) part[wave][r] = v;
  __syncthreads();
  if (threadIdx.x < 8) {
    const int rr = threadIdx.x;
    const float y = ((part[0][rr] + part[1][rr]) + part[2][rr]) + part[3][rr];
    const size_t o = (size_t)n0 + rr;
    if (out_y) out_y[o] = y;
    if (residual) {
      const uint16_t h = f32_to_bf16_rne(bf16_bits_to_f32(residual[o]) + y);
      if (out_h) out_h[o] = h;
      if (out_h2) out_h2[o] = h;
    }
  }
  (void)nslots;
}

// ---------------------------------------------------------------- down for several tokens

// Down + weighted combine + residual for 2..16 tokens, over expert-sorted
// token lists: the slots are the active experts in ascending id order, and
// slot s's tokens are those with a nonzero weight slot_w[s][t].  The shared
// expert, which serves every token, is split into ceil(T / 4) work slots of
// four tokens each (after the routed slots), so no wavefront carries all T
// tokens.  Workgroup (tile, g) owns rows n0 .. n0+31 of y and the work slots
// 4g .. 4g+3, one per wavefront.  A wavefront takes its slot's tokens two at a
// time, staging their activations in LDS (32-value blocks at a 36-float
// stride, so the eight block columns a load touches fall in distinct banks);
// lane (kg, rq) takes rows n0 + 4 rq .. +3 over the MX blocks kg, kg + 8, ...
// and forms the 4 rows x 2 tokens of partial sums from the same decoded
// weights, so the work follows the routed (slot, token) pairs, not slots x T.
// The E2M1 codes are decoded already multiplied by their power-of-two block
// scale (exact), so every product equals the oracle's.  Two tokens per pass
// keep the registers and the LDS stage small enough for three workgroups per
// CU.  Each slot's weighted contribution per (token, row) lands in LDS, the
// four wavefronts are added in slot order into the group's partial, and the
// last workgroup of the tile adds the groups in group order and the residual,
// so the result never depends on timing.
constexpr int kDnRows = 32;

// The products of one pass of the kernel below for its first TCX tokens
// (TCX <= 2): lane (kg, rq) over rows n0 + 4 rq .. +3 and MX blocks kg,
// kg + 8, ..., each token's sum in block, then element order.
template <int NKB, int TCX>
__device__ __forceinline__ void down_token_dots(const uint4 (&cw)[NKB][4], const uint8_t* ls, const float* aw,
                                                int lstride, int kg, int rq, int NB, float (&acc)[4][2]) {
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int j = 0; j < TCX; ++j) acc[r][j] = 0.f;
#pragma unroll
  for (int b = 0; b < NKB; ++b) {
    const int kb = kg + 8 * b;
    if (kb >= NB) continue;
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) {
      float av[TCX][8];
#pragma unroll
      for (int j = 0; j < TCX; ++j) {
        const float4* ap = reinterpret_cast<const float4*>(aw + j * lstride + kb * 36 + c4 * 8);
        const float4 v0 = ap[0], v1 = ap[1];
        av[j][0] = v0.x; av[j][1] = v0.y; av[j][2] = v0.z; av[j][3] = v0.w;
        av[j][4] = v1.x; av[j][5] = v1.y; av[j][6] = v1.z; av[j][7] = v1.w;
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t wd = c4 == 0 ? cw[b][r].x : c4 == 1 ? cw[b][r].y : c4 == 2 ? cw[b][r].z : cw[b][r].w;
        const float sc = e8m0_to_f32(ls[(4 * rq + r) * NB + kb]);
        const f32x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd, sc, 0);
        const f32x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd, sc, 1);
        const f32x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd, sc, 2);
        const f32x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd, sc, 3);
#pragma unroll
        for (int j = 0; j < TCX; ++j) {
          float v = acc[r][j];
          v = fmaf(p0.x, av[j][0], v);
          v = fmaf(p0.y, av[j][1], v);
          v = fmaf(p1.x, av[j][2], v);
          v = fmaf(p1.y, av[j][3], v);
          v = fmaf(p2.x, av[j][4], v);
          v = fmaf(p2.y, av[j][5], v);
          v = fmaf(p3.x, av[j][6], v);
          v = fmaf(p3.y, av[j][7], v);
          acc[r][j] = v;
        }
      }
    }
  }
}

__device__ __forceinline__ int dpos(int i) { return (i >> 5) * 36 + (i & 31); }

int down_sparse_groups(int T, int k) { return (T * k + (T + 3) / 4 + 3) / 4; }

template <int NKB>
__global__ void __launch_bounds__(256) moe_down_sparse_kernel(
    int T, int H, int I, int E, int max_slots, const uint8_t* __restrict__ w2c, const uint8_t* __restrict__ w2s,
    const uint8_t* __restrict__ sh2c, const uint8_t* __restrict__ sh2s, const int32_t* __restrict__ expert_list,
    const float* __restrict__ slot_w, const float* __restrict__ a_in, const uint16_t* __restrict__ residual,
    float* __restrict__ out_y, uint16_t* __restrict__ out_h, uint16_t* __restrict__ out_h2, float* part,
    unsigned* counters) {
  constexpr int TC = 2;   // tokens per pass
  const int s = 4 * (int)blockIdx.y + (int)(threadIdx.x >> 6);   // work slot
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // the list entry, the active count and the slot's row of weights in one
  // round trip (the row is only used if s turns out to be a routed slot)
  int n_active = expert_list[0];
  const int e_slot = s < max_slots - 1 ? expert_list[1 + s] : -1;
  const float wrow = (s < max_slots - 1 && lane < T) ? slot_w[s * T + lane] : 0.f;
  n_active = n_active < 0 ? 0 : (n_active > max_slots - 1 ? max_slots - 1 : n_active);
  const bool has_sh = sh2c != nullptr;
  const int kg = lane & 7, rq = lane >> 3;
  const int n0 = blockIdx.x * kDnRows;
  const int g = blockIdx.y;
  const int NB = I / 32;
  const int lstride = NB * 36;   // floats per token row in LDS
  extern __shared__ __attribute__((aligned(16))) float as[];   // [4][TC][lstride]
  __shared__ float yw[4][WSX_MAX_T_MOE][kDnRows];
  __shared__ __attribute__((aligned(16))) uint8_t lsc[4][kDnRows * 32];   // per wavefront: [row][block], I <= 1024
  __shared__ int flag;
  float* aw = as + (size_t)wave * TC * lstride;
  for (int i = lane; i < WSX_MAX_T_MOE * kDnRows; i += 64) yw[wave][i / kDnRows][i % kDnRows] = 0.f;
  // routed slot s < n_active, or part v = s - n_active of the shared expert
  // (tokens 4 v .. 4 v + 3), whose activations sit in slot n_active
  const bool shared_part = has_sh && s >= n_active && s - n_active < (T + 3) / 4;
  const uint8_t *C = nullptr, *S = nullptr;
  bool active = false;
  if (s < n_active) {
    active = e_slot >= 0 && e_slot < E;
    if (active) {
      C = w2c + (size_t)e_slot * ((size_t)H * (I / 2));
      S = w2s + (size_t)e_slot * ((size_t)H * (I / 32));
    }
  } else if (shared_part) {
    active = true;
    C = sh2c;
    S = sh2s;
  }
  const int as_slot = s < n_active ? s : n_active;
  if (active) {
    const size_t rowc = I / 2, rows = I / 32;
    // the tile's E8M0 scale bytes (32 contiguous rows of NB bytes) into this
    // wavefront's LDS with 16-byte loads, issued before the codes
    uint8_t* ls = lsc[wave];
    const int ns16 = kDnRows * NB / 16;
    const uint4 sv = lane < ns16 ? ld16(S + (size_t)n0 * rows + (size_t)lane * 16) : make_uint4(0, 0, 0, 0);
    uint4 cw[NKB][4];
#pragma unroll
    for (int b = 0; b < NKB; ++b) {
      const int kb = kg + 8 * b;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = n0 + 4 * rq + r;
        cw[b][r] = kb < NB ? ld16(C + row * rowc + (size_t)kb * 16) : make_uint4(0, 0, 0, 0);
      }
    }
    if (lane < ns16) *reinterpret_cast<uint4*>(ls + lane * 16) = sv;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // the slot's token list: lane t < T holds token t's weight
    const int v4 = 4 * (s - n_active);
    const float wl = lane < T ? (s < n_active ? wrow : 1.0f) : 0.f;
    unsigned long long tm = s < n_active ? __ballot(lane < T && wl != 0.f) : __ballot(lane >= v4 && lane < v4 + 4 && lane < T);
    while (tm) {
      int tok[TC];
      float wt[TC];
#pragma unroll
      for (int j = 0; j < TC; ++j) {
        tok[j] = tm ? (int)__builtin_ctzll(tm) : -1;
        wt[j] = tok[j] >= 0 ? readlane_f(wl, tok[j]) : 0.f;
        tm &= tm - 1;
      }
      // these tokens' activations -> LDS (32-value blocks at a 36-float
      // stride), every load issued before the first store (I <= 256 NKB)
      const int nq = I / 4;
      float4 av4[TC][NKB];
#pragma unroll
      for (int j = 0; j < TC; ++j) {
        const float4* src =
            reinterpret_cast<const float4*>(a_in + ((size_t)as_slot * T + (tok[j] < 0 ? 0 : tok[j])) * I);
#pragma unroll
        for (int m = 0; m < NKB; ++m) {
          const int q4 = lane + 64 * m;
          av4[j][m] = (tok[j] >= 0 && q4 < nq) ? src[q4] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
#pragma unroll
      for (int j = 0; j < TC; ++j)
#pragma unroll
        for (int m = 0; m < NKB; ++m) {
          const int q4 = lane + 64 * m;
          if (tok[j] >= 0 && q4 < nq) *reinterpret_cast<float4*>(aw + j * lstride + dpos(4 * q4)) = av4[j][m];
        }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      // a pass with one token (most routed slots of a verify pass) takes
      // only that token's products
      float acc[4][TC];
      if (tok[1] >= 0) {
        down_token_dots<NKB, 2>(cw, ls, aw, lstride, kg, rq, NB, acc);
      } else {
        down_token_dots<NKB, 1>(cw, ls, aw, lstride, kg, rq, NB, acc);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r][1] = 0.f;
      }
      // weighted row sums (fixed DPP tree over the 8 lanes of a row group);
      // each (token, row) of this slot is written by one lane
#pragma unroll
      for (int j = 0; j < TC; ++j) {
        if (tok[j] < 0) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float v = sum8(acc[r][j] * wt[j]);
          if (kg == 0 && tok[j] >= 0) yw[wave][tok[j]][4 * rq + r] = v;
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < T * kDnRows; i += 256) {
    const int t = i / kDnRows, rr = i % kDnRows;
    const float v = ((yw[0][t][rr] + yw[1][t][rr]) + yw[2][t][rr]) + yw[3][t][rr];
    st_dev(part + ((size_t)g * T + t) * H + n0 + rr, v);
  }
  if (!last_block_arrived(counters + blockIdx.x * 16, gridDim.y, &flag)) return;
  for (int i = threadIdx.x; i < T * kDnRows; i += 256) {
    const int t = i / kDnRows, rr = i % kDnRows;
    const float y = sum_group_partials(part, (int)gridDim.y, T, H, t, n0 + rr);
    const size_t o = (size_t)t * H + n0 + rr;
    if (out_y) out_y[o] = y;
    if (residual) {
      const uint16_t h = f32_to_bf16_rne(bf16_bits_to_f32(residual[o]) + y);
      if (out_h) out_h[o] = h;
      if (out_h2) out_h2[o] = h;
    }
  }
}

// ---------------------------------------------------------------- launchers

bool experts_shape_supported(int H, int I) {
  if (H % 32 || I % 32 || H > 8192 || I > 2048) return false;
  const int nj = (H / 32 + 15) / 16, njd = (I / 32 + 7) / 8;
  const bool ok_nj = nj == 1 || nj == 2 || nj == 4 || nj == 5 || nj == 8 || nj == 16;
  const bool ok_njd = njd == 1 || njd == 2 || njd == 3 || njd == 4 || njd == 6 || njd == 8;
  return ok_nj && ok_njd;
}

template <int T>
static hipError_t launch_gateup_t(const uint16_t* x, int H, int I, int E, int max_slots, const uint8_t* w13c,
                                  const uint8_t* w13s, const uint8_t* sh13c, const uint8_t* sh13s,
                                  const int32_t* el, float* a, hipStream_t st) {
  const int nj = (H / 32 + 15) / 16;
  dim3 grid(I / 16, max_slots);
  const size_t lds = (size_t)T * H * 2;
#define WSX_G_CASE(N)                                                                                    \
  case N:                                                                                                \
    moe_gateup_kernel<T, N><<<grid, 256, lds, st>>>(x, H, I, E, max_slots, w13c, w13s, sh13c, sh13s, el, a); \
    break;
  switch (nj) {
    WSX_G_CASE(1) WSX_G_CASE(2) WSX_G_CASE(4) WSX_G_CASE(5) WSX_G_CASE(8) WSX_G_CASE(16)
    default: return hipErrorInvalidValue;
  }
#undef WSX_G_CASE
  return hipGetLastError();
}

template <int T>
static hipError_t launch_gateup_mfma_t(const uint16_t* x, int H, int I, int E, int max_slots, const uint8_t* w13c,
                                       const uint8_t* w13s, const uint8_t* sh13c, const uint8_t* sh13s,
                                       const int32_t* el, float* a, hipStream_t st) {
  const int nq = (H / 32 + 15) / 16;   // four wavefronts x 4 NQ blocks cover H / 32
  dim3 grid(I / 16, max_slots);
  const size_t lds = (size_t)T * H * 2;
#define WSX_GM_CASE(N)                                                                                           \
  case N:                                                                                                        \
    moe_gateup_mfma_kernel<T, N><<<grid, 256, lds, st>>>(x, H, I, E, max_slots, w13c, w13s, sh13c, sh13s, el, a); \
    break;
  switch (nq) {
    WSX_GM_CASE(1) WSX_GM_CASE(2) WSX_GM_CASE(4) WSX_GM_CASE(5) WSX_GM_CASE(8) WSX_GM_CASE(16)
    default: return hipErrorInvalidValue;
  }
#undef WSX_GM_CASE
  return hipGetLastError();
}

static hipError_t launch_gateup_g(const uint16_t* x, int T, int H, int I, int E, int max_slots, const uint8_t* w13c,
                                  const uint8_t* w13s, const uint8_t* sh13c, const uint8_t* sh13s, const int32_t* el,
                                  const float* sw, float* a, hipStream_t st) {
  const int nq = (H / 32 + 15) / 16;
  constexpr int kTiles = 4;   // 16-row tiles per workgroup
  dim3 grid((I / 16 + kTiles - 1) / kTiles, max_slots);
#define WSX_GG_CASE(N)                                                                                              \
  case N:                                                                                                           \
    moe_gateup_mfma_mt_kernel<N, kTiles><<<grid, 256, 0, st>>>(x, T, H, I, E, max_slots, w13c, w13s, sh13c, sh13s, \
                                                               el, sw, a);                                          \
    break;
  switch (nq) {
    WSX_GG_CASE(1) WSX_GG_CASE(2) WSX_GG_CASE(4) WSX_GG_CASE(5) WSX_GG_CASE(8) WSX_GG_CASE(16)
    default: return hipErrorInvalidValue;
  }
#undef WSX_GG_CASE
  return hipGetLastError();
}

hipError_t launch_gateup(const uint16_t* x, int T, int H, int I, int E, int k, const uint8_t* w13c,
                         const uint8_t* w13s, const uint8_t* sh13c, const uint8_t* sh13s, const int32_t* el,
                         const float* sw, float* a, hipStream_t st) {
  const int max_slots = T * k + 1;
  if (T > WSX_MAX_T) return launch_gateup_g(x, T, H, I, E, max_slots, w13c, w13s, sh13c, sh13s, el, sw, a, st);
  if (T >= 2) {
    switch (T) {
      case 2: return launch_gateup_mfma_t<2>(x, H, I, E, max_slots, w13c, w13s, sh13c, sh13s, el, a, st);
      case 3: return launch_gateup_mfma_t<3>(x, H, I, E, max_slots, w13c, w13s, sh13c, sh13s, el, a, st);
      case 4: return launch_gateup_mfma_t<4>(x, H, I, E, max_slots, w13c, w13s, sh13c, sh13s, el, a, st);
    }
  }
  if (T == 1 && H <= 8 * 256 * 2) {
    const int nj = (H / 32 + 15) / 16;
    dim3 grid(I / 16, max_slots);
    const size_t lds = (size_t)H * 2;
#define WSX_G1_CASE(N)                                                                                     \
  case N:                                                                                                  \
    moe_gateup1_kernel<N><<<grid, 256, lds, st>>>(x, H, I, E, max_slots, w13c, w13s, sh13c, sh13s, el, a); \
    return hipGetLastError();
    switch (nj) {
      WSX_G1_CASE(1) WSX_G1_CASE(2) WSX_G1_CASE(4) WSX_G1_CASE(5) WSX_G1_CASE(8) WSX_G1_CASE(16)
      default: return hipErrorInvalidValue;
    }
#undef WSX_G1_CASE
  }
  switch (T) {
    case 1: return launch_gateup_t<1>(x, H, I, E, max_slots, w13c, w13s, sh13c, sh13s, el, a, st);
    case 2: return launch_gateup_t<2>(x, H, I, E, max_slots, w13c, w13s, sh13c, sh13s, el, a, st);
    case 3: return launch_gateup_t<3>(x, H, I, E, max_slots, w13c, w13s, sh13c, sh13s, el, a, st);
    case 4: return launch_gateup_t<4>(x, H, I, E, max_slots, w13c, w13s, sh13c, sh13s, el, a, st);
  }
  return hipErrorInvalidValue;
}

constexpr size_t kDownLdsLimit = 64 * 1024;

template <int T, bool ALDS>
static hipError_t launch_down_t(int H, int I, int E, int max_slots, const uint8_t* w2c, const uint8_t* w2s,
                                const uint8_t* sh2c, const uint8_t* sh2s, const int32_t* el, const float* sw,
                                const float* a, const uint16_t* res, float* y, uint16_t* h, uint16_t* h2,
                                hipStream_t st) {
  const int njd = (I / 32 + 7) / 8;
  const size_t lds = ALDS ? (size_t)max_slots * T * I * 4 : 0;
#define WSX_D_CASE(N)                                                                                             \
  case N:                                                                                                         \
    moe_down_kernel<T, N, ALDS><<<H / 8, 256, lds, st>>>(H, I, E, max_slots, w2c, w2s, sh2c, sh2s, el, sw, a, res, \
                                                          y, h, h2);                                               \
    break;
  switch (njd) {
    WSX_D_CASE(1) WSX_D_CASE(2) WSX_D_CASE(3) WSX_D_CASE(4) WSX_D_CASE(6) WSX_D_CASE(8)
    default: return hipErrorInvalidValue;
  }
#undef WSX_D_CASE
  return hipGetLastError();
}

int down_groups(int max_slots) { return (max_slots + 3) / 4; }
size_t down_grouped_lds(int T, int I) { return (size_t)4 * T * (I / 32) * 36 * 4; }
bool down_grouped_ok(int T, int H, int I) {
  return T >= 2 && H % kDnRows == 0 && I / 32 <= 32 && down_grouped_lds(T, I) <= 64 * 1024;
}

static hipError_t launch_down_sparse(int T, int H, int I, int E, int max_slots, const uint8_t* w2c, const uint8_t* w2s,
                                     const uint8_t* sh2c, const uint8_t* sh2s, const int32_t* el, const float* sw,
                                     const float* a, const uint16_t* res, float* y, uint16_t* h, uint16_t* h2,
                                     float* part, unsigned* counters, hipStream_t st) {
  const int nkb = (I / 32 + 7) / 8;
  dim3 grid(H / kDnRows, down_sparse_groups(T, max_slots > 1 ? (max_slots - 1) / T : 0));
  const size_t lds = down_grouped_lds(2, I);
#define WSX_DS_CASE(N)                                                                                          \
  case N:                                                                                                       \
    moe_down_sparse_kernel<N><<<grid, 256, lds, st>>>(T, H, I, E, max_slots, w2c, w2s, sh2c, sh2s, el, sw, a,  \
                                                      res, y, h, h2, part, counters);                           \
    break;
  switch (nkb) {
    WSX_DS_CASE(1) WSX_DS_CASE(2) WSX_DS_CASE(3) WSX_DS_CASE(4)
    default: return hipErrorInvalidValue;
  }
#undef WSX_DS_CASE
  return hipGetLastError();
}

hipError_t launch_down(int T, int H, int I, int E, int k, const uint8_t* w2c, const uint8_t* w2s,
                       const uint8_t* sh2c, const uint8_t* sh2s, const int32_t* el, const float* sw, const float* a,
                       const uint16_t* res, float* y, uint16_t* h, uint16_t* h2, float* part, unsigned* counters,
                       hipStream_t st) {
  const int max_slots = T * k + 1;
  // 2..16 tokens: expert-sorted token lists
  if (T >= 2 && part && counters && down_grouped_ok(2, H, I))
    return launch_down_sparse(T, H, I, E, max_slots, w2c, w2s, sh2c, sh2s, el, sw, a, res, y, h, h2, part, counters, st);
  if (T > WSX_MAX_T) return hipErrorInvalidValue;
  const bool alds = (size_t)max_slots * T * I * 4 <= kDownLdsLimit;
  if (T == 1 && alds && max_slots <= 12 && (size_t)max_slots * I / 4 <= (size_t)256 * 7) {
    const int njd = (I / 32 + 7) / 8;
    const size_t lds = (size_t)max_slots * I * 4;
#define WSX_D1_CASE(N)                                                                                           \
  case N:                                                                                                        \
    moe_down1_kernel<N, 3><<<H / 8, 256, lds, st>>>(H, I, E, max_slots, w2c, w2s, sh2c, sh2s, el, sw, a, res, y, h, \
                                                    h2);                                                          \
    return hipGetLastError();
    switch (njd) {
      WSX_D1_CASE(1) WSX_D1_CASE(2) WSX_D1_CASE(3) WSX_D1_CASE(4) WSX_D1_CASE(6) WSX_D1_CASE(8)
      default: return hipErrorInvalidValue;
    }
#undef WSX_D1_CASE
  }
#define WSX_DT(TV)                                                                                           \
  case TV:                                                                                                   \
    return alds ? launch_down_t<TV, true>(H, I, E, max_slots, w2c, w2s, sh2c, sh2s, el, sw, a, res, y, h, h2, st) \
                : launch_down_t<TV, false>(H, I, E, max_slots, w2c, w2s, sh2c, sh2s, el, sw, a, res, y, h, h2, st);
  switch (T) { WSX_DT(1) WSX_DT(2) WSX_DT(3) WSX_DT(4) }
#undef WSX_DT
  return hipErrorInvalidValue;
}

}  // namespace wsx
