// W4A8 routed + shared SwiGLU experts on gfx950: MXFP4 weights contracted with
// MXFP8 (E4M3) activations on the matrix cores.
//
// [saipien] "Why one user waits on weights": the baseline of the DGX Spark
// runs was the "W4A8" recipe (MXFP4 expert kernels, 8-bit activations).  Here
// the activations are OCP MXFP8: per 32 consecutive elements along the
// contraction, X = floor(log2 max|v|) - 8 (clamped to [-127, 127], -127 for an
// all-zero block) and element = RNE_E4M3(clamp(v / 2^X, +-448)).
//
// v_mfma_scale_f32_16x16x128_f8f6f4 takes the weights' E2M1 codes and E8M0
// block scales exactly as they are stored, so no weight is decoded on the
// VALU: a lane's 16-byte load of one row's MX block is its A operand.  Per 128
// elements of K (one matrix-core step):
//   A (16 rows x 128, FP4):  lane (row r, group g) holds MX block g of row r:
//                            its 16 stored bytes, and that block's scale byte;
//   B (128 x 16 cols, FP8):  lane (col c, group g) holds elements 16g..16g+15
//                            in its first four registers and 64+16g..64+16g+15
//                            in the last four, and the scale of block g of
//                            column c;
//   D (16 x 16, fp32):       lane (col c, group g) holds rows 4g..4g+3.
// The columns are tokens (T <= 16); columns past T are zero.
//
// Two launches per layer, driven by the device-side expert list (above 4
// tokens a third one first quantizes the T input rows once, and the gate/up
// workgroups copy those bytes instead of quantizing):
//   gate/up  grid (I/32, T*k+1): workgroup (tile, slot) quantizes the T input
//            rows into LDS, its four wavefronts take 16 gate rows, 16 more
//            gate rows and the two matching sets of 16 up rows, and it writes
//            a = silu(g) * u for the tile's 32 values (one MX block per token)
//            already quantized: E4M3 codes [slots][T][I] and E8M0 scales
//            [slots][T][I/32] (optionally also the binary32 a);
//   down     grid (H/16): workgroup owns 16 output rows; wavefront w takes
//            slots w, w+4, ..., each slot's tile weighted per token column,
//            then the four partials are added in wavefront order with the
//            residual: the order never depends on timing.
#include "wsx_device.h"
#include "partials_device.h"
#include "wsx_internal.h"

namespace wsx {

namespace {

typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef float v4f_t __attribute__((ext_vector_type(4)));

constexpr int kFmtFp8 = 0;   // matrix-core operand formats
constexpr int kFmtFp4 = 4;

// 2^n as a binary32 for n in [-127, 127] (2^-127 is subnormal).
__device__ __forceinline__ float pow2i(int n) {
  return n >= -126 ? __uint_as_float((uint32_t)(n + 127) << 23) : __uint_as_float(0x00400000u);
}

// The MXFP8 block exponent of a block whose largest magnitude is amax.
__device__ __forceinline__ int mx_block_exp(float amax) {
  const int e = (int)((__float_as_uint(amax) >> 23) & 0xFFu);
  if (e == 0) return -127;                       // zero (or a subnormal maximum)
  const int X = e - 127 - 8;
  return X < -127 ? -127 : (X > 127 ? 127 : X);
}

__device__ __forceinline__ float sat448(float v) { return fminf(fmaxf(v, -448.0f), 448.0f); }

// Four scaled values -> four E4M3 codes (element order kept), round to nearest even.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(a), sat448(b), 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(sat448(c), sat448(d), lo, true);
}

// One MX block of 32 bf16 values (four 16-byte chunks) -> 32 E4M3 codes (two
// 16-byte chunks) and the E8M0 scale byte.
__device__ __forceinline__ void mx_quant_bf16_block(const uint4 (&in)[4], uint4 (&out)[2], uint32_t& sbyte) {
  float v[32];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t w[4] = {in[q].x, in[q].y, in[q].z, in[q].w};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      v[8 * q + 2 * d] = __uint_as_float(w[d] << 16);
      v[8 * q + 2 * d + 1] = __uint_as_float(w[d] & 0xFFFF0000u);
    }
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const int X = mx_block_exp(amax);
  const float m = pow2i(-X);
  uint32_t c[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) c[i] = e4m3x4(v[4 * i] * m, v[4 * i + 1] * m, v[4 * i + 2] * m, v[4 * i + 3] * m);
  out[0] = make_uint4(c[0], c[1], c[2], c[3]);
  out[1] = make_uint4(c[4], c[5], c[6], c[7]);
  sbyte = (uint32_t)(X + 127);
}

__global__ void __launch_bounds__(256) act_quant_kernel(const uint16_t* __restrict__ x, int nblocks,
                                                        uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b >= nblocks) return;
  uint4 in[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) in[q] = ld16(x + (size_t)b * 32 + 8 * q);
  uint4 out[2];
  uint32_t sb;
  mx_quant_bf16_block(in, out, sb);
  *reinterpret_cast<uint4*>(codes + (size_t)b * 32) = out[0];
  *reinterpret_cast<uint4*>(codes + (size_t)b * 32 + 16) = out[1];
  scales[b] = (uint8_t)sb;
}

// Resolve slot -> (codes, scales) of its expert, as the bf16 path does.
__device__ __forceinline__ bool w4a8_slot(int slot, int n_active, bool has_sh, int E, const int32_t* el,
                                          const uint8_t* wc, const uint8_t* ws_, const uint8_t* shc,
                                          const uint8_t* shs, size_t c_stride, size_t s_stride, const uint8_t** C,
                                          const uint8_t** S) {
  if (slot < n_active) {
    const int e = el[1 + slot];
    if (e < 0 || e >= E) return false;
    *C = wc + (size_t)e * c_stride;
    *S = ws_ + (size_t)e * s_stride;
    return true;
  }
  if (slot == n_active && has_sh) { *C = shc; *S = shs; return true; }
  return false;
}

// The B operand of one 128-element step for token column c of an MXFP8 row
// (codes at `row`, scale bytes at `srow`, K elements): lane group g takes
// elements 16g.. and 64+16g.. of the step and the scale of the step's block g.
__device__ __forceinline__ void b_operand(const uint8_t* row, const uint8_t* srow, int K, int step, int g,
                                          v8i_t& b, int& sb) {
  const int k0 = step * 128 + 16 * g, k1 = k0 + 64;
  const uint4 lo = k0 < K ? *reinterpret_cast<const uint4*>(row + k0) : make_uint4(0, 0, 0, 0);
  const uint4 hi = k1 < K ? *reinterpret_cast<const uint4*>(row + k1) : make_uint4(0, 0, 0, 0);
  b = v8i_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  const int kb = 4 * step + g;
  sb = kb < K / 32 ? (int)srow[kb] : 127;
}

// ---------------------------------------------------------------- gate/up + SwiGLU + quantize a

template <int NS>   // matrix-core steps of 128 covering H
__global__ void __launch_bounds__(256) moe_gateup_w4a8_kernel(
    const uint16_t* __restrict__ x, int T, int H, int I, int E, int max_slots, const uint8_t* __restrict__ w13c,
    const uint8_t* __restrict__ w13s, const uint8_t* __restrict__ sh13c, const uint8_t* __restrict__ sh13s,
    const int32_t* __restrict__ el, uint8_t* __restrict__ aq, uint8_t* __restrict__ aqs, float* __restrict__ act,
    const uint8_t* __restrict__ xin) {
  const int slot = blockIdx.y;
  int n_active = el[0];
  n_active = n_active < 0 ? 0 : (n_active > max_slots - 1 ? max_slots - 1 : n_active);
  const bool has_sh = sh13c != nullptr;
  const int i0 = blockIdx.x * 32;
  const int NI = I / 32;
  const uint8_t *C, *S;
  if (!w4a8_slot(slot, n_active, has_sh, E, el, w13c, w13s, sh13c, sh13s, (size_t)2 * I * (H / 2),
                 (size_t)2 * I * (H / 32), &C, &S)) {
    // a bad id contributes zeros (codes 0, scale byte 0); slots past the list: nothing
    if (slot < n_active + (has_sh ? 1 : 0)) {
      for (int i = threadIdx.x; i < 32 * T; i += 256) {
        const size_t o = ((size_t)slot * T + i / 32) * I + i0 + (i % 32);
        aq[o] = 0;
        if (act) act[o] = 0.f;
        if (i % 32 == 0) aqs[((size_t)slot * T + i / 32) * NI + i0 / 32] = 0;
      }
    }
    return;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int NB = H / 32;
  // weights first: wavefront w takes rows (w >> 1) * I + i0 + 16 (w & 1) + r16
  const int row = (wave >> 1) * I + i0 + 16 * (wave & 1) + r16;
  // the weights' scale bytes (32 gate rows, then 32 up rows, each set
  // contiguous) with 16-byte loads, staged in LDS beside the activations
  __shared__ __attribute__((aligned(16))) uint8_t lsc[2][32 * 4 * NS];
  uint4 sv[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int t16 = (int)threadIdx.x + 256 * u;
    sv[u] = t16 < 4 * NB ? ld16(S + ((size_t)(t16 / (2 * NB)) * I + i0) * NB + (size_t)(t16 % (2 * NB)) * 16)
                         : make_uint4(0, 0, 0, 0);
  }
  uint4 cw[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int b = 4 * s + g;
    cw[s] = b < NB ? ld16(C + (size_t)row * (H / 2) + (size_t)b * 16) : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int t16 = (int)threadIdx.x + 256 * u;
    if (t16 < 4 * NB) *reinterpret_cast<uint4*>(&lsc[t16 / (2 * NB)][(t16 % (2 * NB)) * 16]) = sv[u];
  }
  // the T input rows, quantized into LDS: codes [T][H], scales [T][NB]
  extern __shared__ __attribute__((aligned(16))) uint8_t sm[];
  uint8_t* xq = sm;
  uint8_t* xs = sm + (size_t)T * H;
  if (xin) {
    // quantized once for the layer (the same blocks, the same bytes), laid
    // out as in LDS: copied with 16-byte loads, four per thread in flight
    const int nb = T * H + T * NB, n16 = nb / 16;
    for (int c0 = 0; c0 < n16; c0 += 4 * 256) {
      uint4 v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = c0 + (int)threadIdx.x + 256 * j;
        v[j] = c < n16 ? ld16(xin + (size_t)c * 16) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = c0 + (int)threadIdx.x + 256 * j;
        if (c < n16) *reinterpret_cast<uint4*>(sm + (size_t)c * 16) = v[j];
      }
    }
    for (int i = 16 * n16 + (int)threadIdx.x; i < nb; i += 256) sm[i] = xin[i];
  }
  for (int b = xin ? T * NB : (int)threadIdx.x; b < T * NB; b += 256) {
    const int t = b / NB, kb = b - t * NB;
    uint4 in[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) in[q] = ld16(x + (size_t)t * H + (size_t)kb * 32 + 8 * q);
    uint4 out[2];
    uint32_t sb;
    mx_quant_bf16_block(in, out, sb);
    *reinterpret_cast<uint4*>(xq + (size_t)t * H + kb * 32) = out[0];
    *reinterpret_cast<uint4*>(xq + (size_t)t * H + kb * 32 + 16) = out[1];
    xs[t * NB + kb] = (uint8_t)sb;
  }
  __syncthreads();
  int sw[NS];
  const uint8_t* lrow = &lsc[wave >> 1][(16 * (wave & 1) + r16) * NB];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int b = 4 * s + g;
    sw[s] = b < NB ? (int)lrow[b] : 127;
  }
  v4f_t acc = {0.f, 0.f, 0.f, 0.f};
  const bool col = r16 < T;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    v8i_t b = {0, 0, 0, 0, 0, 0, 0, 0};
    int sb = 127;
    if (col) b_operand(xq + (size_t)r16 * H, xs + r16 * NB, H, s, g, b, sb);
    const v8i_t a = {(int)cw[s].x, (int)cw[s].y, (int)cw[s].z, (int)cw[s].w, 0, 0, 0, 0};
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, kFmtFp4, kFmtFp8, 0, sw[s], 0, sb);
  }
  __shared__ float tile[2][32][17];   // [gate | up][value][token]
  if (col) {
#pragma unroll
    for (int q = 0; q < 4; ++q) tile[wave >> 1][16 * (wave & 1) + 4 * g + q][r16] = acc[q];
  }
  __syncthreads();
  // a = silu(g) * u for (value v, token t); each 32-lane half of a wavefront
  // holds one token's block: its maximum, exponent and codes
  const int v = threadIdx.x & 31;
  for (int t0 = 0; t0 < T; t0 += 8) {
    const int t = t0 + (threadIdx.x >> 5);
    const bool ok = t < T;
    const float av = ok ? silu(tile[0][v][t]) * tile[1][v][t] : 0.f;
    float m = fabsf(av);
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    const int X = mx_block_exp(m);
    const uint32_t code = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(sat448(av * pow2i(-X)), 0.f, 0, false) & 0xFFu;
    if (ok) {
      const size_t o = ((size_t)slot * T + t) * I + i0 + v;
      aq[o] = (uint8_t)code;
      if (act) act[o] = av;
      if (v == 0) aqs[((size_t)slot * T + t) * NI + i0 / 32] = (uint8_t)(X + 127);
    }
  }
}

// ---------------------------------------------------------------- down + combine + residual

// Workgroup (16-row tile, group g) takes the slots 8 g .. 8 g + 7, two per
// wavefront (s = 8 g + wave + 4 i), both slots' rows and scale bytes
// requested at once; the four wavefront sums are added in wavefront order.
// With one group the workgroup writes the output itself; otherwise each
// group's sum is a partial and the tile's last workgroup adds the groups in
// group order and the residual.  Splitting the slots over workgroups keeps
// every wavefront to two weight fetches issued together instead of one
// dependent fetch per slot.
constexpr int kW4A8DownSpw = 2;   // slots per wavefront
int w4a8_down_groups(int max_slots) { return (max_slots + 4 * kW4A8DownSpw - 1) / (4 * kW4A8DownSpw); }

template <int NSD>   // matrix-core steps of 128 covering I
__global__ void __launch_bounds__(256) moe_down_w4a8_kernel(
    int T, int H, int I, int E, int max_slots, const uint8_t* __restrict__ w2c, const uint8_t* __restrict__ w2s,
    const uint8_t* __restrict__ sh2c, const uint8_t* __restrict__ sh2s, const int32_t* __restrict__ el,
    const float* __restrict__ slot_w, const uint8_t* __restrict__ aq, const uint8_t* __restrict__ aqs,
    const uint16_t* __restrict__ residual, float* __restrict__ out_y, uint16_t* __restrict__ out_h, float* part,
    unsigned* counters) {
  constexpr int SPW = kW4A8DownSpw;
  int n_active = el[0];
  n_active = n_active < 0 ? 0 : (n_active > max_slots - 1 ? max_slots - 1 : n_active);
  const bool has_sh = sh2c != nullptr;
  const int nslots = n_active + (has_sh ? 1 : 0);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int n0 = blockIdx.x * 16;
  const int NB = I / 32;
  const bool col = r16 < T;
  const int row = n0 + r16;
  __shared__ __attribute__((aligned(16))) uint8_t lsd[4][SPW][16 * 4 * NSD];   // per wavefront and slot: [row][block]
  __shared__ int flag;
  // both slots' rows and scale bytes first (16 contiguous rows of scales per slot)
  bool use[SPW];
  uint4 sv[SPW];
  uint4 cw[SPW][NSD];
#pragma unroll
  for (int i = 0; i < SPW; ++i) {
    const int s = (int)blockIdx.y * 4 * SPW + wave + 4 * i;
    const uint8_t *C = nullptr, *S = nullptr;
    use[i] = s < nslots &&
             w4a8_slot(s, n_active, has_sh, E, el, w2c, w2s, sh2c, sh2s, (size_t)H * (I / 2), (size_t)H * NB, &C, &S);
    sv[i] = use[i] && lane < NB ? ld16(S + (size_t)n0 * NB + (size_t)lane * 16) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int st = 0; st < NSD; ++st) {
      const int b = 4 * st + g;
      cw[i][st] = use[i] && b < NB ? ld16(C + (size_t)row * (I / 2) + (size_t)b * 16) : make_uint4(0, 0, 0, 0);
    }
  }
#pragma unroll
  for (int i = 0; i < SPW; ++i)
    if (use[i] && lane < NB) *reinterpret_cast<uint4*>(&lsd[wave][i][lane * 16]) = sv[i];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  v4f_t tot = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < SPW; ++i) {
    if (!use[i]) continue;   // uniform across the wavefront
    const int s = (int)blockIdx.y * 4 * SPW + wave + 4 * i;
    int sw[NSD];
#pragma unroll
    for (int st = 0; st < NSD; ++st) {
      const int b = 4 * st + g;
      sw[st] = b < NB ? (int)lsd[wave][i][r16 * NB + b] : 127;
    }
    v4f_t c = {0.f, 0.f, 0.f, 0.f};
    const size_t arow = ((size_t)s * T + (col ? r16 : 0)) * I;
#pragma unroll
    for (int st = 0; st < NSD; ++st) {
      v8i_t b = {0, 0, 0, 0, 0, 0, 0, 0};
      int sb = 127;
      if (col) b_operand(aq + arow, aqs + arow / 32, I, st, g, b, sb);
      const v8i_t a = {(int)cw[i][st].x, (int)cw[i][st].y, (int)cw[i][st].z, (int)cw[i][st].w, 0, 0, 0, 0};
      c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, kFmtFp4, kFmtFp8, 0, sw[st], 0, sb);
    }
    const float wt = col ? (s < n_active ? slot_w[s * T + r16] : 1.0f) : 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) tot[q] = fmaf(wt, c[q], tot[q]);
  }
  __shared__ float pw[4][16][17];   // [wavefront][row][token]
  if (col) {
#pragma unroll
    for (int q = 0; q < 4; ++q) pw[wave][4 * g + q][r16] = tot[q];
  }
  __syncthreads();
  if (gridDim.y == 1) {   // every slot in this workgroup: no partials
    if ((int)threadIdx.x < 16 * T) {
      const int rr = threadIdx.x & 15, t = threadIdx.x >> 4;
      const float y = ((pw[0][rr][t] + pw[1][rr][t]) + pw[2][rr][t]) + pw[3][rr][t];
      const size_t o = (size_t)t * H + n0 + rr;
      if (out_y) out_y[o] = y;
      if (residual && out_h) out_h[o] = f32_to_bf16_rne(bf16_bits_to_f32(residual[o]) + y);
    }
    return;
  }
  if ((int)threadIdx.x < 16 * T) {
    const int rr = threadIdx.x & 15, t = threadIdx.x >> 4;
    const float v = ((pw[0][rr][t] + pw[1][rr][t]) + pw[2][rr][t]) + pw[3][rr][t];
    st_dev(part + ((size_t)blockIdx.y * T + t) * H + n0 + rr, v);
  }
  // the tile's counter: 32-byte stride
  if (!last_block_arrived(counters + blockIdx.x * 8, gridDim.y, &flag)) return;
  if ((int)threadIdx.x < 16 * T) {
    const int rr = threadIdx.x & 15, t = threadIdx.x >> 4;
    const float y = sum_group_partials(part, (int)gridDim.y, T, H, t, n0 + rr);
    const size_t o = (size_t)t * H + n0 + rr;
    if (out_y) out_y[o] = y;
    if (residual && out_h) out_h[o] = f32_to_bf16_rne(bf16_bits_to_f32(residual[o]) + y);
  }
}

constexpr int kW4A8MaxSteps = 20;   // H <= 2560 on the gate/up side, I <= 2560 on the down side

int steps_case(int n) {
  const int cases[] = {1, 2, 3, 4, 5, 6, 8, 10, 12, 16, 20};
  for (int c : cases)
    if (n <= c) return c;
  return -1;
}

}  // namespace

bool w4a8_shape_supported(int T, int H, int I) {
  if (H % 32 || I % 32 || H < 32 || I < 32 || T < 1 || T > 16) return false;
  if ((H + 127) / 128 > kW4A8MaxSteps || (I + 127) / 128 > kW4A8MaxSteps) return false;
  return (size_t)T * H + (size_t)T * (H / 32) <= 64 * 1024;
}

size_t w4a8_act_bytes(int T, int I, int max_slots) {
  // E4M3 codes [slots][T][I], then (16-byte aligned) the E8M0 scales [slots][T][I/32]
  const size_t codes = ((size_t)max_slots * T * I + 15) & ~(size_t)15;
  return codes + (size_t)max_slots * T * (I / 32);
}

hipError_t launch_act_quant(const uint16_t* x, int T, int K, uint8_t* codes, uint8_t* scales, hipStream_t st) {
  const int nblocks = T * (K / 32);
  act_quant_kernel<<<(nblocks + 255) / 256, 256, 0, st>>>(x, nblocks, codes, scales);
  return hipGetLastError();
}

hipError_t launch_w4a8_experts(const uint16_t* x, int T, int H, int I, int E, int k, const uint8_t* w13c,
                               const uint8_t* w13s, const uint8_t* w2c, const uint8_t* w2s, const uint8_t* sh13c,
                               const uint8_t* sh13s, const uint8_t* sh2c, const uint8_t* sh2s, const int32_t* el,
                               const float* sw, const uint16_t* res, float* y, uint16_t* h, float* act, void* abuf,
                               float* part, unsigned* counters, hipStream_t st) {
  const int max_slots = T * k + 1;
  uint8_t* aq = reinterpret_cast<uint8_t*>(abuf);
  uint8_t* aqs = aq + (((size_t)max_slots * T * I + 15) & ~(size_t)15);
  const size_t lds = (size_t)T * H + (size_t)T * (H / 32);
  // more than 4 tokens: every gate/up workgroup would quantize all T input
  // rows itself (one dependent round of loads per 256 blocks); quantize them
  // once instead, into the activation region behind the codes and scales it
  // holds (fp32-sized, so the bytes fit unless I is tiny against H)
  const size_t xin_off = (w4a8_act_bytes(T, I, max_slots) + 15) & ~(size_t)15;
  uint8_t* xin = nullptr;
  if (T > WSX_MAX_T && xin_off + lds <= (size_t)max_slots * T * I * 4) {
    xin = aq + xin_off;
    const hipError_t qe = launch_act_quant(x, T, H, xin, xin + (size_t)T * H, st);
    if (qe != hipSuccess) return qe;
  }
  dim3 gg(I / 32, max_slots);
#define WSX_WG(N)                                                                                              \
  case N:                                                                                                      \
    moe_gateup_w4a8_kernel<N><<<gg, 256, lds, st>>>(x, T, H, I, E, max_slots, w13c, w13s, sh13c, sh13s, el, aq, \
                                                    aqs, act, xin);                                            \
    break;
  switch (steps_case((H + 127) / 128)) {
    WSX_WG(1) WSX_WG(2) WSX_WG(3) WSX_WG(4) WSX_WG(5) WSX_WG(6) WSX_WG(8) WSX_WG(10) WSX_WG(12) WSX_WG(16) WSX_WG(20)
    default: return hipErrorInvalidValue;
  }
#undef WSX_WG
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 gd(H / 16, w4a8_down_groups(max_slots));
#define WSX_WD(N)                                                                                              \
  case N:                                                                                                      \
    moe_down_w4a8_kernel<N><<<gd, 256, 0, st>>>(T, H, I, E, max_slots, w2c, w2s, sh2c, sh2s, el, sw, aq, aqs, res, \
                                                y, h, part, counters);                                         \
    break;
  switch (steps_case((I + 127) / 128)) {
    WSX_WD(1) WSX_WD(2) WSX_WD(3) WSX_WD(4) WSX_WD(5) WSX_WD(6) WSX_WD(8) WSX_WD(10) WSX_WD(12) WSX_WD(16) WSX_WD(20)
    default: return hipErrorInvalidValue;
  }
#undef WSX_WD
  return hipGetLastError();
}

}  // namespace wsx
