// Dense row GEMVs of the decode path on gfx950:
//   * the MoE router: logits = Wr x (bf16 or fp32 weights), then, in the last
//     workgroup to finish, the per-token top-k, the softmax over the selected
//     logits and the compact expert list ([saipien] "Why one user waits on
//     weights": 8 of 512 routed experts per token; [saipien] "Draft three
//     tokens, verify four": up to 32 distinct experts for 4 positions);
//   * the LM head: logits = s .* (Wq x) over FP8 E4M3 rows with a per-row
//     scale, or over BF16 rows, with a fused two-pass greedy argmax ([saipien]
//     "Stop hauling the vocabulary in full precision"; [ncij] "What happens
//     on a real workload?" for greedy decoding).
//
// Layout of the work: a wavefront streams 4 rows at a time, 16 lanes per row.
// Each lane owns the 16-byte granules c, c+16, c+32, ... of its row (c = lane
// mod 16), so one wavefront load instruction reads 4 x 256 contiguous bytes.
// The activation granules a lane needs are the same for every row, so for a
// single token they are held in registers for the whole kernel; with several
// tokens they are read from LDS.  Row sums are formed by a fixed DPP tree
// within each 16-lane row, identical for every row, so equal rows give
// bit-identical logits and ties resolve exactly to the lower index.
#include <atomic>

#include "sample_device.h"
#include "wsx_internal.h"

namespace wsx {

enum WType { W_FP8 = 0, W_BF16 = 1, W_F32 = 2 };

template <int WT> struct WTraits;
template <> struct WTraits<W_FP8> { static constexpr int EPG = 16; static constexpr int ESZ = 1; };
template <> struct WTraits<W_BF16> { static constexpr int EPG = 8; static constexpr int ESZ = 2; };
template <> struct WTraits<W_F32> { static constexpr int EPG = 4; static constexpr int ESZ = 4; };

template <int WT>
__device__ __forceinline__ float granule_dot(uint4 w, const uint32_t* xp) {
  if constexpr (WT == W_FP8) return fp8_granule_dot(w, xp);
  else if constexpr (WT == W_BF16) return bf16_granule_dot(w, xp);
  else return f32_granule_dot(w, xp);
}

constexpr int kMaxK = 8192;          // LDS activation stage: T * K bf16 <= 64 KiB

// Stage the activations [T][K] as bf16 in LDS.  With `norm` set the input is
// the residual stream h and the staged value is u = RNE_bf16(h / sqrt(mean(h^2)
// + 1e-6)), per token; workgroup 0 also writes u to u_out when it is non-null.
// The sum of squares uses one fixed order, so every workgroup derives the
// same u.
template <int T, int NT>
__device__ __forceinline__ void stage_input(const uint16_t* __restrict__ x, int K, bool norm, uint16_t* u_out,
                                            uint16_t* xs, float* red) {
  const int tid = threadIdx.x;
  constexpr int MAXC = (T * 320 + NT - 1) / NT;
  if (norm && T * K / 8 <= MAXC * NT) {
    // every chunk stays in this thread's registers: the sums of squares come
    // from them (each chunk's 8 values in order, then the thread's chunks of
    // a token in order, the wavefront tree and the wavefronts in order), and
    // the normalized chunk goes to LDS (and u_out) in one 16-byte store
    const int cpt = K / 8;   // chunks per token
    uint4 v[MAXC];
#pragma unroll
    for (int j = 0; j < MAXC; ++j) {
      const int i = tid + j * NT;
      v[j] = i < T * cpt ? ld16(x + (size_t)i * 8) : make_uint4(0, 0, 0, 0);
    }
    float ss[T];
#pragma unroll
    for (int t = 0; t < T; ++t) ss[t] = 0.f;
#pragma unroll
    for (int j = 0; j < MAXC; ++j) {
      const int i = tid + j * NT;
      const uint32_t w[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
      float c = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float a = bf16_bits_to_f32(w[q] & 0xFFFFu), b = bf16_bits_to_f32(w[q] >> 16);
        c = fmaf(a, a, c);
        c = fmaf(b, b, c);
      }
      const int tok = i / cpt;
#pragma unroll
      for (int t = 0; t < T; ++t) ss[t] += (t == tok) ? c : 0.f;
    }
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const float w = wave_sum(ss[t]);
      if ((tid & 63) == 0) red[t * (NT / 64) + (tid >> 6)] = w;
    }
    __syncthreads();
    float r[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      float sq = 0.f;
      for (int w = 0; w < NT / 64; ++w) sq += red[t * (NT / 64) + w];
      r[t] = 1.0f / sqrtf(sq / (float)K + 1e-6f);
    }
#pragma unroll
    for (int j = 0; j < MAXC; ++j) {
      const int i = tid + j * NT;
      if (i < T * cpt) {
        const int tok = i / cpt;
        float rt = r[0];
#pragma unroll
        for (int t = 1; t < T; ++t) rt = (t == tok) ? r[t] : rt;
        const uint32_t w[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
        uint32_t o[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          o[q] = f32_to_bf16_rne(bf16_bits_to_f32(w[q] & 0xFFFFu) * rt) |
                 (f32_to_bf16_rne(bf16_bits_to_f32(w[q] >> 16) * rt) << 16);
        const uint4 u = make_uint4(o[0], o[1], o[2], o[3]);
        *reinterpret_cast<uint4*>(xs + (size_t)i * 8) = u;
        if (blockIdx.x == 0 && u_out) *reinterpret_cast<uint4*>(u_out + (size_t)i * 8) = u;
      }
    }
    __syncthreads();
    return;
  }
  stage_to_lds<NT, MAXC>(x, xs, T * K / 8);
  if (!norm) { __syncthreads(); return; }
  __syncthreads();
#pragma unroll
  for (int t = 0; t < T; ++t) {
    float ss = 0.f;
    for (int i = tid; i < K; i += NT) {
      float v = bf16_bits_to_f32(xs[t * K + i]);
      ss = fmaf(v, v, ss);
    }
    ss = wave_sum(ss);
    if ((tid & 63) == 0) red[t * (NT / 64) + (tid >> 6)] = ss;
  }
  __syncthreads();
  float r[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    float s = 0.f;
    for (int w = 0; w < NT / 64; ++w) s += red[t * (NT / 64) + w];
    r[t] = 1.0f / sqrtf(s / (float)K + 1e-6f);
  }
  __syncthreads();
#pragma unroll
  for (int t = 0; t < T; ++t)
    for (int i = tid; i < K; i += NT) {
      uint16_t u = f32_to_bf16_rne(bf16_bits_to_f32(xs[t * K + i]) * r[t]);
      xs[t * K + i] = u;
      if (blockIdx.x == 0 && u_out) u_out[t * K + i] = u;
    }
  __syncthreads();
}

// Dot products of up to UNR row groups (4 rows each) for T tokens.
// Row index of this lane for group u: rg[u] * 4 + (lane >> 4).
template <int WT, int T, int GPL, int UNR>
__device__ __forceinline__ void rows_dot(const uint8_t* __restrict__ W, size_t row_bytes, int V, int G, const int* rg,
                                         const uint32_t (*xr)[WTraits<WT>::EPG / 2], const uint32_t* xs32, int K,
                                         float (*acc)[T]) {
  constexpr int DW = WTraits<WT>::EPG / 2;   // dwords of bf16 activations per granule
  const int lane = threadIdx.x & 63;
  const int c = lane & 15;
  uint4 wv[UNR][GPL];
#pragma unroll
  for (int u = 0; u < UNR; ++u) {
    const int row = rg[u] * 4 + (lane >> 4);
    const bool ok = row < V;
#pragma unroll
    for (int j = 0; j < GPL; ++j) {
      const int g = c + 16 * j;
      wv[u][j] = (ok && g < G) ? ld16(W + (size_t)row * row_bytes + (size_t)g * 16) : make_uint4(0, 0, 0, 0);
    }
  }
#pragma unroll
  for (int u = 0; u < UNR; ++u)
#pragma unroll
    for (int t = 0; t < T; ++t) acc[u][t] = 0.f;
#pragma unroll
  for (int j = 0; j < GPL; ++j) {
    const int g = c + 16 * j;
    if (g >= G) continue;
    if constexpr (T == 1) {
#pragma unroll
      for (int u = 0; u < UNR; ++u) acc[u][0] += granule_dot<WT>(wv[u][j], xr[j]);
    } else {
#pragma unroll
      for (int t = 0; t < T; ++t) {
        uint32_t xp[DW];
        const uint32_t* src = xs32 + (size_t)t * (K / 2) + (size_t)g * DW;
#pragma unroll
        for (int d = 0; d < DW; ++d) xp[d] = src[d];
#pragma unroll
        for (int u = 0; u < UNR; ++u) acc[u][t] += granule_dot<WT>(wv[u][j], xp);
      }
    }
  }
#pragma unroll
  for (int u = 0; u < UNR; ++u)
#pragma unroll
    for (int t = 0; t < T; ++t) acc[u][t] = sum16(acc[u][t]);
}

template <int WT, int GPL>
__device__ __forceinline__ void load_x_regs(const uint32_t* xs32, int G, uint32_t (*xr)[WTraits<WT>::EPG / 2]) {
  constexpr int DW = WTraits<WT>::EPG / 2;
  const int c = threadIdx.x & 15;
#pragma unroll
  for (int j = 0; j < GPL; ++j) {
    const int g = c + 16 * j;
#pragma unroll
    for (int d = 0; d < DW; ++d) xr[j][d] = (g < G) ? xs32[(size_t)g * DW + d] : 0u;
  }
}

// ---------------------------------------------------------------- LM head

// The argmax over the per-workgroup partials (value, row) of the head's T
// tokens, by a 256-thread last workgroup: each thread loads its (at most
// kHeadMaxGrid / 256) partials of every token at once, so the tail is one
// coherent round trip; then the wavefront and workgroup reductions (ties to
// the lower row, so the result does not depend on the order).
template <int T>
__device__ __forceinline__ void head_partials_argmax(const float* part_v, const int* part_i, int nb, float (*wv)[T],
                                                     int (*wi)[T], int32_t* argmax) {
  constexpr int PB = kHeadMaxGrid / 256;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float ov[T][PB];
  int oi[T][PB];
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int j = 0; j < PB; ++j) {
      const int b = (int)threadIdx.x + 256 * j;
      ov[t][j] = b < nb ? __uint_as_float(ld_coh4(part_v, (uint32_t)(b * T + t) * 4)) : -INFINITY;
      oi[t][j] = b < nb ? (int)ld_coh4(part_i, (uint32_t)(b * T + t) * 4) : 0x7FFFFFFF;
    }
#pragma unroll
  for (int t = 0; t < T; ++t) {
    float v = -INFINITY;
    int i = 0x7FFFFFFF;
#pragma unroll
    for (int j = 0; j < PB; ++j)
      if (better(ov[t][j], oi[t][j], v, i)) { v = ov[t][j]; i = oi[t][j]; }
    wave_argmax(v, i);
    if (lane == 0) { wv[wave][t] = v; wi[wave][t] = i; }
  }
  __syncthreads();
  if (threadIdx.x < T) {
    const int t = threadIdx.x;
    float v = wv[0][t];
    int i = wi[0][t];
    for (int w = 1; w < 4; ++w)
      if (better(wv[w][t], wi[w][t], v, i)) { v = wv[w][t]; i = wi[w][t]; }
    argmax[t] = i;
  }
}

template <int WT, int T, int GPL>
__global__ void __launch_bounds__(256) lm_head_kernel(const uint8_t* __restrict__ W, const float* __restrict__ row_scale,
                                                      int V, int K, const uint16_t* __restrict__ x, int norm,
                                                      uint16_t* u_out, float* __restrict__ logits,
                                                      int32_t* __restrict__ argmax, unsigned* counter, float* part_v,
                                                      int* part_i) {
  constexpr int NT = 256, UNR = 2, DW = WTraits<WT>::EPG / 2;
  extern __shared__ __attribute__((aligned(16))) uint16_t xs[];
  __shared__ float red[4 * T * 4];
  __shared__ int flag;
  stage_input<T, NT>(x, K, norm != 0, u_out, xs, red);
  const uint32_t* xs32 = reinterpret_cast<const uint32_t*>(xs);
  const int G = K / WTraits<WT>::EPG;
  const size_t row_bytes = (size_t)K * WTraits<WT>::ESZ;
  uint32_t xr[T == 1 ? GPL : 1][DW];
  if constexpr (T == 1) load_x_regs<WT, GPL>(xs32, G, xr);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nwaves = gridDim.x * 4;
  const int NG = (V + 3) / 4;
  float bv[T];
  int bi[T];
#pragma unroll
  for (int t = 0; t < T; ++t) { bv[t] = -INFINITY; bi[t] = 0x7FFFFFFF; }

  for (int base = blockIdx.x * 4 + wave; base < NG; base += nwaves * UNR) {
    int rg[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) rg[u] = base + u * nwaves;
    float acc[UNR][T];
    float sc[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int row = rg[u] * 4 + (lane >> 4);
      sc[u] = (WT == W_FP8 && row < V && (lane & 15) == 0) ? row_scale[row] : 1.0f;
    }
    rows_dot<WT, T, GPL, UNR>(W, row_bytes, V, G, rg, xr, xs32, K, acc);
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int row = rg[u] * 4 + (lane >> 4);
      if ((lane & 15) == 0 && row < V) {
#pragma unroll
        for (int t = 0; t < T; ++t) {
          const float l = (WT == W_FP8) ? acc[u][t] * sc[u] : acc[u][t];
          if (logits) logits[(size_t)t * V + row] = l;
          if (better(l, row, bv[t], bi[t])) { bv[t] = l; bi[t] = row; }
        }
      }
    }
  }
  // workgroup argmax, then the last workgroup reduces the per-workgroup partials
  __shared__ float wv_[4][T];
  __shared__ int wi_[4][T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    float v = bv[t];
    int i = bi[t];
    wave_argmax(v, i);
    if (lane == 0) { wv_[wave][t] = v; wi_[wave][t] = i; }
  }
  __syncthreads();
  if (threadIdx.x < T) {
    const int t = threadIdx.x;
    float v = wv_[0][t];
    int i = wi_[0][t];
    for (int w = 1; w < 4; ++w)
      if (better(wv_[w][t], wi_[w][t], v, i)) { v = wv_[w][t]; i = wi_[w][t]; }
    st_dev(part_v + (size_t)blockIdx.x * T + t, v);
    st_dev(part_i + (size_t)blockIdx.x * T + t, i);
  }
  if (!last_block_arrived(counter, gridDim.x, &flag)) return;
  head_partials_argmax<T>(part_v, part_i, (int)gridDim.x, wv_, wi_, argmax);
}


// ---------------------------------------------------------------- LM head, one token, wide workgroups

// The 1-token head ([saipien] "Stop hauling the vocabulary in full
// precision": the whole head is read for every token) as one 1024-thread
// workgroup per CU.  Wavefront v of workgroup b (of P) takes row groups
// v * P + b + P * 16 * i: the groups left over after the last full round of
// P * 16 go to wavefronts of every workgroup, not to the first workgroups
// alone, so every CU streams the same number of groups to within one.  Each
// wavefront keeps the next group's loads in flight while it reduces the
// current one, and issues its first group's loads before the activations are
// staged.
// RL lanes per row (RPW = 64 / RL rows per wavefront group), GPL granules per
// lane.  The activations sit in LDS with granule g at byte g * GS (a stride
// that lets the RL lanes of a row read their granules without bank
// conflicts).  The argmax is one 64-bit atomic maximum of rank keys (value,
// then lower row), read by the last workgroup to finish, which resets it.
template <int WT, int GPL, int RL>
struct HeadGroup {
  uint4 w[GPL];
  float sc;
};

template <int WT, int GPL, int RL>
__device__ __forceinline__ void head_group_load(__amdgpu_buffer_rsrc_t W, const float* row_scale, int V, int G,
                                                uint32_t row_bytes, int grp, HeadGroup<WT, GPL, RL>& g) {
  constexpr int RPW = 64 / RL;
  const int lane = threadIdx.x & 63;
  const int row = grp * RPW + lane / RL, c = lane % RL;
  const bool ok = row < V;
  const uint32_t o = (uint32_t)(ok ? row : 0) * row_bytes + (uint32_t)c * 16;
#pragma unroll
  for (int j = 0; j < GPL; ++j)
    g.w[j] = (ok && c + RL * j < G)
                 ? __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(W, o + 16 * RL * j, 0, 2))
                 : make_uint4(0, 0, 0, 0);
  g.sc = 1.0f;
  if (WT == W_FP8 && ok && c == 0) g.sc = row_scale[row];
}

// The wide FP8 head for 2..4 tokens (the verify pass's rows): the row
// streaming of lm_head_wide_kernel, with the TT activation rows staged in LDS
// and each granule's 16 codes converted once and used for every token.  Per
// token the products are added in exactly the 1-token kernel's order, so each
// token's logits equal the 1-token head's bit for bit.  Per token, every
// workgroup joins its best (value, row) to a 64-bit atomic max, and the last
// workgroup publishes the argmaxes.  With `norm` the rows are first RMS-
// normalized (u = RNE_bf16(x / sqrt(mean(x^2) + 1e-6)), the decode step's
// final norm): each token's sum of squares is formed from the staged
// registers in one fixed order (a chunk's 8 values, the thread's chunks, the
// wavefront tree, then the 16 wavefronts in order), so every workgroup
// derives the same u; the first workgroup also writes u to u_out.
template <int TT, int GPL, int RL>
__global__ void __launch_bounds__(1024) lm_head_wide_t_kernel(const uint8_t* __restrict__ W,
                                                              const float* __restrict__ row_scale, int V, int K,
                                                              const uint16_t* __restrict__ x, int norm,
                                                              uint16_t* __restrict__ u_out, float* __restrict__ logits,
                                                              int32_t* __restrict__ argmax, unsigned* counter,
                                                              unsigned long long* best) {
  constexpr int RPW = 64 / RL, NW = 16, GS = 48;   // LayHead: 16 bf16 in 48 bytes per granule
  constexpr int XC = (TT * 2560 / 8 + 1023) / 1024;   // 16-byte input chunks per thread (K <= 2560)
  extern __shared__ __attribute__((aligned(16))) uint8_t xsb[];   // [TT][G][GS]
  __shared__ float wv_[NW][TT];
  __shared__ int wi_[NW][TT];
  __shared__ int flag;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6, c = lane % RL;
  const int G = K / 16;
  const uint32_t row_bytes = (uint32_t)K;
  const __amdgpu_buffer_rsrc_t Wr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(W), 0, 0x7FFFFFFF, 0x00020000);
  const int NG = (V + RPW - 1) / RPW;
  const int stride = (int)gridDim.x * NW;
  const int first = wave * (int)gridDim.x + (int)blockIdx.x;
  int grp = first < NG ? first : -1;
  const int nx = K / 8;
  uint4 xv[XC];
#pragma unroll
  for (int q = 0; q < XC; ++q) {
    const int i = t + 1024 * q;
    xv[q] = i < TT * nx ? ld16(x + 8 * i) : make_uint4(0, 0, 0, 0);
  }
  HeadGroup<W_FP8, GPL, RL> cur;
  if (grp >= 0) head_group_load<W_FP8, GPL, RL>(Wr, row_scale, V, G, row_bytes, grp, cur);
  issue_here();
  if (norm) {
    __shared__ float sq[TT][NW];
    float ss[TT];
#pragma unroll
    for (int k2 = 0; k2 < TT; ++k2) ss[k2] = 0.f;
#pragma unroll
    for (int q = 0; q < XC; ++q) {
      const int i = t + 1024 * q;
      const uint32_t w[4] = {xv[q].x, xv[q].y, xv[q].z, xv[q].w};
      float c2 = 0.f;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const float a = bf16_bits_to_f32(w[h] & 0xFFFFu), b = bf16_bits_to_f32(w[h] >> 16);
        c2 = fmaf(a, a, c2);
        c2 = fmaf(b, b, c2);
      }
      const int tok = i < TT * nx ? i / nx : -1;
#pragma unroll
      for (int k2 = 0; k2 < TT; ++k2) ss[k2] += (k2 == tok) ? c2 : 0.f;
    }
#pragma unroll
    for (int k2 = 0; k2 < TT; ++k2) {
      const float w = wave_sum(ss[k2]);
      if (lane == 0) sq[k2][wave] = w;
    }
    lds_barrier();
    float r[TT];
#pragma unroll
    for (int k2 = 0; k2 < TT; ++k2) {
      float a = 0.f;
      for (int w = 0; w < NW; ++w) a += sq[k2][w];
      r[k2] = 1.0f / sqrtf(a / (float)K + 1e-6f);
    }
#pragma unroll
    for (int q = 0; q < XC; ++q) {
      const int i = t + 1024 * q;
      if (i < TT * nx) {
        const int tok = i / nx;
        float rt = r[0];
#pragma unroll
        for (int k2 = 1; k2 < TT; ++k2) rt = (k2 == tok) ? r[k2] : rt;
        const uint32_t w[4] = {xv[q].x, xv[q].y, xv[q].z, xv[q].w};
        uint32_t o[4];
#pragma unroll
        for (int h = 0; h < 4; ++h)
          o[h] = f32_to_bf16_rne(bf16_bits_to_f32(w[h] & 0xFFFFu) * rt) |
                 (f32_to_bf16_rne(bf16_bits_to_f32(w[h] >> 16) * rt) << 16);
        xv[q] = make_uint4(o[0], o[1], o[2], o[3]);
        if (blockIdx.x == 0 && u_out) *reinterpret_cast<uint4*>(u_out + 8 * (size_t)i) = xv[q];
      }
    }
  }
#pragma unroll
  for (int q = 0; q < XC; ++q) {
    const int i = t + 1024 * q;
    if (i < TT * nx) {
      const int tok = i / nx, ch = i - tok * nx;
      *reinterpret_cast<uint4*>(xsb + (size_t)tok * G * GS + (8 * ch / 16) * GS + (8 * ch % 16) * 2) = xv[q];
    }
  }
  lds_barrier();
  float bv[TT];
  int bi[TT];
#pragma unroll
  for (int k2 = 0; k2 < TT; ++k2) { bv[k2] = -INFINITY; bi[k2] = 0x7FFFFFFF; }
  while (grp >= 0) {
    HeadGroup<W_FP8, GPL, RL> nxt;
    const int ng = grp + stride < NG ? grp + stride : -1;
    if (ng >= 0) head_group_load<W_FP8, GPL, RL>(Wr, row_scale, V, G, row_bytes, ng, nxt);
    issue_here();
    float acc[TT];
#pragma unroll
    for (int k2 = 0; k2 < TT; ++k2) acc[k2] = 0.f;
#pragma unroll
    for (int j = 0; j < GPL; ++j) {
      const int g = c + RL * j;
      if (g < G) {
        const uint32_t w[4] = {cur.w[j].x, cur.w[j].y, cur.w[j].z, cur.w[j].w};
        bf16x2_t wp[8];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          wp[2 * d] = fp8x2_to_bf16x2<false>(w[d]);
          wp[2 * d + 1] = fp8x2_to_bf16x2<true>(w[d]);
        }
#pragma unroll
        for (int k2 = 0; k2 < TT; ++k2) {
          const uint4* src4 = reinterpret_cast<const uint4*>(xsb + (size_t)k2 * G * GS + g * GS);
          const uint4 v0 = src4[0], v1 = src4[1];
          const uint32_t xp[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
          // the order of fp8_granule_dot
          float a0 = 0.f, a1 = 0.f;
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            a0 = dot2(wp[2 * d], as_bf16x2(xp[2 * d + 0]), a0);
            a1 = dot2(wp[2 * d + 1], as_bf16x2(xp[2 * d + 1]), a1);
          }
          acc[k2] += a0 + a1;
        }
      }
    }
    const int row = grp * RPW + lane / RL;
#pragma unroll
    for (int k2 = 0; k2 < TT; ++k2) {
      float a = sum16(acc[k2]);
      if constexpr (RL == 32) a += __shfl_xor(a, 16);
      const float l = a * cur.sc;
      if (c == 0 && row < V) {
        if (logits) logits[(size_t)k2 * V + row] = l;
        if (better(l, row, bv[k2], bi[k2])) { bv[k2] = l; bi[k2] = row; }
      }
    }
    cur = nxt;
    grp = ng;
  }
#pragma unroll
  for (int k2 = 0; k2 < TT; ++k2) {
    wave_argmax(bv[k2], bi[k2]);
    if (lane == 0) { wv_[wave][k2] = bv[k2]; wi_[wave][k2] = bi[k2]; }
  }
  lds_barrier();
  if (t < TT) {
    float v = wv_[0][t];
    int i = wi_[0][t];
    for (int q = 1; q < NW; ++q)
      if (better(wv_[q][t], wi_[q][t], v, i)) { v = wv_[q][t]; i = wi_[q][t]; }
    const RankKey key = (v == v) ? rank_key(v, i) : 0ull;   // a NaN never wins
    __hip_atomic_fetch_max(best + t, key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (!last_block_arrived(counter, gridDim.x, &flag)) return;
  if (t < TT) {
    const RankKey b = __hip_atomic_load(best + t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(best + t, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    argmax[t] = b == 0ull ? -1 : key_id(b);
  }
}

// The sampling epilogue of the 1-token head ([ncij] "What happens on a real
// workload?": temperature, top-p and top-k sampling), fused into its tail.
// The selection rests on one fact: with the rows split into chunks, the k-th
// largest chunk maximum tau is at most the k-th largest logit, so every top-k
// row is >= tau and lies in one of the k chunks whose maximum is >= tau.  Here
// a chunk is the rows one wavefront streamed (at most 64).  Each wavefront
// publishes its maximum and each workgroup the largest of its wavefronts'; the
// last workgroup to finish then
//   1. takes tau_wg, the k-th largest workgroup maximum: a lower bound of tau
//      (the k workgroups at or above it each hold a chunk at their own
//      maximum), so only the chunks of those k workgroups (<= 16 k) can reach
//      tau;
//   2. selects tau among those chunk maxima and lists the k chunks at or
//      above it;
//   3. reads back those chunks' logits (<= 64 k), keeps the ones >= tau, ranks
//      them for the top k in order, and draws.
// Ranks are counted by the whole workgroup over keys staged in LDS
// (wg_rank_keys); one wavefront draws (sample_draw_wave).  Keys are the 64-bit
// rank keys of the greedy path (value, then lower row); a NaN logit gets key 0
// and is never a candidate.  Logits and maxima are written with
// device-coherent stores so that the last workgroup reads them current on any
// XCD.
constexpr int kSampFusedMaxGrid = 512;            // workgroups (so <= 8192 chunks)
constexpr int kSampFusedMaxChunkRows = 64;        // rows one wavefront may stream
constexpr int kSampFusedSurvivors = kSampMaxK * kSampFusedMaxChunkRows;

struct HeadSample {
  RankKey* chunk_max;     // [gridDim.x * 16], by the chunk's first row group
  RankKey* wg_max;        // [gridDim.x]
  int k;
  float temperature, top_p;
  const float* uniforms;  // [1]
  int32_t* token;         // [1]
  int32_t* topk_ids;      // [k] or null
  float* topk_probs;      // [k] or null
};

__device__ __forceinline__ RankKey ld_key(const RankKey* base, int i) {
  const uint2 v = ld_coh8(base, (uint32_t)i * 8);
  return ((RankKey)v.y << 32) | v.x;
}

template <int RPW>
__device__ void head_sample_tail(const HeadSample& P, const float* logits, int V, int NG, int stride) {
  __shared__ __attribute__((aligned(16))) RankKey gm[kSampFusedMaxGrid + 2];      // workgroup maxima
  __shared__ __attribute__((aligned(16))) RankKey bk[16 * kSampMaxK + 2];         // chunk maxima >= tau_wg
  __shared__ int bw[16 * kSampMaxK];                                              // their first row groups
  __shared__ __attribute__((aligned(16))) RankKey sv[kSampFusedSurvivors + 2];    // rows >= tau
  __shared__ RankKey top[kSampMaxK];
  __shared__ int qlist[kSampMaxK];
  __shared__ RankKey tau_wg, tau;
  __shared__ int nb, ns;
  constexpr int kChunkRegs = kSampFusedMaxGrid * 16 / 1024;
  const int t = threadIdx.x, k = P.k;
  const int nwg = (int)gridDim.x, nchunk = nwg * 16;
  // one round of loads: every chunk maximum (in registers), every workgroup
  // maximum, the uniform
  RankKey ck[kChunkRegs];
#pragma unroll
  for (int r = 0; r < kChunkRegs; ++r) ck[r] = t + 1024 * r < nchunk ? ld_key(P.chunk_max, t + 1024 * r) : 0ull;
  const RankKey gk = t < nwg ? ld_key(P.wg_max, t) : 0ull;
  const float u = t < 64 ? P.uniforms[0] : 0.f;
  // zero fill, so that every list below ends in zeros without a pad
#pragma unroll
  for (int r = 0; r < (kSampFusedSurvivors + 2 + 1023) / 1024; ++r)
    if (t + 1024 * r < kSampFusedSurvivors + 2) sv[t + 1024 * r] = 0ull;
  bk[t] = 0ull;
  if (t < kSampMaxK) top[t] = 0ull;
  if (t <= nwg) gm[t] = t < nwg ? gk : 0ull;
  if (t == 0) {
    tau_wg = 1ull;   // no cut unless k workgroups hold a candidate
    tau = 1ull;
    nb = 0;
    ns = 0;
  }
  __syncthreads();
  // 1. tau_wg: the workgroup maximum of rank k - 1 (nonzero maxima are distinct)
  wg_rank_keys(gm, nwg, [&](int i, int r) {
    if (r == k - 1 && gm[i] != 0ull) tau_wg = gm[i];
  });
  __syncthreads();
  // 2. the chunk maxima >= tau_wg (at most 16 k)
  const RankKey tw = tau_wg;
#pragma unroll
  for (int r = 0; r < kChunkRegs; ++r)
    if (ck[r] != 0ull && ck[r] >= tw) {
      const int pos = atomicAdd(&nb, 1);
      if (pos < 16 * kSampMaxK) {
        bk[pos] = ck[r];
        bw[pos] = t + 1024 * r;
      }
    }
  __syncthreads();
  // ranked: the first k are the chunks that can hold a top-k row, the k-th is tau
  const int n_b = min(nb, 16 * kSampMaxK);
  wg_rank_keys(bk, n_b, [&](int i, int r) {
    if (r < k) qlist[r] = bw[i];
    if (r == k - 1) tau = bk[i];
  });
  __syncthreads();
  // 3. the rows of those chunks: the wavefront whose first group is g
  // streamed groups g + stride * i, RPW rows each; all loads issued first
  const int n_q = min(n_b, k);
  const RankKey th = tau;
  constexpr int kRowRegs = kSampFusedSurvivors / 1024;
  float lv[kRowRegs];
  int lrow[kRowRegs];
#pragma unroll
  for (int r = 0; r < kRowRegs; ++r) {
    const int c = t + 1024 * r;
    const int q = c / kSampFusedMaxChunkRows, s = c % kSampFusedMaxChunkRows;
    lrow[r] = -1;
    lv[r] = 0.f;
    if (q < n_q) {
      const int grp = qlist[q] + stride * (s / RPW);
      const int row = grp * RPW + s % RPW;
      if (grp < NG && row < V) {
        lrow[r] = row;
        lv[r] = __uint_as_float(ld_coh4(logits, (uint32_t)row * 4));
      }
    }
  }
#pragma unroll
  for (int r = 0; r < kRowRegs; ++r)
    if (lrow[r] >= 0 && lv[r] == lv[r]) {
      const RankKey key = rank_key(lv[r], lrow[r]);
      if (key >= th) {
        const int pos = atomicAdd(&ns, 1);
        if (pos < kSampFusedSurvivors) sv[pos] = key;
      }
    }
  __syncthreads();
  wg_rank_keys(sv, min(ns, kSampFusedSurvivors), [&](int i, int r) {
    if (r < k) top[r] = sv[i];
  });
  __syncthreads();
  if (t < 64) sample_draw_wave(t < k ? top[t] : 0ull, k, P.temperature, P.top_p, u, P.token, P.topk_ids, P.topk_probs);
}

template <int WT, int GPL, int RL, bool SAMPLE>
__global__ void __launch_bounds__(1024) lm_head_wide_kernel(const uint8_t* __restrict__ W,
                                                            const float* __restrict__ row_scale, int V, int K,
                                                            const uint16_t* __restrict__ x, float* __restrict__ logits,
                                                            int32_t* __restrict__ argmax, unsigned* counter,
                                                            unsigned long long* best, HeadSample smp) {
  constexpr int EPG = WTraits<WT>::EPG, DW = EPG / 2, RPW = 64 / RL, NW = 16;
  constexpr int GS = (WT == W_FP8) ? 48 : 16;   // LDS bytes per activation granule
  extern __shared__ __attribute__((aligned(16))) uint8_t xsb[];
  __shared__ float wv_[NW];
  __shared__ int wi_[NW];
  __shared__ RankKey wk_[NW];
  __shared__ int flag;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6, c = lane % RL;
  const int G = K / EPG;
  const uint32_t row_bytes = (uint32_t)K * WTraits<WT>::ESZ;
  const __amdgpu_buffer_rsrc_t Wr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(W), 0, 0x7FFFFFFF, 0x00020000);
  const int NG = (V + RPW - 1) / RPW;
  const int stride = (int)gridDim.x * NW;
  const int first = wave * (int)gridDim.x + (int)blockIdx.x;
  int grp = first < NG ? first : -1;
  // x first (one 16-byte chunk of 8 bf16 per thread, K <= 8192), then the
  // first group: loads complete in issue order, so the staging below waits
  // for x alone and the group stays in flight across the barrier
  uint4 xv = make_uint4(0, 0, 0, 0);
  if (t < K / 8) xv = ld16(x + 8 * t);
  HeadGroup<WT, GPL, RL> cur;
  if (grp >= 0) head_group_load<WT, GPL, RL>(Wr, row_scale, V, G, row_bytes, grp, cur);
  issue_here();
  if (t < K / 8) *reinterpret_cast<uint4*>(xsb + (8 * t / EPG) * GS + (8 * t % EPG) * 2) = xv;
  lds_barrier();
  float bv = -INFINITY;
  int bi = 0x7FFFFFFF;
  while (grp >= 0) {
    HeadGroup<WT, GPL, RL> nxt;
    const int ng = grp + stride < NG ? grp + stride : -1;
    if (ng >= 0) head_group_load<WT, GPL, RL>(Wr, row_scale, V, G, row_bytes, ng, nxt);
    issue_here();
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < GPL; ++j) {
      const int g = c + RL * j;
      if (g < G) {
        uint32_t xp[DW];
        const uint4* src4 = reinterpret_cast<const uint4*>(xsb + g * GS);
#pragma unroll
        for (int d = 0; d < DW / 4; ++d) {
          const uint4 v = src4[d];
          xp[4 * d] = v.x; xp[4 * d + 1] = v.y; xp[4 * d + 2] = v.z; xp[4 * d + 3] = v.w;
        }
        acc += granule_dot<WT>(cur.w[j], xp);
      }
    }
    acc = sum16(acc);
    if constexpr (RL == 32) acc += __shfl_xor(acc, 16);
    const int row = grp * RPW + lane / RL;
    const float l = (WT == W_FP8) ? acc * cur.sc : acc;
    if (c == 0 && row < V) {
      if constexpr (SAMPLE) st_coh4(logits, (uint32_t)row * 4, __float_as_uint(l));
      else if (logits) logits[row] = l;
      if (better(l, row, bv, bi)) { bv = l; bi = row; }
    }
    cur = nxt;
    grp = ng;
  }
  wave_argmax(bv, bi);
  if constexpr (SAMPLE) {
    // this chunk's maximum (0 when it streamed no row that is a number)
    const RankKey m = bi != 0x7FFFFFFF ? rank_key(bv, bi) : 0ull;
    if (lane == 0) {
      wk_[wave] = m;
      st_coh8(smp.chunk_max, (uint32_t)first * 8, make_uint2((unsigned)m, (unsigned)(m >> 32)));
    }
    lds_barrier();
    if (t == 0) {
      RankKey wm = wk_[0];
      for (int q = 1; q < NW; ++q) wm = wk_[q] > wm ? wk_[q] : wm;
      st_coh8(smp.wg_max, (uint32_t)blockIdx.x * 8, make_uint2((unsigned)wm, (unsigned)(wm >> 32)));
    }
    if (!last_block_arrived(counter, gridDim.x, &flag)) return;
    head_sample_tail<RPW>(smp, logits, V, NG, stride);
  } else {
    if (lane == 0) { wv_[wave] = bv; wi_[wave] = bi; }
    lds_barrier();
    if (t == 0) {
      float v = wv_[0];
      int i = wi_[0];
      for (int q = 1; q < NW; ++q)
        if (better(wv_[q], wi_[q], v, i)) { v = wv_[q]; i = wi_[q]; }
      const RankKey key = (v == v) ? rank_key(v, i) : 0ull;   // a NaN never wins
      __hip_atomic_fetch_max(best, key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (!last_block_arrived(counter, gridDim.x, &flag)) return;
    if (t == 0) {
      const RankKey b = __hip_atomic_load(best, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(best, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      argmax[0] = b == 0ull ? -1 : key_id(b);
    }
  }
}


// ---------------------------------------------------------------- router + top-k

// Top-k of one token's E logits (E <= 4 * 256) by the whole 256-thread
// workgroup, with no sequential selection rounds.  Logits rank by value, then
// by lower id.  Thread t holds logits P t .. P t + P - 1 (positions past E
// hold -inf) and four consecutive threads form a group of 4P.  A logit whose
// group's best logit is beaten by the best logits of k other groups is itself
// beaten by k logits, so the top k lie in the 8 (>= k) groups whose best
// logits rank highest.  The 64 group maxima are ranked by counting pairwise
// wins (16 comparisons per thread, summed over the group's four threads);
// then the 32P logits of the 8 best groups are ranked the same way.  Leaves
// the k (logit, id) pairs in rank order in rv / rid.
constexpr int kTopkGroups = 64;
struct alignas(16) TopkScratch {
  float2 grp[kTopkGroups];   // (best logit, id bits) per group
  float2 cand[8 * 4 * 4];    // every logit of the 8 best groups (P <= 4)
  float rv[WSX_MAX_K];
  int rid[WSX_MAX_K];
};

__device__ __forceinline__ bool rank_before(float2 a, float v, int i) {
  return better(a.x, __float_as_int(a.y), v, i);
}

template <int CTRL>
__device__ __forceinline__ int dpp_int(int v) { return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false); }

template <int P>
__device__ __forceinline__ void block_topk(const float* __restrict__ lrow, int E, int k, TopkScratch* R) {
  constexpr int NC = 8 * 4 * P;   // candidates
  constexpr int TPC = 256 / NC;   // threads per candidate (4 or 2)
  constexpr int CPT = NC / TPC;   // comparisons per thread
  const int t = threadIdx.x, q = t & 3;
  const int e0 = P * t;
  float v[P];
#pragma unroll
  for (int i = 0; i < P; ++i) v[i] = (e0 + i < E) ? __uint_as_float(ld_coh4(lrow, (uint32_t)(e0 + i) * 4)) : -INFINITY;
  float bv = v[0];
  int bi = e0;
#pragma unroll
  for (int i = 1; i < P; ++i)
    if (better(v[i], e0 + i, bv, bi)) { bv = v[i]; bi = e0 + i; }
  {
    const float ov = dpp_f<kQuadSwap1>(bv);
    const int oi = dpp_int<kQuadSwap1>(bi);
    if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
  }
  {
    const float ov = dpp_f<kQuadSwap2>(bv);
    const int oi = dpp_int<kQuadSwap2>(bi);
    if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
  }
  if (q == 0) R->grp[t >> 2] = make_float2(bv, __int_as_float(bi));
  __syncthreads();
  int rank = 0;
  {
    float2 gv[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) gv[j] = R->grp[16 * q + j];   // all reads first
#pragma unroll
    for (int j = 0; j < 16; ++j) rank += rank_before(gv[j], bv, bi);
  }
  rank += dpp_int<kQuadSwap1>(rank);
  rank += dpp_int<kQuadSwap2>(rank);
  if (rank < 8) {
#pragma unroll
    for (int i = 0; i < P; ++i) R->cand[rank * 4 * P + P * q + i] = make_float2(v[i], __int_as_float(e0 + i));
  }
  __syncthreads();
  const int ci = t / TPC, part = t % TPC;
  const float2 me = R->cand[ci];
  const int mid = __float_as_int(me.y);
  int r2 = 0;
#pragma unroll
  for (int j0 = 0; j0 < CPT; j0 += 16) {
    float2 cv[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) cv[j] = R->cand[part * CPT + j0 + j];   // reads of a batch first
#pragma unroll
    for (int j = 0; j < 16; ++j) r2 += rank_before(cv[j], me.x, mid);
  }
  r2 += dpp_int<kQuadSwap1>(r2);
  if constexpr (TPC == 4) r2 += dpp_int<kQuadSwap2>(r2);
  if (part == 0 && r2 < k) {
    R->rv[r2] = me.x;
    R->rid[r2] = mid;
  }
  __syncthreads();
}

// Top-k of one token's E logits (E <= 64 PW, k <= 8) by one wavefront.  Lane
// l holds logits PW l .. PW l + PW - 1 as 64-bit rank keys (order-preserving
// value bits over the complemented id, so one unsigned compare orders by
// value, then lower id; positions past E get key 0).  A logit beaten by the
// maxima of k other lanes is beaten by k logits, so the top k lie in the k
// lanes whose maxima rank highest.  Each lane's maximum is ranked by counting
// the larger ones among all 64, read back from this wavefront's LDS scratch
// (every lane reads the same words, so the reads are broadcasts); the keys of
// the k best lanes go to the candidate slots (rank-major, zeros elsewhere),
// and each of the 8 PW candidates is ranked the same way.  Leaves the k
// (logit, id) pairs in rank order in rv / rid.  scratch: 64 + 8 PW keys,
// 16-byte aligned, used by this wavefront alone.
//
// The logits were stored by other workgroups of the launch: they are read with
// device-coherent buffer loads, which (unlike atomic loads) the compiler
// issues together, so a wavefront pays one round trip for all of them.
template <int PW>
__device__ __forceinline__ void wave_load_logits(const float* logits, size_t row0, int E, float (&v)[PW]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < PW; ++i) {
    const int e = PW * lane + i;
    v[i] = e < E ? __uint_as_float(ld_coh4(logits, (uint32_t)(row0 + e) * 4)) : 0.f;
  }
}

// Number of the N keys at buf (16-byte aligned) greater than m, with the LDS
// reads issued 32 keys at a time, so a count pays N / 32 LDS latencies.
template <int N>
__device__ __forceinline__ int count_greater_n(const RankKey* buf, RankKey m) {
  static_assert(N % 32 == 0, "whole batches");
  int r = 0;
#pragma unroll
  for (int j0 = 0; j0 < N; j0 += 32) {
    ulonglong2 p[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) p[j] = reinterpret_cast<const ulonglong2*>(buf + j0)[j];
#pragma unroll
    for (int j = 0; j < 16; ++j) r += (int)(p[j].x > m) + (int)(p[j].y > m);
  }
  return r;
}

template <int PW>
__device__ __forceinline__ void wave_topk_values(const float (&v)[PW], int E, int k, RankKey* scratch, float* rv,
                                                 int* rid) {
  constexpr int NC = 8 * PW;                  // candidate slots: 8 lanes x PW
  constexpr int CPL = (NC + 63) / 64;         // candidates per lane
  RankKey* mxs = scratch;                     // [64] lane maxima
  RankKey* cand = scratch + 64;               // [NC]
  const int lane = threadIdx.x & 63;
  RankKey key[PW];
#pragma unroll
  for (int i = 0; i < PW; ++i) {
    const int e = PW * lane + i;
    key[i] = e < E ? rank_key(v[i], e) : 0ull;
  }
  RankKey mx = key[0];
#pragma unroll
  for (int i = 1; i < PW; ++i) mx = key[i] > mx ? key[i] : mx;
  mxs[lane] = mx;
#pragma unroll
  for (int m = 0; m < CPL; ++m)
    if (lane + 64 * m < NC) cand[lane + 64 * m] = 0ull;
  // LDS accesses of one wavefront complete in order: only the compiler has to
  // keep these stores before the reads below
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int r = count_greater_n<64>(mxs, mx);
  if (r < k) {
#pragma unroll
    for (int i = 0; i < PW; ++i) cand[r * PW + i] = key[i];
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
  for (int m = 0; m < CPL; ++m) {
    const RankKey cv = lane + 64 * m < NC ? cand[lane + 64 * m] : 0ull;
    const int rk = count_greater_n<NC>(cand, cv);
    if (cv != 0ull && rk < k) {
      rv[rk] = key_value(cv);
      rid[rk] = key_id(cv);
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int PW>
__device__ __forceinline__ void wave_topk(const float* logits, size_t row0, int E, int k, RankKey* scratch, float* rv,
                                          int* rid) {
  float v[PW];
  wave_load_logits<PW>(logits, row0, E, v);
  wave_topk_values<PW>(v, E, k, scratch, rv, rid);
}

// DW consecutive dwords from LDS as one vector read (the address is a multiple
// of 4 DW bytes).
template <int DW>
__device__ __forceinline__ void lds_dwords(const uint32_t* p, uint32_t (&d)[DW]) {
  if constexpr (DW == 4) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
  } else if constexpr (DW == 2) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    d[0] = v.x; d[1] = v.y;
  } else {
#pragma unroll
    for (int i = 0; i < DW; ++i) d[i] = p[i];
  }
}

// Router GEMV with one row per wavefront (64 lanes; lane l takes the 16-byte
// granules l, l + 64, ...; RGPL per lane) for T tokens staged in LDS (and
// normalized there when `norm` is set).  Every row uses the same lanes and the
// same fixed reduction order, so equal rows give bit-identical logits.  The
// row's weights are requested before the activations are staged, so the two
// overlap.  The last workgroup to finish then takes, per token, the top-k and
// the softmax over the selected logits in rank order, and finally builds the
// compact ascending expert list and the slot weight table.
template <int WT, int T, int RGPL, int P>
__global__ void __launch_bounds__(256) router_topk_kernel(
    const uint8_t* __restrict__ W, int E, int K, int k, const uint16_t* __restrict__ x, int norm, uint16_t* u_out,
    float* logits, int32_t* __restrict__ topk_ids, float* __restrict__ topk_w, int32_t* __restrict__ expert_list,
    float* __restrict__ slot_w, unsigned* counter) {
  constexpr int DW = WTraits<WT>::EPG / 2;
  extern __shared__ __attribute__((aligned(16))) uint16_t xs[];
  __shared__ float red[T * 4];
  __shared__ int flag;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int G = K / WTraits<WT>::EPG;
  const size_t row_bytes = (size_t)K * WTraits<WT>::ESZ;
  int row = blockIdx.x * 4 + wave;
  uint4 wv[RGPL];
#pragma unroll
  for (int j = 0; j < RGPL; ++j) {
    const int g = lane + 64 * j;
    wv[j] = (row < E && g < G) ? ld16(W + (size_t)row * row_bytes + (size_t)g * 16) : make_uint4(0, 0, 0, 0);
  }
  stage_input<T, 256>(x, K, norm != 0, u_out, xs, red);
  const uint32_t* xs32 = reinterpret_cast<const uint32_t*>(xs);
  while (row < E) {
    float acc[T];
#pragma unroll
    for (int t = 0; t < T; ++t) acc[t] = 0.f;
    // granules past the row end hold zero weights: their reads (clamped into
    // the row) add nothing, and each token still sums its granules in order
#pragma unroll
    for (int j = 0; j < RGPL; ++j) {
      const int g = min(lane + 64 * j, G - 1);
      uint32_t xp[T][DW];
#pragma unroll
      for (int t = 0; t < T; ++t) lds_dwords<DW>(xs32 + (size_t)t * (K / 2) + (size_t)g * DW, xp[t]);
#pragma unroll
      for (int t = 0; t < T; ++t) acc[t] += granule_dot<WT>(wv[j], xp[t]);
    }
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const float s = wave_sum_dpp(acc[t]);
      if (lane == 0) st_dev(logits + (size_t)t * E + row, s);
    }
    row += gridDim.x * 4;
    if (row < E) {
#pragma unroll
      for (int j = 0; j < RGPL; ++j) {
        const int g = lane + 64 * j;
        wv[j] = (g < G) ? ld16(W + (size_t)row * row_bytes + (size_t)g * 16) : make_uint4(0, 0, 0, 0);
      }
    }
  }
  if (!last_block_arrived(counter, gridDim.x, &flag)) return;

  // ---- last workgroup: the top-k and the softmax over the selected logits
  // in rank order, per token; one token takes the whole workgroup, several
  // take one wavefront each, side by side
  __shared__ TopkScratch R;
  __shared__ __attribute__((aligned(16))) RankKey wcand[WSX_MAX_T][64 + 8 * 4 * P];
  __shared__ float wrv[WSX_MAX_T][WSX_MAX_K];
  __shared__ int wrid[WSX_MAX_T][WSX_MAX_K];
  __shared__ int sel_id[WSX_MAX_T * WSX_MAX_K];
  __shared__ float sel_w[WSX_MAX_T * WSX_MAX_K];
  __shared__ float sw_tab[WSX_MAX_T * WSX_MAX_K * WSX_MAX_T];
  __shared__ unsigned bm[WSX_MAX_E / 32];   // bitmap of the selected ids
  const float* rv_t;
  const int* rid_t;
  int t = 0, j0 = -1;
  if constexpr (T == 1) {
    block_topk<P>(logits, E, k, &R);
    rv_t = R.rv;
    rid_t = R.rid;
    if (threadIdx.x < k) j0 = threadIdx.x;
  } else {
    t = wave;
    if (wave < T) {
      wave_topk<4 * P>(logits, (size_t)t * E, E, k, wcand[t], wrv[t], wrid[t]);
      if (lane < k) j0 = lane;
    }
    rv_t = wrv[t < T ? t : 0];
    rid_t = wrid[t < T ? t : 0];
  }
  if (j0 >= 0) {
    const float top = rv_t[0];
    float zs = 0.f, mine = 0.f;
#pragma unroll
    for (int j = 0; j < WSX_MAX_K; ++j) {
      if (j < k) {
        const float z = __expf(rv_t[j] - top);
        zs += z;
        if (j == j0) mine = z;
      }
    }
    const float wj = mine / zs;
    const int id = rid_t[j0];
    topk_ids[t * k + j0] = id;
    topk_w[t * k + j0] = wj;
    sel_id[t * k + j0] = id;
    sel_w[t * k + j0] = wj;
  }
  __syncthreads();
  const int n = T * k;
  if (wave == 0) {
    // lane j < n holds selection j (token j / k).  The selected ids go into a
    // bitmap; an id's slot is the number of selected ids below it (the
    // popcounts of the words before its own, by a prefix over the lanes, plus
    // the bits below it in its word), so every selection of an id writes the
    // same list entry.  One wavefront does it all: its LDS accesses complete
    // in order, so only the compiler has to keep them in order.
    const int nw = (E + 31) / 32;   // <= 32 words
    // (clamped: a selection is always an id below E, but the bitmap must never be indexed past its end)
    const int id = lane < n ? min(max(sel_id[lane], 0), E - 1) : 0;
    if (lane < nw) bm[lane] = 0u;
    for (int e = lane; e < n * T; e += 64) sw_tab[e] = 0.f;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (lane < n) atomicOr(&bm[id >> 5], 1u << (id & 31));
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const unsigned word = lane < nw ? bm[lane] : 0u;
    const int c = __popc(word);
    int incl = c;
#pragma unroll
    for (int d = 1; d < 32; d <<= 1) {
      const int o = __shfl_up(incl, d);
      if (lane >= d) incl += o;
    }
    const int pre = incl - c;   // selected ids below word `lane`
    const int w = id >> 5;
    const int rank = __shfl(pre, w) + __popc(__shfl(word, w) & ((1u << (id & 31)) - 1u));
    const int total = __shfl(incl, 31);   // (every lane takes part in the shuffle)
    if (lane == 0) expert_list[0] = total;
    if (lane < n) {
      expert_list[1 + rank] = id;
      sw_tab[rank * T + lane / k] = sel_w[lane];   // a token's k ids are distinct: one entry per (slot, token)
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < n * T; e += 256) slot_w[e] = sw_tab[e];
}

// ---------------------------------------------------------------- router for 5..16 tokens

// The router of a small batch or a longer draft (5 <= T <= WSX_MAX_T_MOE
// tokens; [saipien] "Draft three tokens, verify four" for the verify pass
// this generalizes).  The GEMV is the one above with the tokens staged in LDS
// four at a time (their rows stay in registers across the stages), so the
// stage never exceeds 4 K bf16.  Each thread issues all of a stage's loads at
// once; for rows of up to 5 granules per lane every stage is requested before
// the first is stored, for up to 10 the next stage's loads are in flight while
// the current one is multiplied.  The last workgroup ranks
// each token on one wavefront (wavefront w takes tokens w, w + 4, ..., and
// reads all of their logits at once), then builds the compact list from the
// T k selections through a bitmap of the selected ids: an id's slot is the
// number of selected ids below it.
constexpr int kRouteChunk = 4;


// Load / store one stage of up to kRouteChunk tokens (nx 16-byte chunks per
// token) with XPC chunks per thread, every load issued before the first use.
template <int XPC>
__device__ __forceinline__ void route_stage_load(const uint16_t* x, int tc, int nt, int nx, uint4 (&r)[XPC]) {
  const uint4* src = reinterpret_cast<const uint4*>(x) + (size_t)tc * nx;
#pragma unroll
  for (int i = 0; i < XPC; ++i) {
    const int c = threadIdx.x + 256 * i;
    r[i] = c < nt * nx ? src[c] : make_uint4(0, 0, 0, 0);
  }
}
template <int XPC>
__device__ __forceinline__ void route_stage_store(const uint4 (&r)[XPC], int nt, int nx, uint16_t* xs) {
#pragma unroll
  for (int i = 0; i < XPC; ++i) {
    const int c = threadIdx.x + 256 * i;
    if (c < nt * nx) reinterpret_cast<uint4*>(xs)[c] = r[i];
  }
}

template <int WT, int RGPL, int P>
__global__ void __launch_bounds__(256) router_topk_grouped_kernel(
    const uint8_t* __restrict__ W, int E, int K, int k, const uint16_t* __restrict__ x, int T, float* logits,
    int32_t* __restrict__ topk_ids, float* __restrict__ topk_w, int32_t* __restrict__ expert_list,
    float* __restrict__ slot_w, unsigned* counter) {
  constexpr int DW = WTraits<WT>::EPG / 2;
  // 16-byte chunks of one stage per thread: kRouteChunk K / 8 / 256 <= RGPL
  // for both weight types (RGPL = ceil(K / EPG / 64))
  constexpr int XPC = RGPL;
  constexpr bool kAllStages = RGPL <= 5;   // all stages in registers (4 XPC chunks per thread)
  constexpr bool kPrefetch = RGPL <= 10;   // else the next stage in flight during the dots
  // [kRouteChunk][K] bf16 stages; in the last workgroup's tail, the [T][E] logits
  extern __shared__ __attribute__((aligned(16))) uint16_t xs[];
  __shared__ int flag;
  __shared__ float lg[WSX_MAX_T_MOE][4];   // this workgroup's logits, stored once after the stages
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int G = K / WTraits<WT>::EPG;
  const int nx = K / 8;
  const size_t row_bytes = (size_t)K * WTraits<WT>::ESZ;
  const uint32_t* xs32 = reinterpret_cast<const uint32_t*>(xs);
  for (int r0 = blockIdx.x * 4; r0 < E; r0 += gridDim.x * 4) {   // uniform across the workgroup
    const int row = r0 + wave;
    const bool ok = row < E;
    uint4 wv[RGPL];
#pragma unroll
    for (int j = 0; j < RGPL; ++j) {
      const int g = lane + 64 * j;
      wv[j] = (ok && g < G) ? ld16(W + (size_t)row * row_bytes + (size_t)g * 16) : make_uint4(0, 0, 0, 0);
    }
    // the logits of the staged tokens tc .. tc + nt - 1 for this wavefront's
    // row: the four token slots side by side, each granule's activations read
    // for all of them before the products (slots past nt are computed and
    // dropped).  Granules past the row end hold zero weights, so their reads
    // (clamped into the row) add nothing; each token still sums its granules
    // in order.
    auto dots = [&](int tc, int nt) {
      if (!ok) return;
      if constexpr (RGPL > 16) {   // long rows: one token at a time keeps the registers in bounds
        for (int t = 0; t < nt; ++t) {
          float a = 0.f;
#pragma unroll
          for (int j = 0; j < RGPL; ++j) {
            uint32_t xp[DW];
            lds_dwords<DW>(xs32 + (size_t)t * (K / 2) + (size_t)min(lane + 64 * j, G - 1) * DW, xp);
            a += granule_dot<WT>(wv[j], xp);
          }
          const float sres = wave_sum_dpp(a);
          if (lane == 0) lg[tc + t][wave] = sres;
        }
        return;
      }
      float acc[kRouteChunk];
#pragma unroll
      for (int t = 0; t < kRouteChunk; ++t) acc[t] = 0.f;
#pragma unroll
      for (int j = 0; j < RGPL; ++j) {
        const int g = min(lane + 64 * j, G - 1);
        uint32_t xp[kRouteChunk][DW];
#pragma unroll
        for (int t = 0; t < kRouteChunk; ++t) lds_dwords<DW>(xs32 + (size_t)t * (K / 2) + (size_t)g * DW, xp[t]);
#pragma unroll
        for (int t = 0; t < kRouteChunk; ++t) acc[t] += granule_dot<WT>(wv[j], xp[t]);
      }
#pragma unroll
      for (int t = 0; t < kRouteChunk; ++t) {
        const float sres = wave_sum_dpp(acc[t]);
        if (t < nt && lane == 0) lg[tc + t][wave] = sres;
      }
    };
    if constexpr (kAllStages) {
      // every stage requested at once: one memory latency for all of them
      constexpr int NS = WSX_MAX_T_MOE / kRouteChunk;
      uint4 xall[NS][XPC];
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        const int nt = T - st * kRouteChunk;
        route_stage_load<XPC>(x, st * kRouteChunk, nt < 0 ? 0 : (nt > kRouteChunk ? kRouteChunk : nt), nx, xall[st]);
      }
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        const int tc = st * kRouteChunk;
        if (tc >= T) break;
        const int nt = T - tc < kRouteChunk ? T - tc : kRouteChunk;
        lds_barrier();   // the previous stage's LDS reads are done
        route_stage_store<XPC>(xall[st], nt, nx, xs);
        lds_barrier();
        dots(tc, nt);
      }
    } else {
      uint4 xa[XPC];
      route_stage_load<XPC>(x, 0, T < kRouteChunk ? T : kRouteChunk, nx, xa);
      for (int tc = 0; tc < T; tc += kRouteChunk) {
        const int nt = T - tc < kRouteChunk ? T - tc : kRouteChunk;
        lds_barrier();   // the previous stage's LDS reads are done
        route_stage_store<XPC>(xa, nt, nx, xs);
        const int tn = tc + kRouteChunk;
        const int ntn = T - tn < kRouteChunk ? T - tn : kRouteChunk;
        if (kPrefetch && tn < T) route_stage_load<XPC>(x, tn, ntn, nx, xa);   // in flight during the dots
        lds_barrier();
        dots(tc, nt);
        if (!kPrefetch && tn < T) route_stage_load<XPC>(x, tn, ntn, nx, xa);
      }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < T * 4; i += 256) {
      const int t = i >> 2, rr = r0 + (i & 3);
      if (rr < E) st_dev(logits + (size_t)t * E + rr, lg[t][i & 3]);
    }
  }
  if (!last_block_arrived(counter, gridDim.x, &flag)) return;

  // ---- last workgroup: per token, top-k and softmax in rank order
  constexpr int PW = 4 * P;
  __shared__ __attribute__((aligned(16))) RankKey wcand[4][64 + 8 * PW];
  __shared__ float wrv[4][WSX_MAX_K];
  __shared__ int wrid[4][WSX_MAX_K];
  __shared__ int sel_id[WSX_MAX_T_MOE * WSX_MAX_K];
  __shared__ float sel_w[WSX_MAX_T_MOE * WSX_MAX_K];
  __shared__ float sw_tab[WSX_MAX_T_MOE * WSX_MAX_K * WSX_MAX_T_MOE];
  __shared__ unsigned bm[WSX_MAX_E / 32];   // bitmap of the selected ids
  __shared__ int wpre[WSX_MAX_E / 32];      // selected ids below each bitmap word
  // every logit of the layer into LDS (the stage area is free now), with all
  // of a thread's loads in flight together
  float* ls = reinterpret_cast<float*>(xs);
  {
    const int nl = T * E;
    if ((nl & 3) == 0) {
      constexpr int CPT = WSX_MAX_T_MOE * WSX_MAX_E / 4 / 256;   // 16-byte loads per thread at most
      uint4 v[CPT];
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        const int i = threadIdx.x + 256 * j;
        v[j] = i < nl / 4 ? ld_coh16(logits, (uint32_t)i * 16) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        const int i = threadIdx.x + 256 * j;
        if (i < nl / 4) reinterpret_cast<uint4*>(ls)[i] = v[j];
      }
    } else {
      for (int i0 = 0; i0 < nl; i0 += 256 * 16) {
        uint32_t v[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int i = i0 + threadIdx.x + 256 * j;
          v[j] = i < nl ? ld_coh4(logits, (uint32_t)i * 4) : 0u;
        }
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int i = i0 + threadIdx.x + 256 * j;
          if (i < nl) ls[i] = __uint_as_float(v[j]);
        }
      }
    }
  }
  const int n = T * k;
  const int nw = (E + 31) / 32;
  for (int e = threadIdx.x; e < n * T; e += 256) sw_tab[e] = 0.f;
  if (threadIdx.x < nw) bm[threadIdx.x] = 0u;
  __syncthreads();
#pragma unroll 1
  for (int t = wave; t < T; t += 4) {   // uniform across the wavefront
    float lv[PW];
#pragma unroll
    for (int i = 0; i < PW; ++i) lv[i] = PW * lane + i < E ? ls[(size_t)t * E + PW * lane + i] : 0.f;
    wave_topk_values<PW>(lv, E, k, wcand[wave], wrv[wave], wrid[wave]);
    if (lane < k) {
      const float top = wrv[wave][0];
      float zs = 0.f, mine = 0.f;
#pragma unroll
      for (int j = 0; j < WSX_MAX_K; ++j) {
        if (j < k) {
          const float z = __expf(wrv[wave][j] - top);
          zs += z;
          if (j == lane) mine = z;
        }
      }
      const float wj = mine / zs;
      const int id = wrid[wave][lane];
      topk_ids[t * k + lane] = id;
      topk_w[t * k + lane] = wj;
      sel_id[t * k + lane] = id;
      sel_w[t * k + lane] = wj;
    }
    // the next token reuses this wavefront's scratch: only the compiler has
    // to keep the order (LDS accesses of one wavefront complete in order)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
  __syncthreads();
  for (int j = threadIdx.x; j < n; j += 256) {
    const int id = sel_id[j];
    atomicOr(&bm[id >> 5], 1u << (id & 31));
  }
  __syncthreads();
  if (wave == 0) {
    // exclusive prefix of the words' popcounts (nw <= 32 lanes)
    const int c = lane < nw ? __popc(bm[lane]) : 0;
    int incl = c;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(incl, d);
      if (lane >= d) incl += o;
    }
    if (lane < nw) wpre[lane] = incl - c;
    if (lane == 63) expert_list[0] = incl;
  }
  __syncthreads();
  for (int j = threadIdx.x; j < n; j += 256) {
    const int id = sel_id[j];
    const int w = id >> 5;
    const int rank = wpre[w] + __popc(bm[w] & ((1u << (id & 31)) - 1u));
    expert_list[1 + rank] = id;   // every selection of an id writes the same value
    sw_tab[rank * T + j / k] = sel_w[j];   // a token's k ids are distinct: one entry per (slot, token)
  }
  __syncthreads();
  for (int e = threadIdx.x; e < n * T; e += 256) slot_w[e] = sw_tab[e];
}

// ---------------------------------------------------------------- launchers

template <int WT, int T>
static hipError_t launch_head_t(const void* W, const float* s, int V, int K, const uint16_t* x, int norm, uint16_t* u_out,
                                float* logits, int32_t* argmax, unsigned* counter, float* pv, int* pi, int grid,
                                hipStream_t st) {
  const int G = K / WTraits<WT>::EPG;
  const int gpl = (G + 15) / 16;
#define WSX_HEAD_CASE(N)                                                                                        \
  case N:                                                                                                       \
    lm_head_kernel<WT, T, N><<<grid, 256, (size_t)T * K * 2, st>>>((const uint8_t*)W, s, V, K, x, norm, u_out, logits, argmax, \
                                                   counter, pv, pi);                                            \
    break;
  switch (gpl) {
    WSX_HEAD_CASE(1) WSX_HEAD_CASE(2) WSX_HEAD_CASE(4) WSX_HEAD_CASE(5) WSX_HEAD_CASE(8) WSX_HEAD_CASE(10)
    WSX_HEAD_CASE(16) WSX_HEAD_CASE(20) WSX_HEAD_CASE(32)
    default: return hipErrorInvalidValue;
  }
#undef WSX_HEAD_CASE
  return hipGetLastError();
}

bool head_shape_supported(int wt, int K) {
  const int epg = wt == 0 ? 16 : 8;
  if (K % 32 != 0 || K > kMaxK) return false;
  const int gpl = (K / epg + 15) / 16;
  return gpl == 1 || gpl == 2 || gpl == 4 || gpl == 5 || gpl == 8 || gpl == 10 || gpl == 16 || gpl == 20 || gpl == 32;
}

int head_grid(int V) {
  const int NG = (V + 3) / 4;
  const int waves = (NG + 1) / 2;
  int g = (waves + 3) / 4;
  return g < 1 ? 1 : (g > kHeadMaxGrid ? kHeadMaxGrid : g);
}

// The current device's CU count (the wide heads launch one workgroup per
// CU), queried once per device and kept.
static hipError_t device_cus(int* cus) {
  constexpr int kMaxDev = 64;
  static std::atomic<int> cached[kMaxDev];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDev) return hipErrorInvalidDevice;
  int c = cached[dev].load(std::memory_order_relaxed);
  if (c < 1) {
    e = hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (c < 1) return hipErrorInvalidDevice;
    cached[dev].store(c, std::memory_order_relaxed);
  }
  *cus = c;
  return hipSuccess;
}

// The wide 1-token head for the shapes it is compiled for: one workgroup per
// CU; weights addressed with 32-bit offsets, so the head must be below 2 GiB.
// smp non-null: the sampling variant (FP8 only; see head_sample_fused_fits).
static hipError_t launch_head_wide(int wt, const void* W, const float* s, int V, int K, const uint16_t* x,
                                   float* logits, int32_t* argmax, unsigned* counter, unsigned long long* best,
                                   hipStream_t st, bool* done, const HeadSample* smp = nullptr) {
  *done = false;
  if ((size_t)V * K * (wt == W_FP8 ? 1 : 2) >= ((size_t)1 << 31)) return hipSuccess;
  int cus = 0;
  const hipError_t ce = device_cus(&cus);
  if (ce != hipSuccess) return ce;
  const int epg = wt == W_FP8 ? 16 : 8, gs = wt == W_FP8 ? 48 : 16;
  const size_t lds = (size_t)(K / epg) * gs;
#define WSX_WIDE(WTV, GPLV, RLV)                                                                                   \
  {                                                                                                              \
    lm_head_wide_kernel<WTV, GPLV, RLV, false><<<cus, 1024, lds, st>>>((const uint8_t*)W, s, V, K, x, logits,    \
                                                                        argmax, counter, best, HeadSample{});    \
    *done = true;                                                                                                \
    return hipGetLastError();                                                                                    \
  }
#define WSX_WIDE_S(GPLV, RLV)                                                                                      \
  {                                                                                                              \
    if (smp)                                                                                                     \
      lm_head_wide_kernel<W_FP8, GPLV, RLV, true><<<cus, 1024, lds, st>>>((const uint8_t*)W, s, V, K, x, logits, \
                                                                          argmax, counter, best, *smp);          \
    else                                                                                                         \
      lm_head_wide_kernel<W_FP8, GPLV, RLV, false><<<cus, 1024, lds, st>>>((const uint8_t*)W, s, V, K, x,        \
                                                                           logits, argmax, counter, best,        \
                                                                           HeadSample{});                        \
    *done = true;                                                                                                \
    return hipGetLastError();                                                                                    \
  }
  if (wt == W_FP8 && K == 2560) WSX_WIDE_S(10, 16)
  if (wt == W_FP8 && K == 256) WSX_WIDE_S(1, 16)
  if (smp) return hipSuccess;
  if (wt == W_BF16 && K == 2560) WSX_WIDE(W_BF16, 10, 32)
  if (wt == W_BF16 && K == 256) WSX_WIDE(W_BF16, 1, 32)
#undef WSX_WIDE
#undef WSX_WIDE_S
  return hipSuccess;
}

// chunk maxima, then workgroup maxima
size_t head_sample_fused_ws_bytes(int) { return (size_t)kSampFusedMaxGrid * (16 + 1) * sizeof(RankKey); }

// Whether the sampling variant of the wide FP8 head takes (V, K, top_k) on a
// device of `cus` compute units: the wide head's shapes, at most
// kSampFusedMaxGrid workgroups, every wavefront streaming at most 64 rows, and
// at least top_k workgroups with rows (the selection's first cut).
bool head_sample_fused_fits(int V, int K, int top_k, int cus) {
  if (K != 2560 && K != 256) return false;
  if ((size_t)V * K >= ((size_t)1 << 31) || V < 1) return false;
  if (cus < 1 || cus > kSampFusedMaxGrid || top_k < 1 || top_k > kSampMaxK || top_k > V) return false;
  constexpr int RPW = 4;                               // rows per group of the FP8 wide head (16 lanes a row)
  const int NG = (V + RPW - 1) / RPW;
  const int stride = cus * 16;
  const int groups_per_wave = (NG + stride - 1) / stride;
  const int wgs_with_rows = min(cus, (NG + 15) / 16);
  return groups_per_wave * RPW <= kSampFusedMaxChunkRows && wgs_with_rows >= top_k;
}

int head_sample_fused_path(int V, int K, int top_k) {
  int cus = 0;
  if (device_cus(&cus) != hipSuccess) return 0;
  return head_sample_fused_fits(V, K, top_k, cus) ? 1 : 0;
}

hipError_t launch_lm_head_sample_fused(const void* W, const float* s, int V, int K, const uint16_t* x,
                                       float temperature, int top_k, float top_p, const float* uniforms,
                                       float* logits, int32_t* token, int32_t* topk_ids, float* topk_probs,
                                       void* head_ws, void* sample_ws, hipStream_t st, bool* done) {
  *done = false;
  if (!head_sample_fused_path(V, K, top_k)) return hipSuccess;
  int cus = 0;
  const hipError_t ce = device_cus(&cus);
  if (ce != hipSuccess) return ce;
  HeadSample smp;
  smp.chunk_max = reinterpret_cast<RankKey*>(sample_ws);
  smp.wg_max = smp.chunk_max + (size_t)cus * 16;
  smp.k = top_k;
  smp.temperature = temperature;
  smp.top_p = top_p;
  smp.uniforms = uniforms;
  smp.token = token;
  smp.topk_ids = topk_ids;
  smp.topk_probs = topk_probs;
  return launch_head_wide(W_FP8, W, s, V, K, x, logits, nullptr, reinterpret_cast<unsigned*>(head_ws), nullptr, st,
                          done, &smp);
}

hipError_t launch_lm_head(int wt, const void* W, const float* s, int V, int K, const uint16_t* x, int T, int norm,
                          uint16_t* u_out, float* logits, int32_t* argmax, void* ws, hipStream_t st) {
  unsigned* counter = reinterpret_cast<unsigned*>(ws);
  if (T == 1 && !norm) {
    bool done = false;
    const hipError_t e = launch_head_wide(wt, W, s, V, K, x, logits, argmax, counter,
                                          reinterpret_cast<unsigned long long*>((char*)ws + 64), st, &done);
    if (done || e != hipSuccess) return e;
  }
  if (T >= 2 && wt == W_FP8 && (K == 2560 || K == 256) && (size_t)V * K < ((size_t)1 << 31)) {
    // the wide head for the verify pass's rows: one 1024-thread workgroup per CU
    int cus = 0;
    const hipError_t ce = device_cus(&cus);
    if (ce != hipSuccess) return ce;
    {
      unsigned long long* best = reinterpret_cast<unsigned long long*>((char*)ws + 64);   // T words
      const size_t lds = (size_t)T * (K / 16) * 48;
#define WSX_WT(TV)                                                                                                  \
  if (T == TV) {                                                                                                    \
    if (K == 2560)                                                                                                  \
      lm_head_wide_t_kernel<TV, 10, 16><<<cus, 1024, lds, st>>>((const uint8_t*)W, s, V, K, x, norm, u_out, logits,  \
                                                                argmax, counter, best);                             \
    else                                                                                                            \
      lm_head_wide_t_kernel<TV, 1, 16><<<cus, 1024, lds, st>>>((const uint8_t*)W, s, V, K, x, norm, u_out, logits,   \
                                                               argmax, counter, best);                              \
    return hipGetLastError();                                                                                       \
  }
      WSX_WT(2) WSX_WT(3) WSX_WT(4)
#undef WSX_WT
    }
  }
  const int grid = head_grid(V);
  float* pv = reinterpret_cast<float*>((char*)ws + 256);
  int* pi = reinterpret_cast<int*>((char*)ws + 256 + (size_t)kHeadMaxGrid * WSX_MAX_T * 4);
#define WSX_T_CASE(WTV, TV) \
  if (wt == WTV && T == TV) return launch_head_t<WTV, TV>(W, s, V, K, x, norm, u_out, logits, argmax, counter, pv, pi, grid, st);
  WSX_T_CASE(W_FP8, 1) WSX_T_CASE(W_FP8, 2) WSX_T_CASE(W_FP8, 3) WSX_T_CASE(W_FP8, 4)
  WSX_T_CASE(W_BF16, 1) WSX_T_CASE(W_BF16, 2) WSX_T_CASE(W_BF16, 3) WSX_T_CASE(W_BF16, 4)
#undef WSX_T_CASE
  return hipErrorInvalidValue;
}

template <int WT, int T>
static hipError_t launch_router_t(const void* W, int E, int K, int k, const uint16_t* x, int norm, uint16_t* u_out,
                                  float* logits, int32_t* ids, float* w, int32_t* el, float* sw, unsigned* counter,
                                  hipStream_t st) {
  const int G = K / WTraits<WT>::EPG;
  const int rgpl = (G + 63) / 64;
  const int grid = (E + 3) / 4;
  const size_t lds = (size_t)T * K * 2;
  const bool small = E <= 512;
#define WSX_R_CASE(N)                                                                                              \
  case N:                                                                                                          \
    if (small)                                                                                                     \
      router_topk_kernel<WT, T, N, 2><<<grid, 256, lds, st>>>((const uint8_t*)W, E, K, k, x, norm, u_out, logits,  \
                                                              ids, w, el, sw, counter);                            \
    else                                                                                                           \
      router_topk_kernel<WT, T, N, 4><<<grid, 256, lds, st>>>((const uint8_t*)W, E, K, k, x, norm, u_out, logits,  \
                                                              ids, w, el, sw, counter);                            \
    break;
  switch (rgpl) {
    WSX_R_CASE(1) WSX_R_CASE(2) WSX_R_CASE(4) WSX_R_CASE(5) WSX_R_CASE(8) WSX_R_CASE(10) WSX_R_CASE(16)
    WSX_R_CASE(32)
    default: return hipErrorInvalidValue;
  }
#undef WSX_R_CASE
  return hipGetLastError();
}

bool router_shape_supported(int router_dtype, int K) {
  const int epg = router_dtype == WSX_DTYPE_F32 ? 4 : 8;
  if (K % 32 != 0 || K > kMaxK) return false;
  const int rgpl = (K / epg + 63) / 64;
  return rgpl == 1 || rgpl == 2 || rgpl == 4 || rgpl == 5 || rgpl == 8 || rgpl == 10 || rgpl == 16 || rgpl == 32;
}

template <int WT>
static hipError_t launch_router_grouped(const void* W, int E, int K, int k, const uint16_t* x, int T, float* logits,
                                        int32_t* ids, float* w, int32_t* el, float* sw, unsigned* counter,
                                        hipStream_t st) {
  const int G = K / WTraits<WT>::EPG;
  const int rgpl = (G + 63) / 64;
  const int grid = (E + 3) / 4;
  // the stages, and then the [T][E] logits in the last workgroup's tail
  const size_t lds = (size_t)kRouteChunk * K * 2 > (size_t)T * E * 4 ? (size_t)kRouteChunk * K * 2 : (size_t)T * E * 4;
  const bool small = E <= 512;
#define WSX_RG_CASE(N)                                                                                            \
  case N:                                                                                                         \
    if (small)                                                                                                    \
      router_topk_grouped_kernel<WT, N, 2><<<grid, 256, lds, st>>>((const uint8_t*)W, E, K, k, x, T, logits, ids, \
                                                                   w, el, sw, counter);                           \
    else                                                                                                          \
      router_topk_grouped_kernel<WT, N, 4><<<grid, 256, lds, st>>>((const uint8_t*)W, E, K, k, x, T, logits, ids, \
                                                                   w, el, sw, counter);                           \
    break;
  switch (rgpl) {
    WSX_RG_CASE(1) WSX_RG_CASE(2) WSX_RG_CASE(4) WSX_RG_CASE(5) WSX_RG_CASE(8) WSX_RG_CASE(10) WSX_RG_CASE(16)
    WSX_RG_CASE(32)
    default: return hipErrorInvalidValue;
  }
#undef WSX_RG_CASE
  return hipGetLastError();
}

hipError_t launch_router(int router_dtype, const void* W, int E, int K, int k, const uint16_t* x, int T, int norm,
                         uint16_t* u_out, float* logits, int32_t* ids, float* w, int32_t* el, float* sw,
                         unsigned* counter, hipStream_t st) {
  if (T > WSX_MAX_T) {
    if (norm) return hipErrorInvalidValue;   // the normalized (decode-step) router takes at most WSX_MAX_T tokens
    return router_dtype == WSX_DTYPE_F32
               ? launch_router_grouped<W_F32>(W, E, K, k, x, T, logits, ids, w, el, sw, counter, st)
               : launch_router_grouped<W_BF16>(W, E, K, k, x, T, logits, ids, w, el, sw, counter, st);
  }
#define WSX_T_CASE(DT, WTV, TV) \
  if (router_dtype == DT && T == TV) return launch_router_t<WTV, TV>(W, E, K, k, x, norm, u_out, logits, ids, w, el, sw, counter, st);
  WSX_T_CASE(WSX_DTYPE_BF16, W_BF16, 1) WSX_T_CASE(WSX_DTYPE_BF16, W_BF16, 2)
  WSX_T_CASE(WSX_DTYPE_BF16, W_BF16, 3) WSX_T_CASE(WSX_DTYPE_BF16, W_BF16, 4)
  WSX_T_CASE(WSX_DTYPE_F32, W_F32, 1) WSX_T_CASE(WSX_DTYPE_F32, W_F32, 2)
  WSX_T_CASE(WSX_DTYPE_F32, W_F32, 3) WSX_T_CASE(WSX_DTYPE_F32, W_F32, 4)
#undef WSX_T_CASE
  return hipErrorInvalidValue;
}

}  // namespace wsx
