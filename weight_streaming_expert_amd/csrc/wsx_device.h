// Device helpers for the gfx950 (CDNA4) decode-path kernels: number-format
// conversions on the hardware converters, 128-bit block dot products and
// wave64 reductions.  Internal header; not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wsx {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

constexpr int kWave = 64;

// ---------------------------------------------------------------- formats

// E8M0 block scale byte -> 2^(b-127) as a binary32 (b = 0 is the subnormal 2^-127).
__device__ __forceinline__ float e8m0_to_f32(uint32_t b) {
  return b ? __uint_as_float(b << 23) : __uint_as_float(0x00400000u);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// binary32 -> bf16 bits, round to nearest even (inputs are finite).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Two E2M1 codes (byte `sel` of w: low nibble = even element) -> two bf16, exact.
template <int SEL>
__device__ __forceinline__ bf16x2_t fp4x2_to_bf16x2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, SEL);
}
// Two E2M1 codes -> two fp32, exact.
template <int SEL>
__device__ __forceinline__ f32x2_t fp4x2_to_f32x2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
}
// Two E4M3FN codes (half `HI` of w: byte 2*HI is the first element) -> two bf16, exact.
template <bool HI>
__device__ __forceinline__ bf16x2_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI);
}

__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t w) { return __builtin_bit_cast(bf16x2_t, w); }

// Eight E2M1 codes (one dword, element 2j in the low nibble of byte j) times
// their power-of-two block scale -> eight bf16, exact (the matrix cores' A
// operand for 8 consecutive elements).
__device__ __forceinline__ bf16x8_t fp4x8_to_bf16x8(uint32_t w, float scale) {
  const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0);
  const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1);
  const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2);
  const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3);
  bf16x8_t r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

__device__ __forceinline__ float dot2(bf16x2_t a, bf16x2_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(a, b, c, false);
}

// ---------------------------------------------------------------- block dot products
// Each takes one 16-byte granule of weights and the matching activations as
// packed bf16 pairs, and returns the fp32 dot product (unscaled).

// MXFP4: 32 E2M1 codes (one MX block) x 32 bf16 activations (16 dwords).
__device__ __forceinline__ float mx_block_dot(uint4 c, const uint32_t* xp) {
  float a0 = 0.f, a1 = 0.f;
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    a0 = dot2(fp4x2_to_bf16x2<0>(w[d]), as_bf16x2(xp[4 * d + 0]), a0);
    a1 = dot2(fp4x2_to_bf16x2<1>(w[d]), as_bf16x2(xp[4 * d + 1]), a1);
    a0 = dot2(fp4x2_to_bf16x2<2>(w[d]), as_bf16x2(xp[4 * d + 2]), a0);
    a1 = dot2(fp4x2_to_bf16x2<3>(w[d]), as_bf16x2(xp[4 * d + 3]), a1);
  }
  return a0 + a1;
}

// E4M3FN: 16 codes x 16 bf16 activations (8 dwords).
__device__ __forceinline__ float fp8_granule_dot(uint4 c, const uint32_t* xp) {
  float a0 = 0.f, a1 = 0.f;
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    a0 = dot2(fp8x2_to_bf16x2<false>(w[d]), as_bf16x2(xp[2 * d + 0]), a0);
    a1 = dot2(fp8x2_to_bf16x2<true>(w[d]), as_bf16x2(xp[2 * d + 1]), a1);
  }
  return a0 + a1;
}

// bf16: 8 weights x 8 bf16 activations (4 dwords).
__device__ __forceinline__ float bf16_granule_dot(uint4 c, const uint32_t* xp) {
  float a0 = dot2(as_bf16x2(c.x), as_bf16x2(xp[0]), 0.f);
  float a1 = dot2(as_bf16x2(c.y), as_bf16x2(xp[1]), 0.f);
  a0 = dot2(as_bf16x2(c.z), as_bf16x2(xp[2]), a0);
  a1 = dot2(as_bf16x2(c.w), as_bf16x2(xp[3]), a1);
  return a0 + a1;
}

// fp32: 4 weights x 4 bf16 activations (2 dwords), fp32 FMAs.
__device__ __forceinline__ float f32_granule_dot(uint4 c, const uint32_t* xp) {
  float a = __uint_as_float(c.x) * bf16_bits_to_f32(xp[0] & 0xFFFFu);
  a = fmaf(__uint_as_float(c.y), bf16_bits_to_f32(xp[0] >> 16), a);
  a = fmaf(__uint_as_float(c.z), bf16_bits_to_f32(xp[1] & 0xFFFFu), a);
  a = fmaf(__uint_as_float(c.w), bf16_bits_to_f32(xp[1] >> 16), a);
  return a;
}

// ---------------------------------------------------------------- cross-lane reductions

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// DPP controls (gfx9 encoding)
constexpr int kQuadSwap1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;

// Sum over each aligned group of 8 lanes; every lane of the group gets the sum.
// The addition tree is the same for every group and every lane.
__device__ __forceinline__ float sum8(float v) {
  v += dpp_f<kQuadSwap1>(v);
  v += dpp_f<kQuadSwap2>(v);
  v += dpp_f<kRowHalfMirror>(v);
  return v;
}
// Sum over each 16-lane DPP row.
__device__ __forceinline__ float sum16(float v) {
  v = sum8(v);
  v += dpp_f<kRowMirror>(v);
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
  v = sum16(v);
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

__device__ __forceinline__ float readlane_f(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Sum over the wavefront in one fixed order without LDS traffic: the DPP tree
// within each row of 16 lanes, then rows 0 + 1 + 2 + 3.  The result is uniform.
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v = sum16(v);
  return ((readlane_f(v, 0) + readlane_f(v, 16)) + readlane_f(v, 32)) + readlane_f(v, 48);
}

// Maximum over the wavefront (DPP within rows, then the four row maxima).
__device__ __forceinline__ float wave_max_dpp(float v) {
  v = fmaxf(v, dpp_f<kQuadSwap1>(v));
  v = fmaxf(v, dpp_f<kQuadSwap2>(v));
  v = fmaxf(v, dpp_f<kRowHalfMirror>(v));
  v = fmaxf(v, dpp_f<kRowMirror>(v));
  return fmaxf(fmaxf(readlane_f(v, 0), readlane_f(v, 16)), fmaxf(readlane_f(v, 32), readlane_f(v, 48)));
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// (value, index) argmax over the wave: larger value wins, equal values go to
// the lower index.  Every lane returns the winner.
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    float ov = __shfl_xor(v, o);
    int oi = __shfl_xor(i, o);
    if (ov > v || (ov == v && oi < i)) { v = ov; i = oi; }
  }
}

// (v, i) ranks before (bv, bi): larger value, then lower index.  Written
// without short-circuit operators so it compiles to compares and mask logic,
// never to branches.
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return (v > bv) | ((v == bv) & (i < bi));
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

// A value's rank key: the value's bits mapped to an unsigned integer that
// orders as the value does (-0 taken as +0), above the complement of the id.
// A larger key ranks before: larger value, then lower id.
using RankKey = unsigned long long;
__device__ __forceinline__ RankKey rank_key(float v, int id) {
  const unsigned b = __float_as_uint(v + 0.0f);
  const unsigned o = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((RankKey)o << 32) | (unsigned)~id;
}
__device__ __forceinline__ float key_value(RankKey key) {
  const unsigned o = (unsigned)(key >> 32);
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}
__device__ __forceinline__ int key_id(RankKey key) { return (int)~(unsigned)key; }


// ---------------------------------------------------------------- memory

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// Copy n16 16-byte chunks from global memory to LDS with NT threads.  Every
// thread issues all of its loads (at most MAXC) before the first LDS store, so
// the copy costs one memory latency instead of one per loop trip.  Chunks past
// MAXC * NT are copied by a plain trailing loop (only reached by callers that
// pass sizes beyond their fast path).
template <int NT, int MAXC>
__device__ __forceinline__ void stage_to_lds(const void* __restrict__ src, void* dst, int n16) {
  const uint4* s = reinterpret_cast<const uint4*>(src);
  uint4* d = reinterpret_cast<uint4*>(dst);
  uint4 v[MAXC];
#pragma unroll
  for (int j = 0; j < MAXC; ++j) {
    const int i = threadIdx.x + j * NT;
    v[j] = make_uint4(0, 0, 0, 0);
    if (i < n16) v[j] = s[i];
  }
#pragma unroll
  for (int j = 0; j < MAXC; ++j) {
    const int i = threadIdx.x + j * NT;
    if (i < n16) d[i] = v[j];
  }
  for (int i = threadIdx.x + MAXC * NT; i < n16; i += NT) d[i] = s[i];
}

// Wait until every vector memory operation this wave issued has completed, in
// particular until its device-coherent stores have been acknowledged.  The
// memory clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Workgroup barrier for data exchanged through LDS only.  __syncthreads() is
// also a workgroup-scope release fence, which waits for every outstanding
// vector memory access of the wavefront (vmcnt(0)), including loads meant to
// stay in flight across the barrier.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Compiler-only barrier: keeps the loads issued before it (prefetches meant to
// be in flight during a wait) from being sunk past it to their first use.
// Emits no instruction and does not wait for the loads.
__device__ __forceinline__ void issue_here() { asm volatile("" ::: "memory"); }

// Device-coherent (sc1) 8- and 16-byte accesses through buffer instructions.
// They are performed at the device coherence point, so data written this way
// by one workgroup is read back current by any other workgroup on any XCD,
// without cache-wide writeback or invalidation.
constexpr int kCoherent = 16;   // cache-policy bits: sc1
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7FFFFFFF, 0x00020000);
}
__device__ __forceinline__ uint4 ld_coh16(const void* base, uint32_t byte_off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(buf_rsrc(base), byte_off, 0, kCoherent));
}
__device__ __forceinline__ uint2 ld_coh8(const void* base, uint32_t byte_off) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(buf_rsrc(base), byte_off, 0, kCoherent));
}
__device__ __forceinline__ void st_coh16(void* base, uint32_t byte_off, uint4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned, v),
                                         buf_rsrc(base), byte_off, 0, kCoherent);
}
__device__ __forceinline__ void st_coh8(void* base, uint32_t byte_off, uint2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(__attribute__((ext_vector_type(2))) unsigned, v),
                                        buf_rsrc(base), byte_off, 0, kCoherent);
}
__device__ __forceinline__ void st_coh4(void* base, uint32_t byte_off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b32(v, buf_rsrc(base), byte_off, 0, kCoherent);
}
__device__ __forceinline__ uint32_t ld_coh4(const void* base, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b32(buf_rsrc(base), byte_off, 0, kCoherent);
}

// Device-coherent accesses for data exchanged between workgroups inside one
// launch.  Agent-scope relaxed atomics are performed at the device coherence
// point (they bypass the per-XCD L2 for coherence), so no cache-wide
// writeback or invalidate is needed: a store is visible device-wide once it
// has been acknowledged (vmcnt), and such a load never returns a stale line.
__device__ __forceinline__ void st_dev(float* p, float v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ void st_dev(int* p, int v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ float ld_dev(const float* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ int ld_dev(const int* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }

// Last-arriver election.  Every workgroup calls this once, after publishing its
// partial results with st_dev; exactly one workgroup (the last to arrive) gets
// true, and may then read every partial with ld_dev.  Each wave first waits
// until its own device-coherent stores are acknowledged (a workgroup-scope
// fence alone does not wait for them), the barrier then covers the whole
// workgroup before the counter increment.  The winner returns the counter to
// zero, so it is reusable by the next launch without clearing.
__device__ __forceinline__ bool last_block_arrived(unsigned* counter, unsigned nblocks, int* smem_flag) {
  wait_vmem();
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned old = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *smem_flag = (old == nblocks - 1);
    if (old == nblocks - 1) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  return *smem_flag != 0;
}

}  // namespace wsx
