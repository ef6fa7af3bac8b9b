// Pure-read bandwidth probe: the HBM rate a plain streaming read reaches on
// this GPU, the practical ceiling beside the published 8 TB/s peak for the
// weight streams of the decode path ([ncij] "Why is MoE decoding on DGX Spark
// memory-bound?": decode time is set by how fast weights come out of memory).
//
// Every thread issues a chunk's 16-byte nontemporal loads before using any
// of them; each workgroup folds what it read into one word with an atomic XOR
// so the loads cannot be removed.
#include "wsx_device.h"
#include "wsx_internal.h"

namespace wsx {

namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeLoads = 8;   // 16-byte loads in flight per thread
constexpr size_t kProbeGrid = 2048;   // eight 256-thread workgroups per CU

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(kProbeThreads) read_probe_kernel(const uint4* __restrict__ src, size_t n16,
                                                                   uint32_t* out) {
  // chunks of kProbeThreads * kProbeLoads granules, taken grid-stride, so a
  // few workgroups per CU stream the whole buffer and only they fold their
  // results into `out`
  const size_t per_chunk = (size_t)kProbeThreads * kProbeLoads;
  const size_t nchunks = (n16 + per_chunk - 1) / per_chunk;
  uint32_t acc = 0;
  for (size_t c = blockIdx.x; c < nchunks; c += gridDim.x) {
    const size_t base = c * per_chunk + threadIdx.x;
    u32x4_t v[kProbeLoads];
#pragma unroll
    for (int j = 0; j < kProbeLoads; ++j) {
      const size_t i = base + (size_t)j * kProbeThreads;
      v[j] = i < n16 ? __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(src + i)) : u32x4_t{0, 0, 0, 0};
    }
#pragma unroll
    for (int j = 0; j < kProbeLoads; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  }
  acc ^= __shfl_xor(acc, 32);
  acc ^= __shfl_xor(acc, 16);
  acc ^= __shfl_xor(acc, 8);
  acc ^= __shfl_xor(acc, 4);
  acc ^= __shfl_xor(acc, 2);
  acc ^= __shfl_xor(acc, 1);
  __shared__ uint32_t wacc[kProbeThreads / 64];
  if ((threadIdx.x & 63) == 0) wacc[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t a = 0;
    for (int w = 0; w < kProbeThreads / 64; ++w) a ^= wacc[w];
    __hip_atomic_fetch_xor(out, a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace

hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* out, hipStream_t st) {
  const size_t n16 = bytes / 16;
  const size_t per_chunk = (size_t)kProbeThreads * kProbeLoads;
  const size_t nchunks = (n16 + per_chunk - 1) / per_chunk;
  const size_t grid = nchunks < kProbeGrid ? nchunks : kProbeGrid;
  if (grid == 0) return hipSuccess;
  read_probe_kernel<<<(unsigned)grid, kProbeThreads, 0, st>>>(reinterpret_cast<const uint4*>(buf), n16, out);
  return hipGetLastError();
}

}  // namespace wsx
