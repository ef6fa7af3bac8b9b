// Temperature / top-k / top-p sampling of one token per row of the LM head's
// logits, on gfx950: the sampling epilogue of the head.
//
// [ncij] "What happens on a real workload?": the GSM8K run samples with
// temperature 0.6, top_p 0.95 and top_k 29.  The pages name only the three
// settings; the steps taken are: keep the top_k logits by (value desc, id
// asc); e_i = exp((z_i - z_0) / temperature); c_i the running sum in rank
// order; keep ranks 0..m, m the first with c_m >= top_p * c_{k-1}; p_i =
// e_i / c_m; the token is the first rank j <= m with c_j > u * c_m (m if
// none), u being the caller's uniform for that row.  That arithmetic is
// binary32 in this order.
//
// Two launches, both small next to the head itself:
//  1. candidates: one wavefront per 64-logit chunk, grid (ceil(V / 256), T).
//     Each lane forms the 64-bit rank key of its logit (order-preserving value
//     bits over the complemented id, so one unsigned compare orders by value,
//     ties to the lower id), ranks it against the other 63 keys broadcast by
//     readlane, and the lanes of rank < k write the chunk's top k to the
//     workspace; slots past a short chunk get key 0, below every finite
//     logit's key.
//  2. selection: one 1024-thread workgroup per row.  The k-th largest chunk
//     maximum tau (a radix select over the key bytes, stopping once one key
//     matches) bounds the k-th largest logit from below, so every global
//     top-k key is a candidate >= tau of one of the (at most k) chunks whose
//     maximum is >= tau: only those k * k candidates are read, in one round
//     of loads.  Ranking the survivors against each other gives the top k in
//     order; one wavefront then runs the sums in rank order and the draw.
#include "sample_device.h"
#include "wsx_internal.h"

namespace wsx {

constexpr int kSampChunk = 64;          // logits per chunk: one wavefront
constexpr int kSampMaxChunks = 8192;    // V <= 8191 * 64; also bounds the k * k survivors

__global__ void __launch_bounds__(256) sample_candidates_kernel(const float* __restrict__ logits, int V, int k,
                                                               int nchunk, RankKey* __restrict__ cand,
                                                               RankKey* __restrict__ maxima) {
  const int lane = threadIdx.x & 63;
  const int c = blockIdx.x * 4 + (threadIdx.x >> 6), t = blockIdx.y;
  if (c >= nchunk) return;   // whole wavefronts leave together
  const int v = c * kSampChunk + lane;
  const RankKey mine = v < V ? rank_key(logits[(size_t)t * V + v], v) : 0ull;
  // rank within the chunk: every other lane's key broadcast through readlane
  const unsigned hi = (unsigned)(mine >> 32), lo = (unsigned)mine;
  int r = 0;
#pragma unroll
  for (int j = 0; j < 64; ++j) {
    const RankKey o = ((RankKey)(unsigned)__builtin_amdgcn_readlane((int)hi, j) << 32) |
                      (unsigned)__builtin_amdgcn_readlane((int)lo, j);
    r += (int)(o > mine);
  }
  RankKey* out = cand + ((size_t)t * nchunk + c) * k;
  if (mine != 0ull && r < k) out[r] = mine;
  if (mine != 0ull && r == 0) maxima[(size_t)t * nchunk + c] = mine;   // also packed, for the threshold
  const int nvalid = min(kSampChunk, V - c * kSampChunk);
  if (lane >= nvalid && lane < k) out[lane] = 0ull;
}

__global__ void __launch_bounds__(1024) sample_select_kernel(const RankKey* __restrict__ cand,
                                                            const RankKey* __restrict__ maxima, int nchunk, int k,
                                                            float temperature, float top_p,
                                                            const float* __restrict__ uniforms,
                                                            int32_t* __restrict__ token, int32_t* __restrict__ topk_ids,
                                                            float* __restrict__ topk_probs) {
  __shared__ __attribute__((aligned(16))) RankKey buf[kSampMaxChunks];
  __shared__ RankKey top[kSampMaxK];
  __shared__ int qlist[kSampMaxK];
  __shared__ unsigned hist[256];
  __shared__ RankKey tau;
  __shared__ int ns, nq, sel_digit, sel_need, sel_count;
  const int t = blockIdx.x;
  const RankKey* ct = cand + (size_t)t * nchunk * k;
  const float u = threadIdx.x < 64 ? uniforms[t] : 0.f;   // in flight from the start
  if (threadIdx.x == 0) {
    tau = 1ull;   // no cut when there are fewer than k chunks
    ns = 0;
    nq = 0;
  }
  // every chunk maximum, from the packed copy
  for (int c = threadIdx.x; c < nchunk; c += blockDim.x) buf[c] = maxima[(size_t)t * nchunk + c];
  __syncthreads();
  if (nchunk >= k) {
    // tau = the k-th largest maximum, by radix select: up to eight passes over
    // the key bytes from the top, each a histogram of the keys that match the
    // digits chosen so far and a scan by one wavefront for the byte that holds
    // the k-th largest, stopping once a single key matches (the maxima are
    // distinct, so the result is one key)
    RankKey prefix = 0ull, mask = 0ull;
    int need = k;
    bool found = false;
    for (int shift = 56; shift >= 0; shift -= 8) {
      if (threadIdx.x < 256) hist[threadIdx.x] = 0u;
      __syncthreads();
      for (int c = threadIdx.x; c < nchunk; c += blockDim.x) {
        const RankKey key = buf[c];
        if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (threadIdx.x < 64) {
        // lane l holds bins 255 - 4l .. 252 - 4l: digits in descending order
        const int lane = threadIdx.x;
        unsigned h[4], sum = 0u;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          h[q] = hist[255 - 4 * lane - q];
          sum += h[q];
        }
        unsigned incl = sum;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
          const unsigned v = __shfl_up(incl, d, 64);
          if (lane >= d) incl += v;
        }
        unsigned run = incl - sum;   // keys in higher digits
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (run < (unsigned)need && (unsigned)need <= run + h[q]) {
            sel_digit = 255 - 4 * lane - q;
            sel_need = need - (int)run;
            sel_count = (int)h[q];
          }
          run += h[q];
        }
      }
      __syncthreads();
      prefix |= (RankKey)sel_digit << shift;
      mask |= (RankKey)255u << shift;
      need = sel_need;
      if (sel_count == 1) {
        // one key has these leading digits: it is the k-th largest
        for (int c = threadIdx.x; c < nchunk; c += blockDim.x)
          if ((buf[c] & mask) == prefix) tau = buf[c];
        found = true;
        break;
      }
      __syncthreads();   // every thread has read the choice before the next pass
    }
    // the distinct maxima leave one match by the last byte at the latest
    if (!found && threadIdx.x == 0) tau = prefix;
  }
  __syncthreads();
  const RankKey th = tau;
  // the chunks whose maximum is >= tau: exactly k of them when there are at
  // least k chunks (distinct maxima), else all nchunk < k
  for (int c = threadIdx.x; c < nchunk; c += blockDim.x)
    if (buf[c] >= th) {
      const int pos = atomicAdd(&nq, 1);
      if (pos < kSampMaxK) qlist[pos] = c;
    }
  __syncthreads();   // buf is reused for the survivors below
  // their candidates (<= k * k <= 4096 keys): all loads issued at once
  const int nload = min(nq, kSampMaxK) * k;
  RankKey kv[kSampMaxK * kSampMaxK / 1024];
#pragma unroll
  for (int r = 0; r < kSampMaxK * kSampMaxK / 1024; ++r) {
    const int i = threadIdx.x + r * 1024;
    kv[r] = i < nload ? ct[(size_t)qlist[i / k] * k + i % k] : 0ull;
  }
#pragma unroll
  for (int r = 0; r < kSampMaxK * kSampMaxK / 1024; ++r)
    if (kv[r] != 0ull && kv[r] >= th) {
      const int pos = atomicAdd(&ns, 1);
      if (pos < kSampMaxChunks) buf[pos] = kv[r];
    }
  __syncthreads();
  const int n = min(ns, kSampMaxChunks);
  if (threadIdx.x == 0 && (n & 1)) buf[n] = 0ull;
  __syncthreads();
  wg_rank_keys(buf, n, [&](int i, int r) {
    if (r < k) top[r] = buf[i];
  });
  __syncthreads();
  if (threadIdx.x < 64)
    sample_draw_wave((int)threadIdx.x < k ? top[threadIdx.x] : 0ull, k, temperature, top_p, u, token + t,
                     topk_ids ? topk_ids + (size_t)t * k : nullptr, topk_probs ? topk_probs + (size_t)t * k : nullptr);
}

size_t sample_ws_bytes(int T, int V, int k) {
  const size_t nchunk = ((size_t)V + kSampChunk - 1) / kSampChunk;
  return (size_t)T * nchunk * ((size_t)k + 1) * sizeof(RankKey);   // candidates, then the packed maxima
}

bool sample_shape_supported(int V, int k) {
  return V >= 1 && k >= 1 && k <= kSampMaxK && k <= V && (V + kSampChunk - 1) / kSampChunk <= kSampMaxChunks - 1;
}

hipError_t launch_sample(const float* logits, int V, int T, float temperature, int k, float top_p,
                         const float* uniforms, int32_t* token, int32_t* topk_ids, float* topk_probs, void* ws,
                         hipStream_t st) {
  const int nchunk = (V + kSampChunk - 1) / kSampChunk;
  RankKey* cand = reinterpret_cast<RankKey*>(ws);
  RankKey* maxima = cand + (size_t)T * nchunk * k;
  sample_candidates_kernel<<<dim3((nchunk + 3) / 4, T), 256, 0, st>>>(logits, V, k, nchunk, cand, maxima);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  sample_select_kernel<<<T, 1024, 0, st>>>(cand, maxima, nchunk, k, temperature, top_p, uniforms, token, topk_ids,
                                           topk_probs);
  return hipGetLastError();
}

}  // namespace wsx
