// Device pieces shared by the two-launch sampler (sample.hip) and the sampling
// tail of the 1-token FP8 head (gemv_rows.hip): ranking keys held in LDS with
// the whole workgroup, and the draw over the top-k keys by one wavefront.
//
// [ncij] "What happens on a real workload?": the GSM8K run samples with
// temperature 0.6, top_p 0.95 and top_k 29.  The draw below takes the reading
// stated in sample.hip: e_i = exp((z_i - z_0) / temperature) over the top-k
// logits in rank order, running binary32 sums c_i in that order, the nucleus
// cut m = the first rank with c_m >= top_p * c_{k-1}, probabilities e_i / c_m,
// and the token = the first rank j <= m with c_j > u * c_m (m if none).
#pragma once
#include "wsx_device.h"

namespace wsx {

constexpr int kSampMaxK = 64;

__device__ __forceinline__ RankKey readlane_key(RankKey v, int lane) {
  return ((RankKey)(unsigned)__builtin_amdgcn_readlane((int)(unsigned)(v >> 32), lane) << 32) |
         (unsigned)__builtin_amdgcn_readlane((int)(unsigned)v, lane);
}

// Count of the keys in buf[lo..hi) (hi - lo even, 16-byte aligned pairs)
// greater than m, reading eight keys per step so that four LDS reads are in
// flight together.
__device__ __forceinline__ int count_greater(const RankKey* buf, int lo, int hi, RankKey m) {
  int r = 0, j = lo;
  for (; j + 8 <= hi; j += 8) {
    const ulonglong2 a = *reinterpret_cast<const ulonglong2*>(buf + j);
    const ulonglong2 b = *reinterpret_cast<const ulonglong2*>(buf + j + 2);
    const ulonglong2 c = *reinterpret_cast<const ulonglong2*>(buf + j + 4);
    const ulonglong2 d = *reinterpret_cast<const ulonglong2*>(buf + j + 6);
    r += (int)(a.x > m) + (int)(a.y > m) + (int)(b.x > m) + (int)(b.y > m) + (int)(c.x > m) + (int)(c.y > m) +
         (int)(d.x > m) + (int)(d.y > m);
  }
  for (; j < hi; j += 2) {
    const ulonglong2 a = *reinterpret_cast<const ulonglong2*>(buf + j);
    r += (int)(a.x > m) + (int)(a.y > m);
  }
  return r;
}

// Rank of every key buf[i], i < n, among buf[0..n): r = #{j : buf[j] > buf[i]}
// (a larger key ranks first; the keys are distinct apart from zeros).  When n
// is odd, buf[n] must hold 0.  Every thread of the workgroup calls this and
// act(i, r) runs once per key; there is no barrier inside (the caller syncs
// before reading what act wrote).  Up to 16 keys per wavefront, wavefront w
// takes keys 16 w .. 16 w + 15 and four lanes scan a quarter of the keys each
// for one key, their counts meeting by shuffles; beyond that each thread
// ranks whole keys.
template <class Act>
__device__ __forceinline__ void wg_rank_keys(const RankKey* buf, int n, Act act) {
  const int tid = (int)threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = (int)blockDim.x >> 6;
  const int n2 = (n + 1) & ~1;
  if (n <= 16 * nw) {
    const int i = wave * 16 + (lane & 15), s = lane >> 4;
    const int q = ((n2 / 2 + 3) / 4) * 2;   // keys per quarter, even
    int r = 0;
    if (i < n) {
      const int lo = min(n2, s * q), hi = min(n2, lo + q);
      r = count_greater(buf, lo, hi, buf[i]);
    }
    r += __shfl_xor(r, 16);
    r += __shfl_xor(r, 32);
    if (s == 0 && i < n) act(i, r);
  } else {
    for (int i = tid; i < n; i += (int)blockDim.x) act(i, count_greater(buf, 0, n2, buf[i]));
  }
}

// The draw over the top k keys held one per lane in rank order (lane i holds
// rank i; a zero key marks a missing candidate and yields token -1), by the
// 64 lanes of one wavefront.  The running sums are a left fold in rank order
// (one add per rank, as the definition orders them); the cut and the draw are
// the first lanes that pass their tests, found by ballots.  u: the caller's
// uniform, the same in every lane.
__device__ __forceinline__ void sample_draw_wave(RankKey key, int k, float temperature, float top_p, float u,
                                                 int32_t* token, int32_t* topk_ids, float* topk_probs) {
  const int lane = (int)threadIdx.x & 63;
  const bool in = lane < k;
  const RankKey top0 = readlane_key(key, 0);
  const float z0 = key_value(top0);
  const float e = in ? expf((key_value(key) - z0) / temperature) : 0.f;
  float acc = 0.f, c = 0.f;
  for (int i = 0; i < k; ++i) {
    acc += readlane_f(e, i);
    if (lane == i) c = acc;
  }
  const float thr = top_p * acc;
  const unsigned long long cut = __ballot(in && c >= thr);
  const int m = cut ? __builtin_ctzll(cut) : k - 1;   // the first such rank
  const float mass = readlane_f(c, m);
  const float target = u * mass;
  const unsigned long long hit = __ballot(lane <= m && c > target);
  const int j = hit ? __builtin_ctzll(hit) : m;
  const unsigned tlo = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)key, j);
  if (lane == 0) token[0] = top0 == 0ull ? -1 : (int)~tlo;
  if (in) {
    if (topk_ids) topk_ids[lane] = key_id(key);
    if (topk_probs) topk_probs[lane] = lane <= m ? e / mass : 0.f;
  }
}

}  // namespace wsx
