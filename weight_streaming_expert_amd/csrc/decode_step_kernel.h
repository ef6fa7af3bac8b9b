// One decode step (T = 1) of the stacked MoE layers plus the FP8 LM head in a
// single launch on gfx950.
//
// [saipien] "Why one user waits on weights": at batch size 1 the step is a
// stream of weight reads (8 of 512 routed experts plus the shared expert per
// layer, then the 157,184-row vocabulary projection); [saipien] "Stop hauling
// the vocabulary in full precision" for the FP8 head; [ncij] "What happens on
// a real workload?" for greedy decoding.
//
// Why one launch: a kernel boundary in a captured graph costs ~1.7 us on
// MI355X and a layer has three all-to-all dependencies (the full residual
// stream before the router, all router logits before the top-k, all expert
// activations before the down projection), so per-kernel phases would pay
// ~100 boundaries per step.  Here every phase of every layer is a set of
// workgroups of one grid, in dependency order:
//
//   per layer l:  R (router rows)  S (shared gate/up tiles)  G (routed gate/up
//                 tiles, k slots)  D (down rows over all slots, + residual)
//   then:         head rows and one argmax over all of them (a 64-bit atomic max)
//
// A workgroup only ever waits for data produced by workgroups with a LOWER
// index.  Workgroups are dispatched in index order, so the lowest-indexed
// unfinished workgroup never waits for anything unfinished, and the grid
// always drains.  Every wait is also bounded: on timeout it raises the step's
// error word, the step's later waits return at once and the step reports
// argmax = -1.  The error word holds the failed step's tag base, so it never
// affects another step, and the step's last workgroup clears it.
//
// Data crosses workgroups only through device-coherent (sc1) stores and loads,
// performed at the device coherence point, and every exchanged value travels
// with a tag (step and layer) in the same 8-byte store, so a reader that sees
// the tag sees the value and no cache-wide fence is needed.  The exchange
// buffers are reused from layer to layer: a layer only overwrites them after
// every reader of the previous layer has provably finished (each such reader
// is an ancestor of the data the writer waited for).  Weights that do not
// depend on routing (the router rows, the shared expert, the first head rows)
// are loaded BEFORE a workgroup starts waiting, so their HBM reads overlap the
// earlier phases.  A workgroup that is dispatched long before its inputs can
// exist first sleeps on one word of the stage before (cheap), and only then
// polls its whole input.
//
// This header holds the kernel and its device code only, so that the same
// text serves the ahead-of-time build (decode_step.hip instantiates it for the
// shapes compiled in) and the run-time compilation of other shapes through
// hipRTC (its standard headers are then stand-ins the library supplies).
#pragma once

#include "wsx_device.h"
#include "../../include/wsx.h"

namespace wsx {

namespace {

constexpr int NT = 256;            // threads per workgroup
constexpr int kRRows = 8;          // router rows per R workgroup
constexpr int kRouteGroups = 2 * NT / 8;   // groups of 8 logits in the routing (E <= 2 NT)
constexpr int kRouteCand = 8;      // groups whose logits are ranked in full (>= k)
static_assert(kRouteCand >= WSX_MAX_K && kRouteCand * 8 == kRouteGroups, "routing candidate layout");
constexpr int kGRows = 16;         // intermediate values per S/G workgroup
constexpr int kDRows = 8;          // output rows per D workgroup
constexpr int kSpinMax = 1 << 17;  // polls before a wait gives up
constexpr unsigned kEpochMod = (1u << 24) - 1;   // epochs cycle in [0, kEpochMod)
// Copies of each exchange buffer: every consumer polls the copy picked by its
// workgroup index, so no single cache line is hammered by hundreds of pollers.
// Each copy also costs its producer a store, so more copies is not better:
// at the Ling shape 4 copies of the logits and of the activations beat 8 and
// 16 (the residual stream's 8 are fixed by the down role's lane mapping).
constexpr int kCopiesH = 8;        // residual stream (one copy per 8 lanes of the publishing wavefront)
constexpr int kCopiesLg = 4;       // router logits
constexpr int kCopiesA = 4;        // expert activations

struct Ctl {   // control words, each on its own 256-byte line
  unsigned epoch;
  unsigned pad0[63];
  unsigned err;
  unsigned pad1[63];
  unsigned top_counter;
  unsigned pad2[63];
  unsigned long long best;   // the step's best head rank key so far (0: none)
  unsigned pad3[62];
};

}  // namespace

struct FusedBufs {
  void* ctl;                 // Ctl
  uint2* hx;                 // [kCopiesH][2][H/2] (bf16 pair, tag); h_l lives in [.][l & 1] (l >= 1)
  uint2* lg;                 // [kCopiesLg][E] (logit, tag) of the current layer
  uint2* a;                  // [kCopiesA][nslot][I] (activation, tag) of the current layer
};

struct FusedStepArgs {
  const void* router;
  const uint8_t *w13c, *w13s, *w2c, *w2s;
  const uint8_t *sh13c, *sh13s, *sh2c, *sh2s;
  const uint8_t* hq;
  const float* hs;
  const uint16_t* h_in;
  uint16_t* h_out;
  float* logits;
  int32_t* argmax;
  uint16_t* h_trace;
  uint16_t* u_trace;
  int32_t* ids_trace;
  float* w_trace;
  FusedBufs b;
  int L, H, I, E, k, V;
  int nslot, nR, nS, nG, nD, per_layer, n_head;
  int block0;   // index of this launch's first workgroup in the step's workgroup order
};

namespace {

__device__ __forceinline__ Ctl* ctl(const FusedStepArgs& A) { return reinterpret_cast<Ctl*>(A.b.ctl); }
// The error word of a step holds that step's tag base ((epoch + 1) << 8, never
// zero), taken from any of the step's tags.  It is raised before the raising
// workgroup stores anything else (the store is acknowledged first), so every
// workgroup that later sees one of its outputs also sees the error.
__device__ __forceinline__ unsigned err_word(unsigned tag) { return tag & ~0xFFu; }
__device__ __forceinline__ void raise_err(const FusedStepArgs& A, unsigned tag) {
  st_dev(reinterpret_cast<int*>(&ctl(A)->err), (int)err_word(tag));
  wait_vmem();
}
__device__ __forceinline__ bool err_set(const FusedStepArgs& A, unsigned tag) {
  return (unsigned)ld_dev(reinterpret_cast<const int*>(&ctl(A)->err)) == err_word(tag);
}

// LDS layouts of the normalized activations, chosen so that the 8 lanes a
// 16-byte LDS read serves at once hit disjoint banks:
//   LayPlain  element i at i (router rows: lanes read consecutive 16-byte granules)
//   LayMX     32-element MX blocks at an 80-byte stride (gate/up: lane c reads block c)
//   LayHead   16-element FP8 granules at a 48-byte stride (head: lane c reads granule c)
struct LayPlain {
  static __device__ __forceinline__ int pos(int i) { return i; }
  static constexpr int bytes(int H) { return H * 2; }
};
struct LayMX {
  static __device__ __forceinline__ int pos(int i) { return (i >> 5) * 40 + (i & 31); }
  static constexpr int bytes(int H) { return H / 32 * 80; }
};
struct LayHead {
  static __device__ __forceinline__ int pos(int i) { return (i >> 4) * 24 + (i & 15); }
  static constexpr int bytes(int H) { return H / 16 * 48; }
};
// Expert activations in LDS: per slot, 32-value blocks at a 144-byte stride.
__device__ __forceinline__ int apos(int s, int i, int I) { return s * (I / 32) * 36 + (i >> 5) * 36 + (i & 31); }

__device__ __forceinline__ uint2* hx_buf(const FusedStepArgs& A, int l, int c) {
  return A.b.hx + ((size_t)c * 2 + (l & 1)) * (A.H / 2);
}
__device__ __forceinline__ uint2* lg_buf(const FusedStepArgs& A, int c) { return A.b.lg + (size_t)c * A.E; }
__device__ __forceinline__ uint2* a_buf(const FusedStepArgs& A, int c) { return A.b.a + (size_t)c * A.nslot * A.I; }
__device__ __forceinline__ int my_copy(int copies) { return (int)(blockIdx.x % copies); }

// ---------------------------------------------------------------- waits

// Wavefront decision to stop waiting for data carrying `tag`: the wait has run
// too long, or another wait of the same step already failed.  Lane 0 decides
// for the wavefront.
__device__ __forceinline__ bool wave_should_bail(const FusedStepArgs& A, int it, unsigned tag) {
  int bail = 0;
  if ((threadIdx.x & 63) == 0) {
    if (it >= kSpinMax) { raise_err(A, tag); bail = 1; }
    else if ((it & 15) == 15 && err_set(A, tag)) bail = 1;
  }
  return __shfl(bail, 0) != 0;
}

// Sleep on the tag of one exchanged (value, tag) pair until it equals `want`.
// Used to wait cheaply for the stage before the one a workgroup needs; gives
// up quietly, since the full poll that follows has its own bound.
__device__ __forceinline__ void sleep_on_tag(const FusedStepArgs& A, const uint2* p, int index, unsigned want) {
  for (int it = 0; it < kSpinMax; ++it) {
    if (ld_coh4(p, (uint32_t)index * 8 + 4) == want) return;
    if ((it & 15) == 15 && err_set(A, want)) return;
    __builtin_amdgcn_s_sleep(8);
  }
}

// u_l = RNE_bf16(h_l * r) into LDS (layout Lay), r = 1/sqrt(mean(h_l^2) +
// 1e-6), once every pair of h_l carries `tag`.  Each thread polls QPT 16-byte
// chunks (two tagged bf16 pairs each; chunk q = thread + 256 i).  The sum of
// squares is formed from the same values in one fixed order (the thread's
// chunks, the DPP wavefront sum, then the four wavefronts in order), so every
// workgroup that needs u_l derives the same r and the same u_l.
template <int QPT, class Lay>
__device__ __forceinline__ void wait_u(const FusedStepArgs& A, int l, unsigned tag, uint16_t* xs, float* red) {
  const int nq = A.H / 4;
  const uint2* hxl = hx_buf(A, l, my_copy(kCopiesH));
  uint4 v[QPT];
  unsigned pend = 0;   // chunks of this thread still without `tag`; each pass re-reads only those
#pragma unroll
  for (int i = 0; i < QPT; ++i) {
    v[i] = make_uint4(0, 0, 0, 0);
    if ((int)threadIdx.x + NT * i < nq) pend |= 1u << i;
  }
  for (int it = 0;; ++it) {
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
      if (pend & (1u << i)) {
        const uint4 w = ld_coh16(hxl, (uint32_t)(threadIdx.x + NT * i) * 16);
        if ((w.y == tag) & (w.w == tag)) {
          v[i] = w;
          pend &= ~(1u << i);
        }
      }
    }
    if (__all(pend == 0)) break;
    if (wave_should_bail(A, it, tag)) break;
    __builtin_amdgcn_s_sleep(1);
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < QPT; ++i) {
    const float a = bf16_bits_to_f32(v[i].x & 0xFFFFu), b = bf16_bits_to_f32(v[i].x >> 16);
    const float c = bf16_bits_to_f32(v[i].z & 0xFFFFu), d = bf16_bits_to_f32(v[i].z >> 16);
    ss = fmaf(a, a, ss);
    ss = fmaf(b, b, ss);
    ss = fmaf(c, c, ss);
    ss = fmaf(d, d, ss);
  }
  ss = wave_sum_dpp(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float total = ((red[0] + red[1]) + red[2]) + red[3];
  const float r = 1.0f / sqrtf(total / (float)A.H + 1e-6f);
#pragma unroll
  for (int i = 0; i < QPT; ++i) {
    const int q = threadIdx.x + NT * i;
    if (q < nq) {
      const uint32_t a = f32_to_bf16_rne(bf16_bits_to_f32(v[i].x & 0xFFFFu) * r);
      const uint32_t b = f32_to_bf16_rne(bf16_bits_to_f32(v[i].x >> 16) * r);
      const uint32_t c = f32_to_bf16_rne(bf16_bits_to_f32(v[i].z & 0xFFFFu) * r);
      const uint32_t d = f32_to_bf16_rne(bf16_bits_to_f32(v[i].z >> 16) * r);
      *reinterpret_cast<uint2*>(xs + Lay::pos(4 * q)) = make_uint2(a | (b << 16), c | (d << 16));
    }
  }
  __syncthreads();
}

// The kernel's input residual stream -> LDS (layout Lay), 8 elements per chunk.
template <class Lay>
__device__ __forceinline__ void load_h_input(const uint16_t* h, int H, uint16_t* xs) {
  uint4 v[3];
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const int q = threadIdx.x + NT * i;
    v[i] = make_uint4(0, 0, 0, 0);
    if (q < H / 8) v[i] = ld16(h + (size_t)q * 8);
  }
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const int q = threadIdx.x + NT * i;
    if (q < H / 8) *reinterpret_cast<uint4*>(xs + Lay::pos(8 * q)) = v[i];
  }
  for (int q = threadIdx.x + 3 * NT; q < H / 8; q += NT)
    *reinterpret_cast<uint4*>(xs + Lay::pos(8 * q)) = ld16(h + (size_t)q * 8);
  __syncthreads();
}

template <class Lay>
__device__ __forceinline__ void rms_norm_inplace(uint16_t* xs, int H, float* red);

// u_l for layer l into LDS: from the kernel input for l = 0, else from the
// tagged stream; either way with a workgroup reduction for the scale.
template <int QPT, class Lay>
__device__ __forceinline__ void get_u(const FusedStepArgs& A, int l, unsigned base, uint16_t* xs, float* red) {
  if (l == 0) {
    load_h_input<Lay>(A.h_in, A.H, xs);
    rms_norm_inplace<Lay>(xs, A.H, red);
  } else {
    wait_u<QPT, Lay>(A, l, base + l - 1, xs, red);
  }
}

// u = RNE_bf16(h / sqrt(mean(h^2) + 1e-6)) in place.  The sum of squares has
// one fixed order in every workgroup that calls this, so all of them derive
// bit-identical u.
template <class Lay>
__device__ __forceinline__ void rms_norm_inplace(uint16_t* xs, int H, float* red) {
  float ss = 0.f;
  for (int i = threadIdx.x; i < H; i += NT) {
    const float v = bf16_bits_to_f32(xs[Lay::pos(i)]);
    ss = fmaf(v, v, ss);
  }
  ss = wave_sum_dpp(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float s = ((red[0] + red[1]) + red[2]) + red[3];
  const float r = 1.0f / sqrtf(s / (float)H + 1e-6f);
  for (int i = threadIdx.x; i < H; i += NT) xs[Lay::pos(i)] = f32_to_bf16_rne(bf16_bits_to_f32(xs[Lay::pos(i)]) * r);
  __syncthreads();
}

// Streamed weights are read once per step: nontemporal loads keep them from
// displacing the exchange buffers that the workgroups poll.
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16_stream(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// ---------------------------------------------------------------- routing


template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) { return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false); }

template <int CTRL>
__device__ __forceinline__ RankKey dpp_key(RankKey x) {
  const unsigned lo = (unsigned)dpp_i<CTRL>((int)(unsigned)x);
  const unsigned hi = (unsigned)dpp_i<CTRL>((int)(unsigned)(x >> 32));
  return ((RankKey)hi << 32) | lo;
}

// The routing of one layer as each wavefront of the workgroup sees it: the k
// selected experts in rank order and in slot order (ascending ids).
struct WaveRouting {
  int rid[WSX_MAX_K];     // selected ids in rank order
  float rw[WSX_MAX_K];    // routing weights in rank order
  int sid[WSX_MAX_K];     // selected ids, ascending (slot order)
  float sw[WSX_MAX_K];    // routing weight of each slot
};
struct alignas(16) Routing {
  RankKey grp[kRouteGroups];    // best key of each group of 8
  RankKey cand[kRouteGroups];   // all keys of the kRouteCand best groups
  RankKey top[WSX_MAX_K];       // the k selected keys in rank order
  WaveRouting w[NT / 64];       // one copy per wavefront, written and read by it alone
};

// Number of the 16 keys at t that rank before `me` (read in two halves: eight
// 16-byte reads at once make the compiler spill elsewhere in the kernel).
__device__ __forceinline__ int count_above16(const RankKey* t, RankKey me) {
  int n = 0;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    ulonglong2 p[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) p[j] = reinterpret_cast<const ulonglong2*>(t)[4 * h + j];
#pragma unroll
    for (int j = 0; j < 4; ++j) n += (int)(p[j].x > me) + (int)(p[j].y > me);
  }
  return n;
}

// Top-k routing of one layer by the whole workgroup, with no sequential
// selection rounds ([genai] and [sns], the router: softmax over the k largest
// of the E expert logits).  Logits rank by value, then by lower id, through
// their rank keys.  Thread t holds logits 2t and 2t+1 (E <= 2 NT; positions
// past E hold -inf), and each four consecutive threads form a group of 8.  A
// logit whose group's best logit is beaten by the best logits of k other
// groups is itself beaten by k logits, so the top k lie in the kRouteCand
// (>= k) groups whose best logits rank highest.  Both rankings, of the 64
// group maxima and then of the 64 logits of those groups, count pairwise wins
// (16 per thread, summed over the group's four threads), so every rank is
// found at once.  Leaves the k selected keys in rank order in R->top.
__device__ __forceinline__ void route_topk(const FusedStepArgs& A, unsigned tag, Routing* R) {
  const int t = threadIdx.x, q = t & 3, E = A.E, k = A.k;
  const int e0 = 2 * t;
  const uint2* lgc = lg_buf(A, my_copy(kCopiesLg));
  float v0 = -__builtin_inff(), v1 = -__builtin_inff();
  for (int it = 0;; ++it) {
    int ok = 1;
    if (e0 < E) {   // E is even: both logits of the pair exist
      const uint4 w = ld_coh16(lgc, (uint32_t)e0 * 8);
      v0 = __uint_as_float(w.x);
      v1 = __uint_as_float(w.z);
      ok = (w.y == tag) & (w.w == tag);
    }
    if (__all(ok)) break;
    if (wave_should_bail(A, it, tag)) break;
    __builtin_amdgcn_s_sleep(1);
  }
  const RankKey k0 = rank_key(v0, e0), k1 = rank_key(v1, e0 + 1);
  // best key of the group (every thread of the four ends with it)
  RankKey best = k0 > k1 ? k0 : k1;
  RankKey o = dpp_key<kQuadSwap1>(best);
  best = o > best ? o : best;
  o = dpp_key<kQuadSwap2>(best);
  best = o > best ? o : best;
  if (q == 0) R->grp[t >> 2] = best;
  __syncthreads();
  int rank = count_above16(R->grp + 16 * q, best);
  rank += dpp_i<kQuadSwap1>(rank);
  rank += dpp_i<kQuadSwap2>(rank);
  if (rank < kRouteCand) reinterpret_cast<ulonglong2*>(R->cand + rank * 8)[q] = make_ulonglong2(k0, k1);
  __syncthreads();
  const RankKey me = R->cand[t >> 2];
  rank = count_above16(R->cand + 16 * q, me);
  rank += dpp_i<kQuadSwap1>(rank);
  rank += dpp_i<kQuadSwap2>(rank);
  if (q == 0 && rank < k) R->top[rank] = me;
  __syncthreads();
}

// The routing weights, by every wavefront for itself: lane r < k takes the
// logit of rank r, the softmax sums in rank order (the same in every lane),
// and each selected expert's slot is its rank among the selected ids.  The
// result goes to the wavefront's own copy, R->w[wavefront].
__device__ __forceinline__ void route_weights(const FusedStepArgs& A, Routing* R) {
  const int lane = threadIdx.x & 63, k = A.k;
  const RankKey key = (lane < k) ? R->top[lane] : 0ull;
  const float v = key_value(key);
  const int id = key_id(key);
  const float top = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  float zs = 0.f, mine = 0.f;
  int slot = 0;
#pragma unroll
  for (int j = 0; j < WSX_MAX_K; ++j) {
    if (j < k) {
      const float z = __expf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), j)) - top);
      zs += z;
      if (j == lane) mine = z;
      slot += __builtin_amdgcn_readlane(id, j) < id;
    }
  }
  if (lane < k) {
    WaveRouting& W = R->w[threadIdx.x >> 6];
    const float w = mine / zs;
    W.rid[lane] = id;
    W.rw[lane] = w;
    W.sid[slot] = id;
    W.sw[slot] = w;
  }
  // the wavefront reads its copy back in other lanes: LDS accesses of one
  // wavefront complete in order, so only the compiler has to keep them so
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The expert of slot s (the s-th smallest selected id), by every wavefront
// for itself, without the weights.
__device__ __forceinline__ int route_slot_expert(const FusedStepArgs& A, const Routing* R, int s) {
  const int lane = threadIdx.x & 63, k = A.k;
  const int id = key_id((lane < k) ? R->top[lane] : 0ull);
  int slot = 0;
#pragma unroll
  for (int j = 0; j < WSX_MAX_K; ++j)
    if (j < k) slot += __builtin_amdgcn_readlane(id, j) < id;
  const unsigned long long hit = __ballot((lane < k) & (slot == s));
  return hit ? __builtin_amdgcn_readlane(id, __builtin_ctzll(hit)) : 0;
}

// ---------------------------------------------------------------- gate/up tile

// Rows of one expert's [2I][H] gate/up matrix for the intermediate values
// i0 .. i0+15: wavefront w, step st covers gate rows i0+4w+2st+{0,1} (lanes
// 0-15, 16-31) and the matching up rows (lanes 32-47, 48-63); 16 lanes per
// row, lane c takes MX blocks c, c+16, ...
template <int NJ>
struct GateUpRegs {
  uint4 cw[2][NJ];
  uint32_t sb[2][NJ];
};

template <int NJ>
__device__ __forceinline__ void gateup_load(const uint8_t* C, const uint8_t* S, int H, int I, int i0,
                                            GateUpRegs<NJ>& g) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane >> 4, c = lane & 15;
  const int NB = H / 32;
  const size_t rowc = H / 2, rows = H / 32;
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    const int ri = i0 + 4 * wave + 2 * st + (r & 1);
    const int row = (r < 2) ? ri : I + ri;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int b = c + 16 * j;
      g.cw[st][j] = (b < NB) ? ld16_stream(C + row * rowc + (size_t)b * 16) : make_uint4(0, 0, 0, 0);
      g.sb[st][j] = (b < NB) ? (uint32_t)S[row * rows + b] : 127u;
    }
  }
}

// a = silu(Wg u) * (Wu u) for the 16 values of the tile, stored as tagged
// pairs at a_slot[i].
template <int NJ>
__device__ __forceinline__ void gateup_compute(const GateUpRegs<NJ>& g, const uint32_t* xs32, int H, int i0,
                                               uint2* a_region, int slot_off, int copy_stride, unsigned tag) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane >> 4, c = lane & 15;
  const int NB = H / 32;
  // each activation block is read from LDS once and used for both row steps
  float accs[2] = {0.f, 0.f};
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int b = c + 16 * j;
    if (b < NB) {
      uint32_t xp[16];
      const uint4* src = reinterpret_cast<const uint4*>(xs32 + b * 20);   // LayMX: 80-byte blocks
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 t = src[q];
        xp[4 * q] = t.x; xp[4 * q + 1] = t.y; xp[4 * q + 2] = t.z; xp[4 * q + 3] = t.w;
      }
#pragma unroll
      for (int st = 0; st < 2; ++st) accs[st] = fmaf(mx_block_dot(g.cw[st][j], xp), e8m0_to_f32(g.sb[st][j]), accs[st]);
    }
  }
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    const float sum = sum16(accs[st]);
    const float up = __shfl_xor(sum, 32);
    const int ri = i0 + 4 * wave + 2 * st + (r & 1);
    // lanes c < kCopiesA of the two gate rows each publish copy c: one store
    // from the region's base, the copy and slot in the offset
    if (r < 2 && c < kCopiesA)
      st_coh8(a_region, (uint32_t)(c * copy_stride + slot_off + ri) * 8,
              make_uint2(__float_as_uint(silu(sum) * up), tag));
  }
}

// ---------------------------------------------------------------- down tile

// Rows n0 .. n0+7 of one expert's [H][I] down matrix: 8 lanes per row, lane c
// takes MX blocks c, c+8, ...
template <int NJD>
struct DownRegs {
  uint4 cw[NJD];
  uint32_t sb[NJD];
};

template <int NJD>
__device__ __forceinline__ void down_load(const uint8_t* C, const uint8_t* S, int I, int n0, DownRegs<NJD>& d) {
  const int lane = threadIdx.x & 63;
  const int row = n0 + (lane >> 3), c = lane & 7;
  const int NB = I / 32;
  const size_t rowc = I / 2, rows = I / 32;
#pragma unroll
  for (int j = 0; j < NJD; ++j) {
    const int b = c + 8 * j;
    d.cw[j] = (b < NB) ? ld16_stream(C + row * rowc + (size_t)b * 16) : make_uint4(0, 0, 0, 0);
    d.sb[j] = (b < NB) ? (uint32_t)S[row * rows + b] : 127u;
  }
}

// acc += wt * (W a) over this lane's MX blocks of its row (a: fp32 [I] in LDS).
template <int NJD>
__device__ __forceinline__ float down_dot(const DownRegs<NJD>& d, const float* a, int I, float wt, float acc) {
  const int c = threadIdx.x & 7;
  const int NB = I / 32;
#pragma unroll
  for (int j = 0; j < NJD; ++j) {
    const int b = c + 8 * j;
    if (b < NB) {
      const uint32_t w[4] = {d.cw[j].x, d.cw[j].y, d.cw[j].z, d.cw[j].w};
      const float4* ap = reinterpret_cast<const float4*>(a + b * 36);   // 144-byte blocks
      float s0 = 0.f, s1 = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 a0 = ap[2 * q];
        const float4 a1 = ap[2 * q + 1];
        const f32x2_t p0 = fp4x2_to_f32x2<0>(w[q]);
        const f32x2_t p1 = fp4x2_to_f32x2<1>(w[q]);
        const f32x2_t p2 = fp4x2_to_f32x2<2>(w[q]);
        const f32x2_t p3 = fp4x2_to_f32x2<3>(w[q]);
        s0 = fmaf(p0.x, a0.x, s0);
        s1 = fmaf(p0.y, a0.y, s1);
        s0 = fmaf(p1.x, a0.z, s0);
        s1 = fmaf(p1.y, a0.w, s1);
        s0 = fmaf(p2.x, a1.x, s0);
        s1 = fmaf(p2.y, a1.y, s1);
        s0 = fmaf(p3.x, a1.z, s0);
        s1 = fmaf(p3.y, a1.w, s1);
      }
      acc = fmaf(wt * e8m0_to_f32(d.sb[j]), s0 + s1, acc);
    }
  }
  return acc;
}

// One wavefront waits until slot s's I activations carry `tag` and copies
// them to LDS (as fp32).  QA 16-byte chunks (two pairs each) per lane cover
// the I/2 chunks.
template <int QA>
__device__ __forceinline__ void wave_wait_slot(const FusedStepArgs& A, int s, unsigned tag, float* as_slot) {
  const int lane = threadIdx.x & 63;
  const int I = A.I;
  const int nq = I / 2;
  const uint2* src = a_buf(A, my_copy(kCopiesA)) + (size_t)s * I;
  // poll from the start: each pass re-reads only the chunks still missing, and
  // a chunk goes to LDS as soon as it arrives
  unsigned pend = 0;   // chunks of this lane still without `tag`
#pragma unroll
  for (int i = 0; i < QA; ++i)
    if (lane + 64 * i < nq) pend |= 1u << i;
  for (int it = 0;; ++it) {
#pragma unroll
    for (int i = 0; i < QA; ++i) {
      if (pend & (1u << i)) {
        const int q = lane + 64 * i;
        const uint4 w = ld_coh16(src, (uint32_t)q * 16);
        if ((w.y == tag) & (w.w == tag)) {
          *reinterpret_cast<float2*>(as_slot + apos(0, 2 * q, I)) = make_float2(__uint_as_float(w.x), __uint_as_float(w.z));
          pend &= ~(1u << i);
        }
      }
    }
    if (__all(pend == 0)) break;
    if (wave_should_bail(A, it, tag)) break;
    __builtin_amdgcn_s_sleep(1);
  }
}

// One wavefront's routed slots (s = wave + 4 i < k): it polls all of their
// activations at once, copying each chunk to LDS (as fp32) as it arrives, and
// takes a slot's dot product (weight sw[s]) into accs[i] as soon as every
// chunk of that slot is in, so only the slot that arrives last is left for
// after the gate/up stage.  Each slot keeps its own sum, so the result does
// not depend on the order of arrival.
template <int QA, int MAXR, int NJD, int MAXS>
__device__ __forceinline__ void wave_routed_dots(const FusedStepArgs& A, unsigned tag, float* as,
                                                 const DownRegs<NJD> (&dr)[MAXS], const float* sw, float (&accs)[MAXR]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int I = A.I, k = A.k;
  const int nq = I / 2;
  const uint2* abuf = a_buf(A, my_copy(kCopiesA));
  unsigned pend = 0;   // chunks of this lane still without `tag`; each pass re-reads only those
  unsigned todo = 0;   // slots whose dot product is still to take (the same in every lane)
#pragma unroll
  for (int i = 0; i < MAXR; ++i) {
    accs[i] = 0.f;
    if (wave + 4 * i < k) {
      todo |= 1u << i;
#pragma unroll
      for (int j = 0; j < QA; ++j)
        if (lane + 64 * j < nq) pend |= 1u << (i * QA + j);
    }
  }
  for (int it = 0; todo; ++it) {
#pragma unroll
    for (int i = 0; i < MAXR; ++i) {
#pragma unroll
      for (int j = 0; j < QA; ++j) {
        if (pend & (1u << (i * QA + j))) {
          const int q = lane + 64 * j;
          const uint4 w = ld_coh16(abuf + (size_t)(wave + 4 * i) * I, (uint32_t)q * 16);
          if ((w.y == tag) & (w.w == tag)) {
            *reinterpret_cast<float2*>(as + apos(wave + 4 * i, 2 * q, I)) =
                make_float2(__uint_as_float(w.x), __uint_as_float(w.z));
            pend &= ~(1u << (i * QA + j));
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < MAXR; ++i) {
      const unsigned m = ((1u << QA) - 1u) << (i * QA);
      if ((todo & (1u << i)) && __all((pend & m) == 0)) {
        // the chunks came from every lane of this wavefront: its LDS accesses
        // complete in order, so the reads below see them
        const int s = wave + 4 * i;
        accs[i] = down_dot<NJD>(dr[i], as + apos(s, 0, I), I, sw[s], 0.f);
        todo &= ~(1u << i);
      }
    }
    if (!todo) break;
    if (wave_should_bail(A, it, tag)) break;
    __builtin_amdgcn_s_sleep(1);
  }
}

// ---------------------------------------------------------------- roles

// R: 8 router rows of layer l (RB-byte elements: 2 = bf16, 4 = fp32); 32 lanes
// per row, 16-byte granules c, c+32, ...
template <int RJ, int QPT, int RB>
__device__ __forceinline__ void role_router(const FusedStepArgs& A, int l, int r, unsigned base, uint16_t* xs,
                                            float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int H = A.H, E = A.E;
  const int row = r * kRRows + 2 * wave + (lane >> 5);
  const int c = lane & 31;
  const int G = H * RB / 16;   // granules per row
  uint4 wr[RJ];
  const uint8_t* W = reinterpret_cast<const uint8_t*>(A.router) + ((size_t)l * E + row) * (size_t)H * RB;
#pragma unroll
  for (int j = 0; j < RJ; ++j) {
    const int g = c + 32 * j;
    wr[j] = g < G ? ld16_stream(W + (size_t)g * 16) : make_uint4(0, 0, 0, 0);
  }
  issue_here();
  // the previous layer's gate/up stage completes before its down stage can:
  // sleep on it first
  if (l > 0 && threadIdx.x == 0)
    sleep_on_tag(A, a_buf(A, my_copy(kCopiesA)), (A.k - 1) * A.I + A.I - 1, base + l - 1);
  get_u<QPT, LayPlain>(A, l, base, xs, red);
  if (l == 0 && r == 0 && A.h_trace)
    for (int i = threadIdx.x; i < H; i += NT) A.h_trace[i] = A.h_in[i];
  if (r == 0 && A.u_trace)
    for (int i = threadIdx.x; i < H; i += NT) A.u_trace[(size_t)l * H + i] = xs[i];
  const uint32_t* xs32 = reinterpret_cast<const uint32_t*>(xs);
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < RJ; ++j) {
    const int g = c + 32 * j;
    if (g < G) {
      if constexpr (RB == 2) acc += bf16_granule_dot(wr[j], xs32 + g * 4);
      else acc += f32_granule_dot(wr[j], xs32 + g * 2);
    }
  }
  // rows of 32 lanes: the DPP tree within each 16-lane row, then the pair
  acc = sum16(acc);
  const float r0 = readlane_f(acc, 0) + readlane_f(acc, 16);
  const float r1 = readlane_f(acc, 32) + readlane_f(acc, 48);
  // lane c publishes copy c: one store from the region's base, the copy in the offset
  const int row0 = r * kRRows + 2 * wave;
  if (lane < kCopiesLg)
    st_coh16(A.b.lg, (uint32_t)(lane * A.E + row0) * 8,
             make_uint4(__float_as_uint(r0), base + l, __float_as_uint(r1), base + l));
}

// S: 16 intermediate values of the shared expert of layer l.
template <int NJ, int QPT>
__device__ __forceinline__ void role_shared_gateup(const FusedStepArgs& A, int l, int t, unsigned base, uint16_t* xs,
                                                   float* red) {
  const int H = A.H, I = A.I;
  GateUpRegs<NJ> g;
  gateup_load<NJ>(A.sh13c + (size_t)l * 2 * I * (H / 2), A.sh13s + (size_t)l * 2 * I * (H / 32), H, I, t * kGRows, g);
  issue_here();
  if (l > 0 && threadIdx.x == 0) sleep_on_tag(A, a_buf(A, my_copy(kCopiesA)), (A.k - 1) * I + I - 1, base + l - 1);
  get_u<QPT, LayMX>(A, l, base, xs, red);
  gateup_compute<NJ>(g, reinterpret_cast<const uint32_t*>(xs), H, t * kGRows, A.b.a, A.k * I, A.nslot * I,
                     base + l);
}

// G: 16 intermediate values of routed slot s of layer l.
template <int NJ, int QPT>
__device__ __forceinline__ void role_routed_gateup(const FusedStepArgs& A, int l, int s, int t, unsigned base,
                                                   uint16_t* xs, float* red, Routing* R) {
  const int H = A.H, I = A.I;
  // the layer input is needed by the router too, so it is complete before the
  // routing can be: sleep on it, normalize it, then wait for the routing
  if (l > 0 && threadIdx.x == 0) sleep_on_tag(A, hx_buf(A, l, my_copy(kCopiesH)), H / 2 - 1, base + l - 1);
  __syncthreads();
  get_u<QPT, LayMX>(A, l, base, xs, red);
  route_topk(A, base + l, R);
  // clamped: after a failed wait the routing is garbage, but reads stay in bounds
  const int e = min(max(route_slot_expert(A, R, s), 0), A.E - 1);
  GateUpRegs<NJ> g;
  const size_t c13 = (size_t)2 * I * (H / 2), s13 = (size_t)2 * I * (H / 32);
  gateup_load<NJ>(A.w13c + ((size_t)l * A.E + e) * c13, A.w13s + ((size_t)l * A.E + e) * s13, H, I, t * kGRows, g);
  gateup_compute<NJ>(g, reinterpret_cast<const uint32_t*>(xs), H, t * kGRows, A.b.a, s * I, A.nslot * I,
                     base + l);
}

// D: 8 output rows of layer l over every slot, the weighted combine, the
// residual add and the tagged store of h_{l+1}.  Wavefront w owns slots w,
// w+4, w+8 and handles the shared expert's slot (ready early) before its
// routed slots, always in that fixed order.
template <int NJD, int QA>
__device__ __forceinline__ void role_down(const FusedStepArgs& A, int l, int d, unsigned base, float* as,
                                          Routing* R, float* part) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int H = A.H, I = A.I, E = A.E, k = A.k, nslot = A.nslot;
  const int n0 = d * kDRows;
  const unsigned tag = base + l;
  const size_t c2 = (size_t)H * (I / 2), s2 = (size_t)H * (I / 32);
  // the shared expert's slot k belongs to wavefront k % 4: prefetch its rows
  const bool shared_here = nslot > k && wave == (k & 3);
  DownRegs<NJD> dsh;
  if (shared_here) down_load<NJD>(A.sh2c + (size_t)l * c2, A.sh2s + (size_t)l * s2, I, n0, dsh);
  issue_here();
  if (l > 0 && threadIdx.x == 0) sleep_on_tag(A, hx_buf(A, l, my_copy(kCopiesH)), H / 2 - 1, base + l - 1);
  __syncthreads();
  // residual rows of this tile (complete: the stream was waited for above)
  if (threadIdx.x < kDRows) {
    const int n = n0 + threadIdx.x;
    float res;
    if (l == 0) {
      res = bf16_bits_to_f32(A.h_in[n]);
    } else {
      uint2 p = make_uint2(0, 0);
      for (int it = 0; it < kSpinMax; ++it) {
        p = ld_coh8(hx_buf(A, l, my_copy(kCopiesH)), (uint32_t)(n >> 1) * 8);
        if (p.y == base + l - 1 || ((it & 15) == 15 && err_set(A, base))) break;
        __builtin_amdgcn_s_sleep(1);
      }
      if (p.y != base + l - 1) raise_err(A, base);
      res = bf16_bits_to_f32((n & 1) ? (p.x >> 16) : (p.x & 0xFFFFu));
    }
    part[4 * kDRows + threadIdx.x] = res;
  }
  // the shared expert first (owned by wavefront k % 4): its activations are
  // stored before the routing is known, so this wait overlaps the routing's
  float acc = 0.f;
  if (shared_here) {
    wave_wait_slot<QA>(A, k, tag, as + apos(k, 0, I));
    acc = down_dot<NJD>(dsh, as + apos(k, 0, I), I, 1.0f, acc);
  }
  route_topk(A, tag, R);
  route_weights(A, R);
  if (d == 0 && threadIdx.x < k) {
    if (A.ids_trace) A.ids_trace[(size_t)l * k + threadIdx.x] = R->w[0].rid[threadIdx.x];
    if (A.w_trace) A.w_trace[(size_t)l * k + threadIdx.x] = R->w[0].rw[threadIdx.x];
  }
  constexpr int MAXR = (WSX_MAX_K + 3) / 4;   // routed slots per wavefront: s = wave + 4 i
  DownRegs<NJD> dr[MAXR];
#pragma unroll
  for (int i = 0; i < MAXR; ++i) {
    const int s = wave + 4 * i;
    if (s < k) {
      const int e = min(max(R->w[wave].sid[s], 0), E - 1);
      down_load<NJD>(A.w2c + ((size_t)l * E + e) * c2, A.w2s + ((size_t)l * E + e) * s2, I, n0, dr[i]);
    }
  }
  issue_here();
  float accs[MAXR];
  wave_routed_dots<QA, MAXR>(A, tag, as, dr, R->w[wave].sw, accs);
  // the shared slot, then the routed slots in slot order: a fixed order
#pragma unroll
  for (int i = 0; i < MAXR; ++i)
    if (wave + 4 * i < k) acc += accs[i];
  acc = sum8(acc);
  if ((lane & 7) == 0) part[wave * kDRows + (lane >> 3)] = acc;
  __syncthreads();
  if (threadIdx.x < 64) {
    // wavefront 0, lane (copy c = lane / 8, row rr = lane % 8): every lane
    // forms its row of h_{l+1}; the even lanes publish the row pair of their copy
    const int rr = lane & 7, cpy = lane >> 3;
    const float y = ((part[rr] + part[kDRows + rr]) + part[2 * kDRows + rr]) + part[3 * kDRows + rr];
    const uint32_t hb = f32_to_bf16_rne(part[4 * kDRows + rr] + y);
    const uint32_t hn = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)hb, kQuadSwap1, 0xF, 0xF, false);
    const int n = n0 + rr;
    const uint2 pv = make_uint2(hb | (hn << 16), tag);
    // one store from the region's base, the copy in the offset
    if ((rr & 1) == 0)
      st_coh8(A.b.hx, (uint32_t)((cpy * 2 + ((l + 1) & 1)) * (H / 2) + (n >> 1)) * 8, pv);
    if (cpy == 0 && A.h_trace) A.h_trace[(size_t)(l + 1) * H + n] = (uint16_t)hb;
    if (cpy == 0 && l == A.L - 1) A.h_out[n] = (uint16_t)hb;
  }
}

// Head rows: wavefront row groups of 4 rows, 16 lanes per row, HJ granules of
// 16 codes per lane; the next group's loads are in flight while the current
// one is reduced.
template <int HJ>
__device__ __forceinline__ void head_load(const FusedStepArgs& A, int grp, uint4 (&w)[HJ], float& sc) {
  const int lane = threadIdx.x & 63;
  const int row = grp * 4 + (lane >> 4), c = lane & 15;
  const int G = A.H / 16;
  const bool ok = row < A.V;
#pragma unroll
  for (int j = 0; j < HJ; ++j) {
    const int g = c + 16 * j;
    w[j] = (ok && g < G) ? ld16_stream(A.hq + (size_t)row * A.H + (size_t)g * 16) : make_uint4(0, 0, 0, 0);
  }
  sc = (ok && c == 0) ? A.hs[row] : 0.f;
}

template <int HJ, int QPT>
__device__ __forceinline__ void role_head(const FusedStepArgs& A, int hb, unsigned base, uint16_t* xs, float* red,
                                          float* wv_, int* wi_, int* flag) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int H = A.H, V = A.V, L = A.L;
  const int NG = (V + 3) / 4;
  const int stride = A.n_head * 4;
  int grp = hb * 4 + wave;
  uint4 w[HJ];
  float sc = 0.f;
  if (grp < NG) head_load<HJ>(A, grp, w, sc);
  issue_here();
  if (threadIdx.x == 0) sleep_on_tag(A, a_buf(A, my_copy(kCopiesA)), (A.k - 1) * A.I + A.I - 1, base + L - 1);
  wait_u<QPT, LayHead>(A, L, base + L - 1, xs, red);
  if (hb == 0 && A.u_trace)
    for (int i = threadIdx.x; i < H; i += NT) A.u_trace[(size_t)L * H + i] = xs[LayHead::pos(i)];
  const uint32_t* xs32 = reinterpret_cast<const uint32_t*>(xs);
  const int G = H / 16, c = lane & 15;
  float bv = -__builtin_inff();
  int bi = 0x7FFFFFFF;
  while (grp < NG) {
    uint4 wn[HJ];
    float scn = 0.f;
    const int nxt = grp + stride;
    if (nxt < NG) head_load<HJ>(A, nxt, wn, scn);
    issue_here();
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < HJ; ++j) {
      const int g = c + 16 * j;
      if (g < G) acc += fp8_granule_dot(w[j], xs32 + g * 12);   // LayHead: 48-byte granules
    }
    acc = sum16(acc);
    const int row = grp * 4 + (lane >> 4);
    if (c == 0 && row < V) {
      const float lv = acc * sc;
      if (A.logits) A.logits[row] = lv;
      if (better(lv, row, bv, bi)) { bv = lv; bi = row; }
    }
#pragma unroll
    for (int j = 0; j < HJ; ++j) w[j] = wn[j];
    sc = scn;
    grp = nxt;
  }
  // workgroup argmax
  wave_argmax(bv, bi);
  if (lane == 0) { wv_[wave] = bv; wi_[wave] = bi; }
  __syncthreads();
  // the workgroup's best (value, row) joins the step's maximum rank key: one
  // 64-bit atomic max orders by value, then lower row, as `better` does
  if (threadIdx.x == 0) {
    float v = wv_[0];
    int i = wi_[0];
    for (int q = 1; q < 4; ++q)
      if (better(wv_[q], wi_[q], v, i)) { v = wv_[q]; i = wi_[q]; }
    const RankKey key = (v == v) ? rank_key(v, i) : 0ull;   // a NaN never wins
    __hip_atomic_fetch_max(&ctl(A)->best, key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // the last workgroup to arrive reads the maximum, publishes the argmax
  // (-1 if a wait of this step gave up), clears the maximum and the error
  // word, and advances the epoch for the next step.  Every other workgroup of
  // the step has passed all of its waits by now (each one's last store feeds
  // the head), so none can raise the error after this point.
  if (!last_block_arrived(&ctl(A)->top_counter, A.n_head, flag)) return;
  if (threadIdx.x == 0) {
    const RankKey best = __hip_atomic_load(&ctl(A)->best, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&ctl(A)->best, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool failed = err_set(A, base);
    A.argmax[0] = (failed || best == 0ull) ? -1 : key_id(best);
    st_dev(reinterpret_cast<int*>(&ctl(A)->err), 0);
    const unsigned ep = (unsigned)ld_dev(reinterpret_cast<const int*>(&ctl(A)->epoch));
    st_dev(reinterpret_cast<int*>(&ctl(A)->epoch), (int)((ep + 1) % kEpochMod));
  }
}

}  // namespace

template <int NJ, int NJD, int RJ, int HJ, int QPT, int QA, int RB>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(4))) decode_step_kernel(FusedStepArgs A) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ float red[4];
  __shared__ Routing R;
  __shared__ float part[5 * kDRows];
  __shared__ float wv_[4];
  __shared__ int wi_[4];
  __shared__ int flag;
  // tags: (epoch + 1) in the upper 24 bits, the layer below
  const unsigned base = ((unsigned)ld_dev(reinterpret_cast<const int*>(&ctl(A)->epoch)) + 1u) << 8;
  const int bid = A.block0 + (int)blockIdx.x;
  if (bid >= A.L * A.per_layer) {
    role_head<HJ, QPT>(A, bid - A.L * A.per_layer, base, reinterpret_cast<uint16_t*>(smem), red, wv_, wi_, &flag);
    return;
  }
  const int l = bid / A.per_layer;
  int j = bid - l * A.per_layer;
  if (j < A.nR) { role_router<RJ, QPT, RB>(A, l, j, base, reinterpret_cast<uint16_t*>(smem), red); return; }
  j -= A.nR;
  if (j < A.nS) { role_shared_gateup<NJ, QPT>(A, l, j, base, reinterpret_cast<uint16_t*>(smem), red); return; }
  j -= A.nS;
  if (j < A.nG) {
    const int tiles = A.I / kGRows;
    role_routed_gateup<NJ, QPT>(A, l, j / tiles, j % tiles, base, reinterpret_cast<uint16_t*>(smem), red,
                                         &R);
    return;
  }
  j -= A.nG;
  role_down<NJD, QA>(A, l, j, base, reinterpret_cast<float*>(smem), &R, part);
}

}  // namespace wsx
