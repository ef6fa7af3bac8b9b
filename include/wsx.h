/*
 * wsx.h — C ABI of libwsx.so, the MI355X (gfx950) batch-1 MoE + FP8 LM-head
 * decode path.
 *
 * Sources (web pages on NVIDIA's Ling-3.0-flash decode work on one DGX Spark):
 *   [saipien] saipien.org/?p=9636
 *   [ncij]    ncijnetwork.com, "NVIDIA shows 3 ways to speed up MoE inference
 *             on DGX Spark, lifting Ling-3.0-flash throughput 42.5%"
 *   [genai]   generativeaipub.com, "NVIDIA engineers boost MoE inference"
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every pointer argument is DEVICE memory owned by the caller.  The library
 *    never allocates, frees, copies to the host or synchronizes; all work is
 *    enqueued on `stream` (a hipStream_t; NULL means the null stream).
 *  - bf16 values travel as raw uint16_t bit patterns (the top half of an IEEE
 *    binary32).  E4M3 codes are OCP E4M3FN bytes.  MXFP4 matrices are stored
 *    row-major along the contraction dimension K: `codes` [N][K/2] with
 *    element 2j in the low nibble of byte j and element 2j+1 in the high
 *    nibble, and `scales` [N][K/32] of E8M0 bytes, byte b scaling elements
 *    32b..32b+31 of its row.  Both arrays start 16-byte aligned (the kernels
 *    read the scale bytes 16 at a time).
 *  - Every argument check runs on the host before anything is enqueued.  On
 *    an error nothing is enqueued and outputs are untouched.  A failed launch
 *    returns WSX_ERR_HIP.  The library never aborts or prints.
 *  - Workspaces: `ws` is caller-allocated device memory of at least the size
 *    returned by the matching *_workspace_bytes query, 256-byte aligned, and
 *    ZERO-FILLED BEFORE ITS FIRST USE.  Counters and error words inside it
 *    return to zero at the end of every call, so it is reusable without
 *    clearing (moe_decode_step also keeps a step counter there that advances
 *    by one per call).  A workspace may be reused with any T; a decode-step
 *    workspace serves one stack shape (H, I, E, k, V) and must be zero-filled
 *    again before it is used with another.  Calls that may run concurrently
 *    (different streams) need distinct workspaces.
 *  - Inputs must be finite and must not contain the E8M0 byte 0xFF (NaN);
 *    otherwise results are unspecified but the call still completes.
 *  - Reductions use a fixed order, so repeated calls give bit-identical
 *    results.
 */
#ifndef WSX_H
#define WSX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum wsx_status {
  WSX_OK = 0,
  WSX_ERR_NULL = 1,        /* a required pointer is NULL */
  WSX_ERR_SHAPE = 2,       /* a size is out of range or not a multiple of 32 */
  WSX_ERR_ALIGN = 3,       /* a pointer is not 16-byte aligned (workspace: 256) */
  WSX_ERR_UNSUPPORTED = 4, /* valid but not built: T > 4, k > 8, E > 1024, ... */
  WSX_ERR_WORKSPACE = 5,   /* workspace missing or smaller than required */
  WSX_ERR_DTYPE = 6,       /* unknown dtype code */
  WSX_ERR_HIP = 7          /* the HIP runtime rejected a launch */
} wsx_status;

enum { WSX_DTYPE_BF16 = 0, WSX_DTYPE_F32 = 1 };

#define WSX_MAX_T 4    /* tokens per pass of the head, the sampler and the decode step: 1 = decode, 4 = MTP verify */
#define WSX_MAX_T_MOE 16 /* tokens per pass of one MoE layer (router and experts): a small batch or a longer draft */
#define WSX_MAX_K 8    /* routed experts chosen per token */
#define WSX_MAX_E 1024 /* routed experts per layer */

/*
 * moe_route_topk — router GEMV, top-k selection, routing weights and the
 * compact expert list of one MoE layer.
 *
 * [saipien] "Why one user waits on weights": each token is sent to 8 of 512
 * routed experts (plus one shared expert that always runs); [saipien] "Draft
 * three tokens, verify four": a 4-position verify pass wakes up to 32 routed
 * experts.
 *
 *   logits[t][e] = sum_h Wr[e][h] * x[t][h]            (fp32 accumulate)
 *   topk_ids[t]  = the k experts with the largest logits, in rank order
 *                  (logit descending, ties to the LOWER expert id)
 *   topk_w[t][j] = softmax over the k selected logits
 *   expert_list  = [n_active, ids...]: the distinct ids of all T tokens,
 *                  ascending; n_active <= T*k
 *   slot_w[s][t] = routing weight of token t for expert_list[1+s], or 0
 *
 * x         bf16 [T][H]
 * w_router  [E][H], bf16 (router_dtype = WSX_DTYPE_BF16) or fp32 (WSX_DTYPE_F32)
 * topk_ids  int32 [T][k]; topk_w float [T][k]
 * expert_list int32 [1 + T*k]; slot_w float [T*k][T] (rows past n_active are 0)
 * logits_out float [T][E] or NULL
 * Limits: 1 <= T <= WSX_MAX_T_MOE (16: a small batch or a longer draft),
 * 1 <= k <= 8, k <= E <= 1024, H % 32 == 0.
 * Workspace: wsx_moe_workspace_bytes(T, H, I, E, k) (any I).
 */
wsx_status moe_route_topk(const uint16_t* x, const void* w_router, int router_dtype,
                          int T, int H, int E, int k,
                          int32_t* topk_ids, float* topk_w, int32_t* expert_list, float* slot_w,
                          float* logits_out, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_expert_gemv_mxfp4 — the routed + shared SwiGLU experts of one MoE layer
 * with MXFP4 weights, driven by the device-side expert list (no host round
 * trip), and the weighted combine with the bf16 residual.
 *
 * [saipien] "Kernels built for the shape you actually have" (narrow expert
 * intermediate size 768, MXFP4 expert kernels); [genai] "1. A Better Kernel
 * for Ling's Experts".
 *
 * For each active slot s with expert e = expert_list[1+s] and each token t:
 *   g = Wg[e] x[t], u = Wu[e] x[t]   (Wg = rows 0..I-1, Wu = rows I..2I-1 of W13[e])
 *   a = silu(g) * u                  (fp32, not rounded)
 *   y[t] = sum_s slot_w[s][t] * (W2[e] a) + (W2sh (silu(Wg_sh x) * Wu_sh x))
 *   out_h[t] = RNE_bf16(residual[t] + y[t])  (fp32 add, then round)
 *
 * x        bf16 [T][H]
 * w13_codes [E][2I][H/2], w13_scales [E][2I][H/32]
 * w2_codes  [E][H][I/2],  w2_scales  [E][H][I/32]
 * sh13_*, sh2_*: the shared expert with the same layouts (without [E]); all
 *          four NULL for no shared expert.
 * expert_list, slot_w: as written by moe_route_topk (or built by the caller).
 * residual bf16 [T][H] or NULL; out_y float [T][H] or NULL; out_h bf16 [T][H]
 *          or NULL (requires residual).
 * Each active expert serves the tokens with a nonzero weight in its slot row
 * (the expert-sorted token lists); the shared expert serves every token.
 * Limits: 1 <= T <= WSX_MAX_T_MOE (16), 1 <= k <= 8, H % 32 == 0, I % 32 == 0,
 *          I <= 2048, H <= 8192.  Ids in expert_list must lie in [0, E).
 * Workspace: wsx_moe_workspace_bytes(T, H, I, E, k).
 */
wsx_status moe_expert_gemv_mxfp4(const uint16_t* x,
                                 const uint8_t* w13_codes, const uint8_t* w13_scales,
                                 const uint8_t* w2_codes, const uint8_t* w2_scales,
                                 const uint8_t* sh13_codes, const uint8_t* sh13_scales,
                                 const uint8_t* sh2_codes, const uint8_t* sh2_scales,
                                 const int32_t* expert_list, const float* slot_w,
                                 int T, int H, int I, int E, int k,
                                 const uint16_t* residual, float* out_y, uint16_t* out_h,
                                 void* ws, size_t ws_bytes, void* stream);

/*
 * act_quantize_mxfp8 — the W4A8 path's activation quantizer: bf16 rows to
 * MXFP8 with E4M3 elements.
 *
 * [saipien] "Why one user waits on weights": the baseline recipe was "W4A8",
 * which the page reads as 4-bit weights and 8-bit activations.  Per block of
 * 32 consecutive elements of a row:
 *   X = floor(log2(max |x|)) - 8, clamped to [-127, 127] (-127 for a zero block)
 *   codes = E4M3FN_RNE(clamp(x / 2^X, -448, 448)),  scale byte = X + 127
 *
 * x bf16 [T][K]; codes uint8 [T][K]; scales uint8 [T][K/32].
 * Limits: T >= 1, K % 32 == 0.  No workspace.
 */
wsx_status act_quantize_mxfp8(const uint16_t* x, int T, int K, uint8_t* codes, uint8_t* scales, void* stream);

/*
 * moe_expert_gemv_w4a8 — moe_expert_gemv_mxfp4 with 8-bit activations: the
 * same MXFP4 weights contracted on the matrix cores with MXFP8 activations
 * ([saipien] "Why one user waits on weights", the W4A8 baseline recipe).
 *
 * For each active slot s (expert e) and token t:
 *   xq = MXFP8(x[t])                       (as act_quantize_mxfp8)
 *   g = Wg[e] xq, u = Wu[e] xq,  a = silu(g) * u   (fp32)
 *   aq = MXFP8(a)                          (per 32 values of I, from binary32)
 *   y[t] = sum_s slot_w[s][t] * (W2[e] aq) + (the shared expert, weight 1)
 *   out_h[t] = RNE_bf16(residual[t] + y[t])
 *
 * Arguments, layouts and limits as moe_expert_gemv_mxfp4, plus act_out:
 * float [T*k+1][T][I] or NULL, the binary32 a of every slot (slots in list
 * order, then the shared expert) before its quantization.  Shapes: H and I
 * multiples of 32, at most 2560 each; T * (H + H/32) <= 65536.
 * Workspace: wsx_moe_workspace_bytes(T, H, I, E, k).
 */
wsx_status moe_expert_gemv_w4a8(const uint16_t* x,
                                const uint8_t* w13_codes, const uint8_t* w13_scales,
                                const uint8_t* w2_codes, const uint8_t* w2_scales,
                                const uint8_t* sh13_codes, const uint8_t* sh13_scales,
                                const uint8_t* sh2_codes, const uint8_t* sh2_scales,
                                const int32_t* expert_list, const float* slot_w,
                                int T, int H, int I, int E, int k,
                                const uint16_t* residual, float* out_y, uint16_t* out_h, float* act_out,
                                void* ws, size_t ws_bytes, void* stream);

/*
 * lm_head_quantize_fp8 — load-time BF16 -> FP8 E4M3FN quantization of the
 * vocabulary projection, one fp32 scale per row.
 *
 * [saipien] "Stop hauling the vocabulary in full precision" and [genai]
 * "2. Compressing the Output Head": only the LM head is quantized to FP8,
 * once, when the layer is built, halving its bytes.
 *
 *   s[v] = absmax_k |w[v][k]| / 448        (IEEE binary32 division)
 *   q[v][k] = E4M3FN_RNE(clamp(w[v][k] / s[v], -448, 448))  (binary32 division)
 *   an all-zero row gets s = 0 and all codes 0x00.
 *
 * w bf16 [V][K]; q uint8 [V][K]; row_scale float [V].
 * Limits: V >= 1, K % 32 == 0, K <= 16384.  No workspace.
 */
wsx_status lm_head_quantize_fp8(const uint16_t* w, int V, int K, uint8_t* q, float* row_scale,
                                void* stream);

/*
 * lm_head_gemv_fp8_argmax — per-token FP8 LM-head GEMV with the row scale in
 * the epilogue and a fused greedy argmax.
 *
 * [saipien] "Stop hauling the vocabulary in full precision" (the head is read
 * for every token); [ncij] "What happens on a real workload?" (greedy decoding).
 *
 *   logits[t][v] = s[v] * sum_k E4M3(q[v][k]) * x[t][k]   (fp32 accumulate)
 *   argmax[t] = the v with the largest logit, ties to the LOWER index
 *
 * q uint8 [V][K] and row_scale float [V] as written by lm_head_quantize_fp8;
 * x bf16 [T][K]; logits float [T][V] or NULL; argmax int32 [T].
 * Limits: 1 <= T <= 4, K % 32 == 0, K <= 8192, V >= 1.
 * Workspace: wsx_lm_head_workspace_bytes(T, V, K).
 */
wsx_status lm_head_gemv_fp8_argmax(const uint8_t* q, const float* row_scale, int V, int K,
                                   const uint16_t* x, int T, float* logits, int32_t* argmax,
                                   void* ws, size_t ws_bytes, void* stream);

/*
 * lm_head_gemv_bf16_argmax — the unquantized BF16 head, the 2x-bytes
 * comparison for the FP8 head.  Same contract as lm_head_gemv_fp8_argmax
 * without row scales: logits[t][v] = sum_k w[v][k] * x[t][k].
 *
 * [saipien] "Why one user waits on weights" and "Stop hauling the vocabulary
 * in full precision": before the FP8 head, the 157,184 x 2,560 projection was
 * read in full precision for every token.
 */
wsx_status lm_head_gemv_bf16_argmax(const uint16_t* w, int V, int K, const uint16_t* x, int T,
                                    float* logits, int32_t* argmax, void* ws, size_t ws_bytes,
                                    void* stream);

/*
 * lm_sample_topk_topp — one sampled token per row of the head's logits, with
 * temperature, top-k and top-p, the uniform draw supplied by the caller.
 *
 * [ncij] "What happens on a real workload?": the GSM8K run samples with
 * temperature 0.6, top_p 0.95 and top_k 29.  The pages give only the three
 * settings; the steps are (binary32, in this order):
 *   z_0 >= ... >= z_{k-1}: the top_k logits, ties to the LOWER id;
 *   e_i = exp((z_i - z_0) / temperature);  c_i = e_0 + ... + e_i;
 *   m = the first i with c_i >= top_p * c_{k-1}   (ranks 0..m are kept);
 *   token = id of the first rank j <= m with c_j > u * c_m (rank m if none).
 *
 * logits float [T][V]; uniforms float [T], each in [0, 1); token int32 [T];
 * topk_ids int32 [T][top_k] (ranked ids) and topk_probs float [T][top_k]
 * (e_i / c_m for i <= m, else 0) may be NULL.
 * Limits: 1 <= T <= 4, 1 <= top_k <= min(64, V), V <= 524,224,
 * temperature > 0 and finite, 0 < top_p <= 1 (else WSX_ERR_SHAPE or
 * WSX_ERR_UNSUPPORTED).  Workspace: wsx_sample_workspace_bytes(T, V, top_k)
 * (no zero fill needed).
 */
size_t wsx_sample_workspace_bytes(int T, int V, int top_k);
wsx_status lm_sample_topk_topp(const float* logits, int V, int T, float temperature, int top_k,
                               float top_p, const float* uniforms, int32_t* token,
                               int32_t* topk_ids, float* topk_probs, void* ws, size_t ws_bytes,
                               void* stream);

/*
 * lm_head_gemv_fp8_sample — the FP8 head of lm_head_gemv_fp8_argmax with the
 * sampler of lm_sample_topk_topp on its logits: the sampling decode of [ncij]
 * "What happens on a real workload?" in place of greedy.  Results are those of
 * lm_sample_topk_topp on the logits written here, bit for bit.  For T = 1 on
 * the head shapes the wide kernel serves (wsx_lm_head_sample_path returns 1)
 * it is one launch: each wavefront of the head publishes the maximum of the
 * rows it streamed and the last workgroup to finish selects the top_k and
 * draws; otherwise the head and the two sampler launches run in turn on the
 * stream.  logits float [T][V] is required (an output in both forms).
 * Limits: those of both calls.  A NaN logit is never drawn in the one-launch
 * form; with fewer than top_k logits that are numbers the token is unspecified
 * (-1 when none is).  Workspace: wsx_lm_head_sample_workspace_bytes(T, V, K,
 * top_k), zero-filled before its first use; its counter returns to zero, so
 * it is reusable without clearing; calls that share it must not overlap.
 */
size_t wsx_lm_head_sample_workspace_bytes(int T, int V, int K, int top_k);
/* 1: lm_head_gemv_fp8_sample runs as one launch on the current device for
 * these sizes; 0: as three launches; -1: the sizes are not supported. */
int wsx_lm_head_sample_path(int T, int V, int K, int top_k);
wsx_status lm_head_gemv_fp8_sample(const uint8_t* q, const float* row_scale, int V, int K,
                                   const uint16_t* x, int T, float temperature, int top_k,
                                   float top_p, const float* uniforms, float* logits,
                                   int32_t* token, int32_t* topk_ids, float* topk_probs,
                                   void* ws, size_t ws_bytes, void* stream);

/*
 * Weights of L stacked MoE layers of one shape, each tensor one contiguous
 * allocation with a leading [L] axis:
 *   w_router  [L][E][H] (bf16 or fp32, router_dtype)
 *   w13_codes [L][E][2I][H/2]   w13_scales [L][E][2I][H/32]
 *   w2_codes  [L][E][H][I/2]    w2_scales  [L][E][H][I/32]
 *   sh13_codes [L][2I][H/2] ... sh2_scales [L][H][I/32], or all four NULL.
 */
typedef struct wsx_moe_stack {
  const void* w_router;
  int router_dtype;
  const uint8_t* w13_codes;
  const uint8_t* w13_scales;
  const uint8_t* w2_codes;
  const uint8_t* w2_scales;
  const uint8_t* sh13_codes;
  const uint8_t* sh13_scales;
  const uint8_t* sh2_codes;
  const uint8_t* sh2_scales;
  int L, H, I, E, k;
} wsx_moe_stack;

/*
 * moe_decode_step — one decode (T = 1) or MTP-verify (T <= 4) pass through L
 * stacked MoE layers and the FP8 LM head, with no host synchronization.
 *
 * [saipien] "Why one user waits on weights": a batch-1 decode step streams,
 * for every layer, the router, 8 of 512 routed experts and the shared expert,
 * then the whole vocabulary projection; [saipien] "Stop hauling the
 * vocabulary in full precision" for the FP8 head; [saipien] "Draft three
 * tokens, verify four" for the 4-position verify pass.
 *
 * For l = 0..L-1:  u_l = RNE_bf16(h_l / sqrt(mean(h_l^2) + 1e-6))   (per token)
 *                  h_{l+1} = moe layer l on input u_l with residual h_l
 * then logits = FP8 head applied to u_L, argmax as lm_head_gemv_fp8_argmax.
 * The unit-gain RMS norm between layers is a reading taken for the stacked
 * synthetic layers (the pages give no norm); the MoE layer is
 * moe_route_topk followed by moe_expert_gemv_mxfp4.
 *
 * h_in bf16 [T][H]; h_out bf16 [T][H] (the final residual stream);
 * logits float [T][V] or NULL; argmax int32 [T].
 * Failure report: at T = 1 with a compiled shape (see wsx_build_info) the
 * whole step is one launch whose workgroups wait on each other with bounded
 * waits.  If a wait gives up (it never should), the step still completes,
 * argmax[0] is -1 and h_out / logits are unspecified; the error does not
 * carry over, so the next call on the same workspace runs normally.  The
 * return status only reports host-side checks and launch errors.
 * Optional traces (each NULL or the full size): h_trace bf16 [L+1][T][H]
 * (h_0..h_L), u_trace bf16 [L+1][T][H] (u_0..u_L, u_L being the head input),
 * ids_trace int32 [L][T][k], w_trace float [L][T][k].
 * Workspace: wsx_decode_step_workspace_bytes(...).
 */
wsx_status moe_decode_step(const uint16_t* h_in, int T, const wsx_moe_stack* stack,
                           const uint8_t* head_q, const float* head_scale, int V,
                           uint16_t* h_out, float* logits, int32_t* argmax,
                           uint16_t* h_trace, uint16_t* u_trace, int32_t* ids_trace, float* w_trace,
                           void* ws, size_t ws_bytes, void* stream);

/*
 * wsx_decode_step_path — how moe_decode_step runs a stack of this shape:
 *   0  per-phase launches (T > 1, no shared expert, or a shape outside the
 *      one-launch kernel's layout: E > 512, H > 4096, I > 2048, ...);
 *   1  one launch, compiled ahead of time (H 2560 / I 768 / bf16 router, and
 *      H 256 / I 64 / fp32 router);
 *   2  one launch, compiled at run time with hipRTC on the first call for the
 *      shape on each device (about a second), then reused.
 * [saipien] "Kernels built for the shape you actually have": the pages' MoE
 * kernels are specialized to the model's shapes at run time.  A failed
 * run-time compilation makes moe_decode_step return WSX_ERR_HIP.
 */
int wsx_decode_step_path(int T, int router_dtype, int has_shared, int H, int I, int E, int k);

/*
 * wsx_read_probe — measurement utility, not a step of the decode path: one
 * plain streaming read of `bytes` bytes at `buf` (16-byte loads, all issued
 * before use), the reference rate for "how fast can weights come out of
 * memory" ([ncij] "Why is MoE decoding on DGX Spark memory-bound?").
 * `out` (one uint32) receives an XOR of what was read, so the reads cannot be
 * optimized away; its value has no meaning.
 * Limits: bytes > 0 and a multiple of 16, buf 16-byte aligned.
 */
wsx_status wsx_read_probe(const void* buf, size_t bytes, uint32_t* out, void* stream);

/*
 * moe_decode_step_noalloc — moe_decode_step without a workspace argument, for
 * callers that cannot allocate device memory (code under graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  It allocates nothing: its
 * workspace is a static device array of WSX_NOALLOC_SCRATCH_BYTES held by each
 * GPU the library runs on until the process ends.
 *
 * Same arguments, results and failure report as moe_decode_step.  Shapes
 * whose decode-step workspace (wsx_decode_step_workspace_bytes) exceeds
 * WSX_NOALLOC_SCRATCH_BYTES return WSX_ERR_WORKSPACE before anything is
 * enqueued.  On the first call on a device, and whenever the stack shape
 * (H, I, E, k, V) differs from the previous call's on that device, the array
 * is cleared by a kernel enqueued on `stream` ahead of the step.  Every call
 * on one GPU shares that GPU's array: calls that overlap on one GPU (different
 * streams, or host threads) race and give unspecified results.
 */
#define WSX_NOALLOC_SCRATCH_BYTES ((size_t)2 << 20)
wsx_status moe_decode_step_noalloc(const uint16_t* h_in, int T, const wsx_moe_stack* stack,
                                   const uint8_t* head_q, const float* head_scale, int V,
                                   uint16_t* h_out, float* logits, int32_t* argmax,
                                   uint16_t* h_trace, uint16_t* u_trace, int32_t* ids_trace,
                                   float* w_trace, void* stream);

size_t wsx_moe_workspace_bytes(int T, int H, int I, int E, int k);
size_t wsx_lm_head_workspace_bytes(int T, int V, int K);
size_t wsx_decode_step_workspace_bytes(int T, int H, int I, int E, int k, int V);

const char* wsx_status_string(wsx_status s);
/* Build description: target architecture and the kernel variants compiled in. */
const char* wsx_build_info(void);

#ifdef __cplusplus
}
#endif

#endif /* WSX_H */
