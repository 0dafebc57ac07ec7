/*
 * moe_fp4.h -- C ABI of the MI355X (gfx950) FP4 routed-expert MoE layer.
 *
 * The layer: top-k routing over router logits, a stable expert sort/permute
 * of the (token, slot) pairs, MXFP8 quantisation of the activations, the
 * gate/up (W1/W3) and down (W2) grouped GEMMs over packed 4-bit e2m1 weights
 * with one E8M0 scale per 32 elements along K, SwiGLU between them, and a
 * gate-weighted combine back to token order.  The pages name this "FP4 routed
 * mixture-of-experts computation" and trace the wrong outputs of the first
 * fast path to a routed-expert W2 layout mismatch repaired once at load time
 * ("DeepSeek-V4-Flash on AMD gfx90a: Correctness Recovery and Inference
 * Performance Engineering", abstract).
 *
 * Around the layer: the router logits from the hidden states and shared
 * experts (moe_router_logits, moe_fp4_layer_forward_full, the shared-expert
 * stage calls), and the FP8 dense projections the same pages list beside the
 * FP4 experts (moe_fp8_dense_*).
 *
 * Conventions shared by every call:
 *  - Pointers are DEVICE pointers unless a comment says (host).  The caller
 *    allocates and frees everything, including workspaces sized by the
 *    *_workspace_size() queries and the packed-weight buffer.  The library
 *    never allocates, frees or synchronises, and never copies device data to
 *    the host, so a chain of calls can be captured in a HIP graph: launches
 *    take device pointers and sizes only and read no host scalars mid-way
 *    (the capture rule of the aijianwen.com MI300X log, HIP graph section).
 *  - Every call only enqueues work on `stream`, in order.  MOE_OK means
 *    "enqueued"; results are ready when the stream reaches that point.
 *  - All argument checks run on the host before anything is enqueued.  On an
 *    error nothing is enqueued and outputs are untouched.  Device data is not
 *    validated: logits must be finite and expert ids must come from
 *    moe_route_topk.
 *  - Tensors are row-major and contiguous.  Byte tensors and x must be
 *    16-byte aligned; the packed-weight buffer 256-byte aligned.
 *  - Formats: e2m1 nibbles two per byte along K, the EVEN K index in the LOW
 *    nibble; E8M0 scale code c means 2^(c-127); activations use OCP e4m3fn
 *    (bias 7, max 448, 0x7F/0xFF NaN) -- the dialect MI355X uses (aijianwen.com
 *    MI300X log, FP8 section); x is bf16, logits/gates/y are fp32.
 *  - Determinism: the same inputs give bitwise-identical outputs, run to run.
 *    No floating-point atomics anywhere; reductions go in a fixed order
 *    (pwwt.cn review, section 4.2).
 *  - Size queries take (T, E, k, H, I, ...) in that order, like
 *    moe_sort_permute_workspace_size; the compute calls take their own
 *    argument lists as declared.
 *  - Supported shapes: 1 <= k <= min(E, 32), E <= 1024, H % 128 == 0,
 *    I % 128 == 0, 0 <= T, T*k < 2^31.  T == 0 is a no-op.  Anything else
 *    returns MOE_ERR_UNSUPPORTED (or MOE_ERR_INVALID_ARGUMENT for negative
 *    sizes and null pointers).
 *  - Re-entrant; outputs must not alias inputs.
 */
#ifndef MOE_FP4_H
#define MOE_FP4_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARGUMENT = 1, /* null pointer, negative or inconsistent size, misalignment */
  MOE_ERR_UNSUPPORTED = 2,      /* well-formed but outside the supported shapes above */
  MOE_ERR_WORKSPACE = 3,        /* workspace smaller than the matching *_workspace_size() */
  MOE_ERR_HIP = 4               /* a HIP launch failed; see moe_last_hip_error() */
} moe_status_t;

/* Static string naming a status code (never NULL). */
const char* moe_status_string(moe_status_t status);

/* The hipError_t of the calling thread's most recent HIP operation through
 * this library (a kernel launch, or the scratch lookup of the no-allocation
 * entry point): 0 when it succeeded or when the thread has made none (a call
 * rejected by the argument checks makes none and leaves the value as it was).
 * Read it after a call returned MOE_ERR_HIP. */
int moe_last_hip_error(void);

/* Layout version of moe_fp4_prepack_weights' output. */
#define MOE_FP4_LAYOUT_VERSION 1u

/*
 * Top-k routing (step 1 of the layer).
 * For each token t the k experts with the largest logits, ties to the LOWER
 * expert index (a fixed tie-break by expert id: pwwt.cn review, section 4.1
 * table row "MoE routing top-k", and section 4.2), compared as fp32 values
 * (-0 equals +0).  Slot j = 0 holds the largest.  Gates are a softmax over the
 * k selected logits: g_j = exp(l_j - l_0) / sum_i exp(l_i - l_0), in fp32.
 *   logits     [T, E] fp32, finite
 *   topk_ids   [T, k] int32 (out)
 *   topk_gates [T, k] fp32  (out)
 */
moe_status_t moe_route_topk(const float* logits, int32_t T, int32_t E, int32_t k,
                            int32_t* topk_ids, float* topk_gates, hipStream_t stream);

/*
 * Expert sort / permute (step 2; "retuned expert sorting" in the abstract).
 * Pairs p = t*k + j.  expert_counts[e] = #pairs routed to e; expert_offsets
 * is the exclusive prefix sum with expert_offsets[E] = T*k; sorted_pair lists
 * the pairs grouped by expert in ascending e, and ascending p inside each
 * group (stable: pwwt.cn review, section 4.2 forbids unstable sorting);
 * pair_pos is its inverse (pair_pos[sorted_pair[s]] = s).
 *   topk_ids       [T, k] int32, each in [0, E)
 *   expert_counts  [E] int32 (out);  expert_offsets [E+1] int32 (out)
 *   sorted_pair    [T*k] int32 (out); pair_pos      [T*k] int32 (out)
 *   workspace      >= moe_sort_permute_workspace_size(T, E, k) bytes, 256-aligned
 */
size_t moe_sort_permute_workspace_size(int32_t T, int32_t E, int32_t k);
moe_status_t moe_sort_permute(const int32_t* topk_ids, int32_t T, int32_t E, int32_t k,
                              int32_t* expert_counts, int32_t* expert_offsets,
                              int32_t* sorted_pair, int32_t* pair_pos,
                              void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * MXFP8 activation quantisation (step 3; the pages' gfx90a path used INT8
 * activation quantisation, the abstract).  For each row and each block of 32
 * consecutive elements: X = floor(log2(max|v|)) - 8 (8 = largest e4m3
 * exponent), X = -127 for an all-zero block, X clamped to [-127, 127]; scale
 * code X + 127; element code = v * 2^-X rounded to e4m3fn, nearest, ties to
 * even, saturating to +-448, sign kept (so -tiny -> 0x80).
 *   x_bf16 [M, K] bf16 bit patterns; K % 32 == 0
 *   q      [M, K] e4m3fn bytes (out);  s [M, K/32] E8M0 codes (out)
 */
moe_status_t moe_quant_act_mxfp8(const uint16_t* x_bf16, int32_t M, int32_t K,
                                 uint8_t* q, uint8_t* s, hipStream_t stream);

/*
 * Load-time weight prepack, which also fixes the W2 layout once (the abstract:
 * the output permutation was identified and the weight layout repaired at
 * load time).  Canonical inputs (device):
 *   w1, w3 [E, I, H/2] packed e2m1;  s1, s3 [E, I, H/32] E8M0
 *   w2     [E, H, I/2] packed e2m1;  s2     [E, H, I/32] E8M0
 * Output: `packed` (device, >= moe_fp4_packed_weight_bytes(E, H, I) bytes,
 * 256-byte aligned) in the kernels' tile order, and `desc` (host) which the
 * forward calls take.  The caller keeps `packed` alive and unmodified while
 * `desc` is in use; the canonical inputs may be freed once the stream has
 * passed this call.
 */
typedef struct moe_fp4_weights {
  int32_t E, H, I;
  uint32_t layout_version;
  const void* packed;   /* device */
  size_t packed_bytes;
} moe_fp4_weights_t;

size_t moe_fp4_packed_weight_bytes(int32_t E, int32_t H, int32_t I);
moe_status_t moe_fp4_prepack_weights(const uint8_t* w1, const uint8_t* s1,
                                     const uint8_t* w3, const uint8_t* s3,
                                     const uint8_t* w2, const uint8_t* s2,
                                     int32_t E, int32_t H, int32_t I,
                                     void* packed, size_t packed_bytes,
                                     moe_fp4_weights_t* desc, hipStream_t stream);

/* Path selection for the expert GEMMs.  By default the host picks from the
 * host-known T*k and E only (never from device counts): the weight-streaming
 * decode path when T*k <= 16*E (about 16 rows per expert, where the two paths
 * measured equal on MI355X at the larger decode-sized expert shape), the MFMA-tiled
 * prefill path otherwise.  The flags force one path (both compute the same
 * function). */
#define MOE_FLAG_FORCE_DECODE 1u
#define MOE_FLAG_FORCE_PREFILL 2u

/*
 * Expert gate/up GEMM + SwiGLU + MXFP8 of h (steps 4-5), in sorted order.
 * For each expert e and each sorted position s in [off[e], off[e+1]) with
 * token t = sorted_pair[s] / k:
 *   G[s,i] = sum_h x[t,h] W1[e,i,h],  U[s,i] = sum_h x[t,h] W3[e,i,h]
 * (MXFP8 x times FP4 W, fp32 accumulation), h = G / (1 + e^-G) * U in fp32,
 * then hq/hs = MXFP8 of h per 32 along I (the rule of moe_quant_act_mxfp8).
 *   xq [T, H], xs [T, H/32] from moe_quant_act_mxfp8
 *   expert_offsets [E+1], sorted_pair [T*k] from moe_sort_permute
 *   hq [T*k, I] (out), hs [T*k, I/32] (out), rows in sorted order
 *   An expert-parallel shard may pass expert_offsets[E] < T*k (the pairs of
 *   its own E experts, offsets re-based to 0): rows from expert_offsets[E]
 *   on are neither computed nor written, but sorted_pair keeps T*k entries,
 *   each a valid pair index.  The same holds for moe_fp4_expert_down.
 *   The prefill path needs T*H < 2^32 (MOE_ERR_UNSUPPORTED otherwise).
 *   workspace >= moe_fp4_stage_workspace_size(T, E, k, H, I), 256-aligned
 *   (the prefill path's tile list and its activation scales rearranged by
 *   K-step; contents on entry are ignored)
 */
size_t moe_fp4_stage_workspace_size(int32_t T, int32_t E, int32_t k, int32_t H, int32_t I);
moe_status_t moe_fp4_expert_up(const moe_fp4_weights_t* w /*(host)*/,
                               const uint8_t* xq, const uint8_t* xs,
                               const int32_t* expert_offsets, const int32_t* sorted_pair,
                               int32_t T, int32_t k, uint8_t* hq, uint8_t* hs,
                               void* workspace, size_t workspace_bytes,
                               uint32_t flags, hipStream_t stream);

/*
 * Expert down GEMM (step 6): O[s,r] = sum_i h[s,i] W2[e,r,i], rows in sorted
 * order, accumulated in fp32 and stored as bf16 (round to nearest even): a
 * matrix-multiply output kept at low precision, its sum over experts taken
 * in fp32 by moe_combine (pwwt.cn review, section 4.1, the precision table).
 *   hq [T*k, I], hs [T*k, I/32] from moe_fp4_expert_up
 *   O  [T*k, H] bf16 bits (out, 16-byte aligned)
 */
moe_status_t moe_fp4_expert_down(const moe_fp4_weights_t* w /*(host)*/,
                                 const uint8_t* hq, const uint8_t* hs,
                                 const int32_t* expert_offsets, int32_t T, int32_t k,
                                 uint16_t* O, void* workspace, size_t workspace_bytes,
                                 uint32_t flags, hipStream_t stream);

/*
 * Gate-weighted combine (step 7): y[t,r] = sum_{j=0..k-1, in this order}
 * gates[t,j] * O[pair_pos[t*k+j], r], fp32 fused multiply-adds, no atomics.
 *   O [T*k, H] bf16 bits (8-byte aligned); topk_gates [T, k]; pair_pos [T*k];
 *   y [T, H] fp32 (out, 16-byte aligned)
 *   H % 4 == 0
 */
moe_status_t moe_combine(const uint16_t* O, const float* topk_gates, const int32_t* pair_pos,
                         int32_t T, int32_t k, int32_t H, float* y, hipStream_t stream);

/*
 * Steps 4-7 in one call: expert_up -> expert_down -> combine, with hq, hs, O
 * and the tile map held in `workspace`
 * (>= moe_fp4_forward_workspace_size(T, E, k, H, I, flags) bytes, 256-aligned).
 *   y [T, H] fp32 (out, overwritten)
 */
size_t moe_fp4_forward_workspace_size(int32_t T, int32_t E, int32_t k, int32_t H, int32_t I,
                                      uint32_t flags);
moe_status_t moe_fp4_grouped_forward(const moe_fp4_weights_t* w /*(host)*/,
                                     const uint8_t* xq, const uint8_t* xs, const float* topk_gates,
                                     const int32_t* expert_offsets, const int32_t* sorted_pair,
                                     const int32_t* pair_pos, int32_t T, int32_t k,
                                     float* y, void* workspace, size_t workspace_bytes,
                                     uint32_t flags, hipStream_t stream);

/*
 * The whole layer, steps 1-7, in one call: route -> sort/permute -> MXFP8(x)
 * -> expert_up -> expert_down -> combine.  Results are bitwise identical to
 * the chain of the single-stage calls above on the same inputs.  For
 * T <= 16 the three front steps run as one fused launch (routing and sort in
 * one workgroup, quantisation in the others); larger T uses the stand-alone
 * kernels.  Every intermediate lives in `workspace`
 * (>= moe_fp4_layer_workspace_size(T, E, k, H, I, flags) bytes, 256-aligned;
 * contents on entry are ignored, on exit unspecified).
 *   x_bf16 [T, H] bf16 bits (16-byte aligned); logits [T, E] fp32
 *   y [T, H] fp32 (out, overwritten, 16-byte aligned)
 *   flags: MOE_FLAG_FORCE_DECODE / MOE_FLAG_FORCE_PREFILL as above
 */
size_t moe_fp4_layer_workspace_size(int32_t T, int32_t E, int32_t k, int32_t H, int32_t I,
                                    uint32_t flags);
moe_status_t moe_fp4_layer_forward(const moe_fp4_weights_t* w /*(host)*/,
                                   const uint16_t* x_bf16, const float* logits,
                                   int32_t T, int32_t k, float* y,
                                   void* workspace, size_t workspace_bytes,
                                   uint32_t flags, hipStream_t stream);

/*
 * The whole layer as moe_fp4_layer_forward, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  The intermediates live in a fixed scratch array of
 * MOE_NOALLOC_SCRATCH_BYTES in device memory that the library holds on each
 * GPU it runs on until the process ends (its address is looked up on the
 * first call on a device).  The call allocates, frees and clears nothing; the
 * caller passes inputs and outputs only.  Results are bitwise those of
 * moe_fp4_layer_forward on the same inputs.
 *  - Shapes whose moe_fp4_layer_workspace_size(T, E, k, H, I, flags) exceeds
 *    MOE_NOALLOC_SCRATCH_BYTES return MOE_ERR_WORKSPACE, nothing enqueued
 *    (64 MiB holds T <= 476 at H7168 I2048 E256 top-8, T <= 1052 at H4096
 *    I1536 E64 top-6).
 *  - Every call on a GPU uses that GPU's one scratch array and leaves its
 *    contents behind (none is read before the call writes it): calls that
 *    overlap on one GPU -- other streams, other host threads -- race, and the
 *    caller must order them.
 *  - x_bf16 [T, H] bf16 bits (16-byte aligned); logits [T, E] fp32;
 *    y [T, H] fp32 (out, overwritten, 16-byte aligned); flags as above.
 */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
moe_status_t moe_fp4_layer_forward_noalloc(const moe_fp4_weights_t* w /*(host)*/,
                                           const uint16_t* x_bf16, const float* logits,
                                           int32_t T, int32_t k, float* y, uint32_t flags,
                                           hipStream_t stream);

/*
 * Router logits, the gate network's first layer ahead of step 1:
 * logits[t,e] = sum_h x[t,h] * Wg[e,h], x and Wg bf16, products accumulated
 * in fp32 by the bf16 matrix cores (the pwwt.cn review, section 4.1, lets the
 * gate network's first layers run at low precision while the top-k compare
 * stays fp32).  The summation order is fixed per shape, so results are
 * reproducible; they differ from an exact sum by at most the fp32 bound
 * gamma_H * sum_h |x[t,h] * Wg[e,h]| (gamma_n = n*u/(1-n*u), u the fp32
 * unit roundoff).  The sum over H is split into a shape-dependent number of
 * K slices whose fp32 partial sums are added in slice order in `workspace`.
 *   x_bf16 [T, H] bf16 bits, router_w [E, H] bf16 bits (both 16-byte aligned)
 *   logits [T, E] fp32 (out, overwritten)
 *   workspace >= moe_router_workspace_size(T, H, E) bytes, 256-aligned (may
 *   be NULL when that size is 0)
 *   H % 128 == 0, 1 <= E <= 1024
 */
size_t moe_router_workspace_size(int32_t T, int32_t H, int32_t E);
moe_status_t moe_router_logits(const uint16_t* x_bf16, const uint16_t* router_w, int32_t T,
                               int32_t H, int32_t E, float* logits, void* workspace,
                               size_t workspace_bytes, hipStream_t stream);

/*
 * Shared expert: one always-active expert of the same FP4 format (E == 1 in
 * `w`, its own intermediate size w->I) applied to every token's MXFP8 row:
 * O_shared[t] = W2 * MXFP8(silu(W1 x_t) * (W3 x_t)), bf16 (RNE) as O of the
 * routed experts.  The DeepSeekMoE layer (pwwt.cn review, section 1.2) pairs
 * the routed experts with such an expert; this stage call takes one of any
 * intermediate size and runs the same gate/up and down kernels as the routed
 * path with the trivial routing pair = token (shared experts of the routed
 * intermediate size run inside the routed GEMMs: moe_fp4_layer_forward_full).
 *   xq [T, H] e4m3, xs [T, H/32] E8M0 (as from moe_quant_mxfp8)
 *   O_shared [T, H] bf16 bits (out, 16-byte aligned)
 *   workspace >= moe_fp4_shared_workspace_size(T, H, w->I, flags), 256-aligned
 *   flags: MOE_FLAG_FORCE_DECODE / MOE_FLAG_FORCE_PREFILL as above
 */
size_t moe_fp4_shared_workspace_size(int32_t T, int32_t H, int32_t I_shared, uint32_t flags);
moe_status_t moe_fp4_shared_expert(const moe_fp4_weights_t* w /*(host), E == 1*/,
                                   const uint8_t* xq, const uint8_t* xs, int32_t T,
                                   uint16_t* O_shared, void* workspace, size_t workspace_bytes,
                                   uint32_t flags, hipStream_t stream);

/*
 * Combine with a shared expert: moe_combine's sum over the k slots in order,
 * then + O_shared[t, r] (weight 1), all in fp32.  O_shared [T, H] bf16 bits,
 * 8-byte aligned; the other arguments as for moe_combine.
 */
moe_status_t moe_combine_shared(const uint16_t* O, const float* topk_gates, const int32_t* pair_pos,
                                const uint16_t* O_shared, int32_t T, int32_t k, int32_t H, float* y,
                                hipStream_t stream);

/*
 * The layer from hidden states, with shared experts: router logits ->
 * top-k routing over the routed experts -> every token also sent to each
 * shared expert with weight 1 -> sort/permute -> MXFP8(x) -> expert GEMMs ->
 * combine.  The DeepSeekMoE layer (pwwt.cn review, section 1.2) pairs routed
 * experts with always-active shared ones; here they are the LAST n_shared
 * experts of `w` (same format and intermediate size as the routed ones: a
 * shared FFN of intermediate n*I is n such experts), so they run inside the
 * routed grouped GEMMs as one more group of T rows each.  Token t's slots are
 * its k routed experts in rank order, then the shared experts in index order
 * with gate 1.0, so y_t = sum_j g_j O_j + sum_s O_shared_s, added in that
 * order in fp32.  The router's K-slice partial sums are read by the routing
 * launch directly (summed in the same order as moe_router_logits), so the
 * logits equal moe_router_logits' bit for bit.
 *   w: E = E_routed + n_shared experts (0 <= n_shared < E); router_w
 *   [E_routed, H] bf16 bits; x_bf16 [T, H] bf16 bits; y [T, H] fp32 (out)
 *   1 <= k <= E_routed, k + n_shared <= 32
 *   workspace >= moe_fp4_layer_full_workspace_size(T, E, k, H, I, n_shared,
 *   flags) bytes, 256-aligned
 *   flags: MOE_FLAG_FORCE_DECODE / MOE_FLAG_FORCE_PREFILL as above
 */
size_t moe_fp4_layer_full_workspace_size(int32_t T, int32_t E, int32_t k, int32_t H, int32_t I,
                                         int32_t n_shared, uint32_t flags);
moe_status_t moe_fp4_layer_forward_full(const moe_fp4_weights_t* w /*(host)*/, int32_t n_shared,
                                        const uint16_t* router_w, const uint16_t* x_bf16,
                                        int32_t T, int32_t k, float* y, void* workspace,
                                        size_t workspace_bytes, uint32_t flags,
                                        hipStream_t stream);

/*
 * FP8 dense projection (a non-expert linear layer): y[t, n] = sum_k x[t, k] *
 * W[n, k].  W is OCP e4m3 with one E8M0 scale per 32 consecutive K elements
 * of a row (block-wise FP8: the pages list "FP8 dense projections" beside the
 * FP4 experts, arxivdaily abstract, and name block-wise quantisation as the
 * way FP8 pays off, pwwt.cn review, section 5.3); x is given as MXFP8 rows
 * (moe_quant_act_mxfp8); the products accumulate in fp32 in the scaled MFMA
 * and y is stored as bf16, RNE (pwwt.cn review, section 4.1: low-precision
 * matrix-multiply outputs, fp32 accumulation).
 *
 * moe_fp8_dense_prepack: wq [N, K] e4m3 codes (16-byte aligned), ws [N, K/32]
 * E8M0 -> `packed` (device, >= moe_fp8_dense_packed_bytes(N, K) bytes,
 * 256-byte aligned) in the kernels' tile order, and `desc` (host), as for the
 * expert weights.  N % 32 == 0, K % 128 == 0, packed size < 4 GiB.
 *
 * moe_fp8_dense_forward: xq [T, K] (16-byte aligned), xs [T, K/32] (4-byte
 * aligned), y [T, N] bf16 bits (out).  T * K < 2^32.  Path: weight streaming
 * for T <= 96 (MOE_FLAG_FORCE_DECODE for any T; the two paths measured equal
 * near T = 110 at K 16384, N 7168), an LDS-tiled GEMM otherwise
 * (MOE_FLAG_FORCE_PREFILL for any T); both compute the same function.  No
 * workspace; the same inputs give the same bits.
 */
#define MOE_FP8_DENSE_LAYOUT_VERSION 1u

typedef struct moe_fp8_dense_weights {
  int32_t N, K;
  uint32_t layout_version;
  const void* packed;   /* device */
  size_t packed_bytes;
} moe_fp8_dense_weights_t;

size_t moe_fp8_dense_packed_bytes(int32_t N, int32_t K);
moe_status_t moe_fp8_dense_prepack(const uint8_t* wq, const uint8_t* ws, int32_t N, int32_t K,
                                   void* packed, size_t packed_bytes,
                                   moe_fp8_dense_weights_t* desc /*(host)*/, hipStream_t stream);
moe_status_t moe_fp8_dense_forward(const moe_fp8_dense_weights_t* w /*(host)*/,
                                   const uint8_t* xq, const uint8_t* xs, int32_t T, uint16_t* y,
                                   uint32_t flags, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_FP4_H */
