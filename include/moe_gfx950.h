/*
 * moe_gfx950.h -- C ABI of the fused Mixture-of-Experts layer for AMD MI355X
 * (gfx950).
 *
 * The layer is the fused MoE operation: token routing, data shuffling into
 * expert order, the expert network and the weighted aggregation of expert
 * outputs, run as one batched GPU operation (readmex.ai, "AWS details fused
 * MoE kernel optimizations on SageMaker, up to 10% throughput gain", summary;
 * agentic-affairs.com, "Swap-AB targets matrix execution on Hopper").  The
 * FP8 mode folds the tensor scales into the matrix pass and aggregates the
 * expert outputs in the same pipeline (codebridge-ai.com,
 * "aws-moe-kernel-wgmma-triton-ttft", section "2. Backend routing";
 * agentic-affairs.com, "Triton improves the FP8 execution path").
 *
 * Conventions for every entry point:
 *  - Pointers are DEVICE pointers unless stated otherwise; `moe_shape` is a
 *    host struct.  The caller owns every buffer.  The library never allocates
 *    or frees memory and keeps no state between calls.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Calls only enqueue work; nothing synchronises the host.  Outputs are
 *    ready when the stream reaches them.
 *  - Arguments are checked on the host before anything is enqueued; a
 *    failed check returns a negative moe_status and leaves every buffer
 *    untouched.  A launch failure returns MOE_ERR_HIP.  T = 0 (with otherwise
 *    valid sizes) returns MOE_OK at once: no buffer is checked or touched.
 *  - Limits: 1 <= E <= 1024, 1 <= k <= min(E, 16), 0 <= T, T*k < 2^31,
 *    H and I positive multiples of 128 (MOE_ERR_UNSUPPORTED otherwise),
 *    every device pointer 16-byte aligned.
 *  - Preconditions the device does not check (violations are undefined,
 *    except that a NaN logit is read as -inf, which keeps every expert id in
 *    range): logits hold no NaN and at least k non-(-inf) entries per row;
 *    topk_ids lie in [0, E); sorted_ids / expert_offsets / inv_perm are the
 *    outputs of moe_align_sort for the same ids.
 *  - Results are deterministic: routing outputs are bit-identical run to run
 *    and floating-point outputs do not depend on scheduling (no floating
 *    atomics; maxima use integer atomics, which are order-free).
 *
 * Data types by mode (moe_shape.wdtype):
 *   MOE_F32      : x, h, out fp32; w13, w2 fp32; no scales.
 *   MOE_BF16     : x, h, out bf16; w13, w2 bf16; no scales.
 *   MOE_FP8_E4M3 : x, h, out bf16; w13, w2 OCP e4m3fn codes with one fp32
 *                  dequantisation scale per expert and matrix; x and h are
 *                  quantised to e4m3 inside the layer with dynamic
 *                  per-tensor scales (amax / 448).
 * Layouts (row-major, last index contiguous):
 *   x [T,H]; logits [T,E] fp32; w13 [E,2I,H] (rows 0..I-1 gate, I..2I-1 up);
 *   w2 [E,H,I]; h [T*k,I] and y [T*k,H] in expert-sorted pair order;
 *   out [T,H]; topk_ids / topk_weights [T,k]; a pair (t,j) has flat index
 *   f = t*k + j.
 */
#ifndef MOE_GFX950_H
#define MOE_GFX950_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_FP8_E4M3 = 2 } moe_dtype;

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* null / misaligned pointer, bad T, E, k, dtype */
  MOE_ERR_UNSUPPORTED = -2, /* H or I not a multiple of 128 */
  MOE_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required */
  MOE_ERR_HIP = -4,         /* a kernel launch failed */
  MOE_ERR_TOO_LARGE = -5    /* beyond moe_fused_forward_noalloc's scratch */
} moe_status;

/* Layer shape (host struct).  renormalize: 1 = top-k softmax renormalised
 * over the selected experts, 0 = plain softmax probabilities. */
typedef struct {
  int32_t T, H, E, k, I;
  int32_t wdtype;
  int32_t renormalize;
} moe_shape;

/* Host only.  Checks a shape against the limits above; returns a moe_status. */
int moe_check_shape(const moe_shape* s);

/* Host only.  Bytes of device workspace that every entry point of this
 * shape may use (the fused entry point needs the most).  Returns 0 for an
 * invalid shape.  The workspace must be 256-byte aligned. */
size_t moe_workspace_bytes(const moe_shape* s);

/* Host only.  Static description of a status code. */
const char* moe_status_string(int status);

/* Host only.  Where the fused entry points leave the routing of a call
 * inside the caller's workspace: byte offsets from the start of `ws` (of
 * this shape) of
 *   topk_ids [T,k] int32, topk_weights [T,k] fp32 (written there only when
 *     the caller passes NULL for those outputs),
 *   expert_counts [E], expert_offsets [E+1], sorted_ids [T*k], inv_perm
 *     [T*k] (int32, always written),
 * each with the meaning of moe_align_sort's outputs.  They hold the call's
 * values once the stream has passed it and until the next call that uses
 * the same workspace.  Returns a moe_status (out == NULL: invalid). */
typedef struct {
  size_t topk_ids, topk_weights, expert_counts, expert_offsets, sorted_ids, inv_perm;
} moe_routing_offsets;
int moe_workspace_routing(const moe_shape* s, moe_routing_offsets* out);

/* Top-k softmax gating: the token routing that opens the fused operation
 * (readmex.ai, "AWS details fused MoE kernel optimizations on SageMaker, up
 * to 10% throughput gain", summary; agentic-affairs.com, "Swap-AB targets
 * matrix execution on Hopper": routing, data shuffling and the expert
 * calculations in one batched GPU operation).  The pages name the stage but
 * not its rule; the rule below is the softmax top-k this library implements.
 *   logits       [T,E] fp32 in, row-major
 *   topk_ids     [T,k] int32 out: slot j holds the expert with the (j+1)-th
 *                largest logit; equal logits go to the lower expert index;
 *                -0 equals +0
 *   topk_weights [T,k] fp32 out: exp(l - l_max) over the selected experts
 *                divided by their sum (renormalize = 1) or by the sum over
 *                all E experts (renormalize = 0)
 * Null or misaligned pointers, or T, E, k outside the limits, give
 * MOE_ERR_INVALID_ARG with nothing enqueued.  A NaN logit (a precondition
 * violation) is read as -inf, so the ids stay inside [0, E). */
int moe_topk_gating(const float* logits, int32_t T, int32_t E, int32_t k, int32_t renormalize,
                    int32_t* topk_ids, float* topk_weights, void* stream);

/* Host only.  Bytes of device workspace moe_align_sort needs for T tokens,
 * top-k and E experts (0 when T, E, k are outside the limits).  The
 * workspace must be 256-byte aligned. */
size_t moe_align_sort_workspace_bytes(int32_t T, int32_t k, int32_t E);

/* Grouping of the (token, slot) pairs by expert: the "data shuffling" stage
 * of the fused operation (readmex.ai, "AWS details fused MoE kernel
 * optimizations on SageMaker, up to 10% throughput gain", summary), whose
 * per-expert batch sizes are data dependent (explore.n1n.ai,
 * "Mixture-of-Experts Kernel Engineering on Amazon SageMaker AI", section
 * "The Core Bottlenecks of MoE Inference on H200 GPUs").
 *   topk_ids       [T,k] int32 in, every id in [0, E)
 *   expert_counts  [E] int32 out: pairs routed to expert e
 *   expert_offsets [E+1] int32 out: exclusive prefix sum of the counts,
 *                  expert_offsets[E] = T*k
 *   sorted_ids     [T*k] int32 out: flat pair indices f = t*k + j by expert
 *                  ascending and, inside an expert, by f ascending
 *   inv_perm       [T*k] int32 out (may be NULL): inv_perm[sorted_ids[p]] = p
 *   ws, ws_bytes   device workspace of moe_align_sort_workspace_bytes
 *                  bytes, 256-byte aligned, caller-owned
 * The kernels are chosen by the pair count exactly as the fused entry point
 * chooses them (one block up to 256 pairs, one block per expert below 8192,
 * a chunked counting sort from 8192 on), so both run the same grouping.
 * Errors: as moe_topk_gating; a missing, misaligned or small workspace gives
 * MOE_ERR_WORKSPACE. */
int moe_align_sort(const int32_t* topk_ids, int32_t T, int32_t k, int32_t E,
                   int32_t* expert_counts, int32_t* expert_offsets, int32_t* sorted_ids,
                   int32_t* inv_perm, void* ws, size_t ws_bytes, void* stream);

/* Expert gate/up projection with SwiGLU, grouped over experts: the first
 * half of the expert network calculation of the fused operation (readmex.ai,
 * "AWS details fused MoE kernel optimizations on SageMaker, up to 10%
 * throughput gain", summary), with the large expert dimension on the matrix
 * unit's row side for few-token batches (codebridge-ai.com,
 * "aws-moe-kernel-wgmma-triton-ttft", section "1. Matrix swap") and the FP8
 * tensor scales folded into the same pass (agentic-affairs.com, "Triton
 * improves the FP8 execution path").
 * For sorted position p (pair f = sorted_ids[p], token t = f / k, expert e
 * with offsets[e] <= p < offsets[e+1]):
 *   g_n = x[t] . w13[e][n],  u_n = x[t] . w13[e][I+n]    (fp32 accumulation)
 *   FP8: x is first quantised per tensor (codes e4m3(x * 448/amax(x))), the
 *        products use the codes and both sums are scaled by
 *        fl32(s_x * w13_scale[e]), s_x = amax(x)/448.
 *   h[p][n] = silu(g_n) * u_n, stored in the activation type.
 * act_scales [4] fp32 out (FP8 mode; left untouched otherwise):
 *   {s_x, s_h, amax(x), amax(h)} with s_h = amax(h)/448 (amax = 0 -> scale 1).
 * w13_scale [E] is required in FP8 mode and ignored otherwise. */
int moe_grouped_gemm_w13_swiglu(const moe_shape* s, const void* x, const void* w13,
                                const float* w13_scale, const int32_t* sorted_ids,
                                const int32_t* expert_offsets, void* h, float* act_scales,
                                void* ws, size_t ws_bytes, void* stream);

/* Expert down projection, grouped over experts, unweighted: the second half
 * of the expert network calculation (readmex.ai, "AWS details fused MoE
 * kernel optimizations on SageMaker, up to 10% throughput gain", summary),
 * with the FP8 scales applied to the fp32 accumulators in the same pass
 * (codebridge-ai.com, "aws-moe-kernel-wgmma-triton-ttft", section "2.
 * Backend routing": scaling and matmul not as discrete steps).
 * h is in sorted order, so the position p alone names its expert (through
 * expert_offsets); no sorted_ids argument is needed.
 * h [T*k,I] activation type in, sorted order; w2 [E,H,I]; w2_scale [E] fp32
 * (FP8 only); act_scales [4] fp32 in as written by
 * moe_grouped_gemm_w13_swiglu (FP8 only; only act_scales[3] is read);
 * ws / ws_bytes as for moe_workspace_bytes(s).
 *   y[p][m] = h[p] . w2[e][m] (fp32 accumulation), e the expert of position p.
 *   FP8: h is quantised per tensor with the scale derived from
 *        act_scales[3] = amax(h) (codes e4m3(h * 448/amax)), and y is scaled
 *        by fl32(s_h * w2_scale[e]).
 * y [T*k,H] fp32 out, sorted order. */
int moe_grouped_gemm_w2(const moe_shape* s, const void* h, const void* w2, const float* w2_scale,
                        const int32_t* expert_offsets, const float* act_scales, float* y,
                        void* ws, size_t ws_bytes, void* stream);

/* Expert aggregation, the last stage of the fused FP8 pass
 * (agentic-affairs.com, "Triton improves the FP8 execution path";
 * codebridge-ai.com, "aws-moe-kernel-wgmma-triton-ttft", section "2. Backend
 * routing"): out[t][m] = sum_{j<k} topk_weights[t][j] * y[inv_perm[t*k+j]][m],
 * summed in fp32 in slot order and rounded once to the activation type.
 * y [T*k,H] fp32 in (sorted order), inv_perm [T*k] int32, topk_weights [T,k]
 * fp32, out [T,H] activation type out; every row of out is written once.
 * Errors: null or misaligned pointers or a bad shape (MOE_ERR_INVALID_ARG /
 * MOE_ERR_UNSUPPORTED), nothing enqueued. */
int moe_combine(const moe_shape* s, const float* y, const int32_t* inv_perm,
                const float* topk_weights, void* out, void* stream);

/* Dynamic per-tensor FP8 quantisation of an activation, the step the FP8
 * mode applies to x before the gate/up projection and to h before the down
 * projection (FP8 tensor scaling in the same pass as the matrix work:
 * agentic-affairs.com, "Triton improves the FP8 execution path";
 * codebridge-ai.com, "aws-moe-kernel-wgmma-triton-ttft", section "2.
 * Backend routing").
 *   a      [n]  bf16, device; n a positive multiple of 8
 *   codes  [n]  OCP e4m3fn codes out: e4m3(fl32(a * fl32(448 / amax))),
 *               rounded to nearest even, saturated to +-448
 *   scales [2]  fp32 out: scales[0] = s = fl32(amax / 448), scales[1] = amax
 *               = max |a| (amax = 0 gives s = 1 and multiplier 1)
 * a holds no NaN (precondition).  Null or misaligned (16 B) pointers, or n
 * not a positive multiple of 8, give MOE_ERR_INVALID_ARG; n = 0 returns
 * MOE_OK with nothing enqueued. */
int moe_act_quant_e4m3(const void* a, int64_t n, uint8_t* codes, float* scales, void* stream);

/* Inverse rotary position embedding fused with per-head FP8 quantisation:
 * the pages' second fused kernel, whose token count changes from call to
 * call (codebridge-ai.com, "aws-moe-kernel-wgmma-triton-ttft", section "3.
 * Kill JIT recompilation"; agentic-affairs.com, "Removing recompilation
 * improves the first-token result").  Compiled ahead of time; T and the
 * positions are run-time arguments, so no token count is a specialisation.
 *   x         [T, n_heads, head_dim] bf16 in, contiguous
 *   positions [T] int32: token t uses row positions[t] of the table (a value
 *             outside [0, max_pos) breaks the contract and is clamped)
 *   cos_sin   [max_pos, rot_dim] fp32: per position, the cosines of the
 *             rot_dim/2 pair angles, then their sines
 *   codes     [T, n_heads, head_dim] OCP e4m3fn codes out
 *   scales    [T, n_heads] fp32 out
 * Over the first rot_dim values of each head, a pair (a, b) -- (i, i +
 * rot_dim/2), or (2i, 2i+1) with interleaved = 1 -- becomes y_a = x_a c +
 * x_b s, y_b = x_b c - x_a s (the rotation by the negative angle: the
 * inverse of a forward rotary embedding), each product and sum a single
 * fp32 operation; values past rot_dim pass through.  Each (token, head) is
 * then quantised with its own scale: A = max |y| over the head, scales =
 * fl32(A/448), codes = e4m3(fl32(y * fl32(448/A))) rounded to nearest even
 * and saturated (A = 0: scale 1).
 * Limits: head_dim and rot_dim multiples of 16, 16 <= rot_dim <= head_dim <=
 * 512 (MOE_ERR_UNSUPPORTED otherwise); T >= 0, n_heads >= 1, max_pos >= 1,
 * T * n_heads < 2^31, pointers 16-byte aligned (MOE_ERR_INVALID_ARG).
 * T = 0 returns MOE_OK with nothing enqueued. */
int moe_inv_rope_fp8_quant(const void* x, const int32_t* positions, const float* cos_sin,
                           int32_t T, int32_t n_heads, int32_t head_dim, int32_t rot_dim,
                           int32_t max_pos, int32_t interleaved, uint8_t* codes, float* scales,
                           void* stream);

/* The whole layer in one call, the single batched operation that merges
 * routing, data shuffling and the expert calculations (readmex.ai, "AWS
 * details fused MoE kernel optimizations on SageMaker, up to 10% throughput
 * gain", summary): gating, grouping, (FP8: x quantisation), gate/up +
 * SwiGLU, (FP8: h quantisation), down projection and aggregation, enqueued
 * back to back on `stream`, with no host synchronisation.  Every token row
 * of `out` is written exactly once.
 *   x [T,H], logits [T,E] fp32, w13 [E,2I,H], w13_scale [E] (FP8), w2
 *   [E,H,I], w2_scale [E] (FP8), out [T,H]; topk_ids / topk_weights are
 *   optional outputs (NULL = kept in the workspace, see
 *   moe_workspace_routing); ws of moe_workspace_bytes(s) bytes.
 * Errors: as the step entry points, all checked before anything is
 * enqueued. */
int moe_fused_forward(const moe_shape* s, const void* x, const float* logits, const void* w13,
                      const float* w13_scale, const void* w2, const float* w2_scale, void* out,
                      int32_t* topk_ids, float* topk_weights, void* ws, size_t ws_bytes,
                      void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * layer as moe_fused_forward, same kernels and same results, without a
 * workspace argument.  Its scratch is a static device array of
 * MOE_NOALLOC_SCRATCH_BYTES per GPU, which the library holds from its first
 * use on that GPU until the process ends; nothing is allocated or freed per
 * call.  Shapes whose moe_workspace_bytes exceeds that size return
 * MOE_ERR_TOO_LARGE with nothing enqueued.  Every call on one GPU shares
 * that GPU's array: calls that overlap in time on one GPU (two streams, two
 * threads) race and give undefined results; calls ordered on one stream are
 * safe.  Arguments and errors otherwise as moe_fused_forward. */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
int moe_fused_forward_noalloc(const moe_shape* s, const void* x, const float* logits,
                              const void* w13, const float* w13_scale, const void* w2,
                              const float* w2_scale, void* out, int32_t* topk_ids,
                              float* topk_weights, void* stream);

/* Router GEMM: logits[t][e] = sum_h x[t][h] * wg[e][h] with fp32
 * accumulation, for the top-k gating (readmex.ai, "AWS details fused MoE
 * kernel optimizations on SageMaker", summary: token routing is the first
 * stage of the fused operation).
 *   x      [T,H]  activation type (fp32 in F32 mode, bf16 otherwise), device
 *   wg     [E,H]  the router weights, one row per expert, same type as x
 *   logits [T,E]  fp32 out, row-major
 * Products are exact (bf16 x bf16, or fp32 FMA in F32 mode) and summed in
 * fp32, in an order that depends on the shape, so logits may differ from an
 * exact sum by a few fp32 rounding steps of sum_h |x w|.  Uses the
 * workspace of moe_workspace_bytes(s).  Null, misaligned (16 B) pointers or
 * a small workspace give MOE_ERR_INVALID_ARG / MOE_ERR_WORKSPACE. */
int moe_router_logits(const moe_shape* s, const void* x, const void* wg, float* logits,
                      void* ws, size_t ws_bytes, void* stream);

/* The whole layer from the token activations and the router weights:
 * moe_router_logits followed by moe_fused_forward on its logits, enqueued
 * on `stream`.  logits [T,E] (optional out, NULL = kept in the workspace)
 * receives the router output the gating used. */
int moe_fused_forward_router(const moe_shape* s, const void* x, const void* wg, const void* w13,
                             const float* w13_scale, const void* w2, const float* w2_scale,
                             void* out, float* logits, int32_t* topk_ids, float* topk_weights,
                             void* ws, size_t ws_bytes, void* stream);

/* Stage timing for profiling: identical to moe_fused_forward, and in
 * addition takes timestamps into events[i] (a hipEvent_t created by the
 * caller, or NULL to skip that point) at stage boundary i, so that the
 * elapsed time between two of them is the time of the stages between:
 *   0 before gating | 1 after gating | 2 after grouping | 3 after the tile
 *   list | 4 start of the gate/up GEMM kernel | 5 its end | 6 start of the
 *   down GEMM kernel | 7 its end | 8 after the aggregation.
 * Boundaries 4-7 are the GEMM kernels' own start and end times (attached to
 * their dispatches, no marker packets around them), so 4->5 and 6->7 are
 * exactly those kernels' durations; 3->4 holds the FP8 x quantisation and
 * 5->6 the FP8 h quantisation.  The others are marker events on `stream`.
 * For few-token batches (few pairs per expert and T*k <= 256) one kernel
 * runs gating, grouping, the tile list and the x quantisation, so
 * boundaries 1 to 3 fall at the same point after it.
 * n_events must be MOE_NUM_STAGE_EVENTS. */
#define MOE_NUM_STAGE_EVENTS 9
int moe_fused_forward_events(const moe_shape* s, const void* x, const float* logits,
                             const void* w13, const float* w13_scale, const void* w2,
                             const float* w2_scale, void* out, int32_t* topk_ids,
                             float* topk_weights, void* ws, size_t ws_bytes, void* stream,
                             void** events, int32_t n_events);

#ifdef __cplusplus
}
#endif
#endif /* MOE_GFX950_H */
