/*
 * beam_moe.h -- forward pass of one Beam mixture-of-experts block on an
 * AMD Instinct MI355X (gfx950), as a plain C ABI.
 *
 * What the block computes (「Reflection 发布 Beam 501B 开源模型，支持 1M tokens 上下文」,
 * the Chinese translation of the Hugging Face post "Welcome Beam: a 501B open
 * model you can own, customize, and scale", section 专家混合模型 (mixture of
 * experts); config.json fields n_group, topk_group, norm_topk_prob,
 * routed_scaling_factor as listed in 「Reflection 放出 501B 的 Beam 权重：四套
 * 精度、滑动窗口和一场榜单落差」, section "config.json 里还有六处能直接抄的细节"):
 *
 *   1. router: s[t,e] = sigmoid(sum_h x[t,h] * W_r[e,h] + b[e]), in FP32;
 *   2. the E experts form G contiguous groups of E/G; a group's score is the
 *      sum of its two highest s; the TG best groups are kept; the K experts
 *      with the highest s inside the kept groups are selected (no shared
 *      expert);
 *   3. w[t,k] = s[t,id_k] / sum_j s[t,id_j] * routed_scaling   (x2.5 for Beam);
 *   4. every selected expert is a SwiGLU MLP:
 *        y = W_down (silu(W_gate x) * (W_up x)), no biases;
 *      the SwiGLU product is FP32 (same translation, section 残差流);
 *   5. out[t] = sum_k w[t,k] * y[t,k].
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensor pointers are DEVICE pointers owned by the caller. The library
 *   never allocates or frees device memory; scratch space is the caller's
 *   workspace (see beam_moe_workspace_bytes).
 * - Every call is asynchronous on `stream` (a hipStream_t, NULL = the null
 *   stream) and performs no host synchronisation.
 * - Arguments are validated on the host before anything is launched; on
 *   failure a negative status is returned and no output is touched. A failed
 *   launch returns BEAM_MOE_ERR_HIP; outputs are then undefined.
 * - Outputs are fully overwritten, never accumulated into. Outputs must not
 *   alias inputs.
 * - Layouts are row-major. Weights use the [out, in] ("Linear") layout.
 *   bf16 tensors are raw bfloat16 bit patterns (uint16). Every pointer must be
 *   16-byte aligned.
 * - Supported dims: 1 <= num_groups <= 64, num_experts <= 256,
 *   num_experts % num_groups == 0, 1 <= topk_groups <= num_groups,
 *   1 <= topk <= min(16, topk_groups * num_experts / num_groups),
 *   hidden % 256 == 0, intermediate % 128 == 0, routed_scaling finite.
 *   0 <= T and T * topk <= 2^28 (268,435,456 routed pairs); T == 0 is a valid
 *   no-op. Larger batches return BEAM_MOE_ERR_UNSUPPORTED.
 * - Determinism: no floating-point atomics are used; every output, integer
 *   or floating point, is bitwise identical from run to run on one device.
 * - Ties in scores are broken towards the lower group / expert index; the K
 *   ids of a token are listed by score descending, then id ascending.
 */
#ifndef BEAM_MOE_H
#define BEAM_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct beam_moe_dims {
  int32_t hidden;        /* H: 5120 for Beam (same translation, section 注意力)   */
  int32_t intermediate;  /* I: 2560 for Beam (same translation, 专家混合模型)     */
  int32_t num_experts;   /* E: 256                                                 */
  int32_t num_groups;    /* G: 8  (config.json n_group)                            */
  int32_t topk_groups;   /* TG: 4 (config.json topk_group)                         */
  int32_t topk;          /* K: 8  experts per token                                */
  float routed_scaling;  /* 2.5   (config.json routed_scaling_factor)              */
} beam_moe_dims;

enum {
  BEAM_MOE_OK = 0,
  BEAM_MOE_ERR_INVALID_ARG = -1, /* null pointer, misaligned pointer, negative T */
  BEAM_MOE_ERR_UNSUPPORTED = -2, /* dims outside the supported set above        */
  BEAM_MOE_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required  */
  BEAM_MOE_ERR_HIP = -4,         /* a HIP launch failed                          */
  BEAM_MOE_ERR_SCRATCH = -5      /* beam_moe_forward_noalloc: the batch's workspace
                                    exceeds BEAM_MOE_SCRATCH_BYTES                */
};

/* Size of the device scratch array built into the library for
 * beam_moe_forward_noalloc (one per GPU, held until the process ends). */
#define BEAM_MOE_SCRATCH_BYTES (64u << 20)

/* Bytes of workspace that the forward entry points need for T tokens (one size
 * serves all of them, and it is also enough for beam_moe_route and
 * beam_moe_dispatch; it grows linearly in T: at Beam dims about 132 KB per
 * token, mostly the fp16 SwiGLU activations [T*K, I] and the fp16 expert
 * outputs [T*K, H], each with a power-of-two scale per 64 columns).
 * Returns SIZE_MAX for invalid or unsupported dims or T. */
size_t beam_moe_workspace_bytes(const beam_moe_dims* dims, int32_t T);

/* The smaller workspace that beam_moe_route alone needs: its split-K partial
 * logits, fp32 [splits, T, E] with splits <= 16 (T * E * 4 bytes from about
 * 4096 tokens at Beam dims, where every token tile gets its own workgroup).
 * Returns SIZE_MAX for invalid or unsupported dims or T. */
size_t beam_moe_route_workspace_bytes(const beam_moe_dims* dims, int32_t T);

/* The smaller workspace that beam_moe_dispatch alone needs: int32 expert
 * histograms of each unit of 1024 pairs, ceil(T * K / 1024) * E * 4 bytes.
 * Returns SIZE_MAX for invalid or unsupported dims or T. */
size_t beam_moe_dispatch_workspace_bytes(const beam_moe_dims* dims, int32_t T);

/* Router + group-limited top-k (steps 1-3 above).
 *   x_bf16      [T, H]  bf16 hidden states
 *   w_router    [E, H]  fp32 router weight
 *   logit_bias  [E]     fp32, added to the logit before the sigmoid; NULL = none
 *   select_bias [E]     fp32 selection-only bias, NULL = none: groups and experts
 *                       are ranked by c = fl32(s + select_bias[e]) while the
 *                       weights stay the normalised unbiased scores s (the
 *                       DeepSeek-V3 scheme the post's mixture-of-experts
 *                       section names; the pages show no such vector in use)
 *   topk_ids    [T, K]  int32 out
 *   topk_w      [T, K]  fp32 out: normalised weights times routed_scaling
 *   scores_out  [T, E]  fp32 out, post-sigmoid scores; NULL = not written
 *   ws, ws_bytes        workspace of at least beam_moe_route_workspace_bytes(dims, T)
 *                       (beam_moe_workspace_bytes(dims, T) is always enough)
 * The logits are accumulated in FP32 (bf16 x times fp32 W_r, exact products). */
int beam_moe_route(const beam_moe_dims* dims, int32_t T, const void* x_bf16, const float* w_router,
                   const float* logit_bias, const float* select_bias, int32_t* topk_ids, float* topk_w,
                   float* scores_out, void* ws, size_t ws_bytes, void* stream);

/* Steps 2-3 on caller-supplied post-sigmoid FP32 scores [T, E] (select_bias as
 * in beam_moe_route, NULL = none).  Fixed FP32 evaluation order, so results are
 * reproducible bit for bit by any implementation that follows it:
 *   selection value  c = fl32(s + select_bias[e]), or c = s;
 *   group score      = fl32(c_first + c_second) of the group's two largest;
 *   topk_ids[t,:]    = the K largest c among the kept groups, c descending,
 *                      ties to the lower id;
 *   sum              = fl32 running sum of the K selected s in output order;
 *   topk_w[t,k]      = fl32(fl32(s_k / sum) * routed_scaling)   (IEEE division).
 * Needs no workspace. */
int beam_moe_select(const beam_moe_dims* dims, int32_t T, const float* scores, const float* select_bias,
                    int32_t* topk_ids, float* topk_w, void* stream);

/* Counting-sort dispatch of the T*K (token, slot) pairs by expert.
 *   topk_ids        [T, K]  int32 in [0, E) (ids outside it are skipped and
 *                           leave the outputs undefined, without faulting)
 *   expert_counts   [E]     int32 out: pairs routed to each expert
 *   expert_offsets  [E+1]   int32 out: exclusive prefix sum, [E] = T*K
 *   sorted_slots    [T*K]   int32 out: values i = t*K + k, ascending expert,
 *                           ascending i inside an expert (stable; unique)
 *   ws, ws_bytes            workspace of at least
 *                           beam_moe_dispatch_workspace_bytes(dims, T)
 *                           (beam_moe_workspace_bytes(dims, T) is always enough) */
int beam_moe_dispatch(const beam_moe_dims* dims, int32_t T, const int32_t* topk_ids, int32_t* expert_counts,
                      int32_t* expert_offsets, int32_t* sorted_slots, void* ws, size_t ws_bytes, void* stream);

/* The whole block (steps 1-5).
 *   x_bf16, w_router, logit_bias, select_bias: as in beam_moe_route
 *   w_gate, w_up  [E, I, H] bf16;  w_down [E, H, I] bf16
 *   out           [T, H] fp32 out
 *   topk_ids, topk_w, expert_counts, expert_offsets, sorted_slots: as above,
 *   written as by-products (caller-owned, all required).
 * Precision: the gate/up GEMMs run on bf16 MFMA with FP32 accumulation and
 * silu(g)*u is formed in FP32. It reaches the down projection as fp16 (RNE)
 * times a power-of-two scale shared by a block of 64 columns of a row group,
 * chosen so the block's largest magnitude stays below 2^15 (no overflow);
 * the down projection runs on fp16 MFMA with FP32 accumulation, with W_down
 * converted from bf16 to fp16, exactly where representable (magnitudes below
 * 2^-14 become fp16 subnormals, rounded toward zero; above 65504 they would
 * not be representable, far outside any weight range). The accumulators carry
 * the activations' power-of-two scales (rescaled exactly from one 64-column
 * block to the next), so large activations set no limit on the weights. The expert
 * outputs leave the down projection the same way (fp16 times a power-of-two
 * scale per 64 columns of a row group); out is their weighted sum in FP32,
 * over k in ascending order.
 * Supported intermediate sizes additionally satisfy intermediate <= 32768. */
int beam_moe_forward(const beam_moe_dims* dims, int32_t T, const void* x_bf16, const float* w_router,
                     const float* logit_bias, const float* select_bias, const void* w_gate, const void* w_up,
                     const void* w_down, float* out, int32_t* topk_ids, float* topk_w, int32_t* expert_counts,
                     int32_t* expert_offsets, int32_t* sorted_slots, void* ws, size_t ws_bytes, void* stream);

/* Converts W_down [E, H, I] from bf16 to fp16 once, for beam_moe_forward_packed
 * (a weight-load step, like quantising to FP8: the forward never repeats it).
 * Each value is converted exactly as the down kernels convert bf16 weights as
 * they read them: exactly for magnitudes in fp16's normal range [2^-14, 65504],
 * toward zero below it (subnormals), so beam_moe_forward_packed on the result
 * gives the same bits as beam_moe_forward on the bf16 weights.  Magnitudes
 * above 65504 do not fit fp16 (far outside any weight range); the result is
 * then undefined.
 *   w_down_bf16    [E, H, I] bf16
 *   w_down_packed  [E, H, I] fp16 out (caller-owned, not aliasing w_down_bf16)
 * Asynchronous on `stream`, like every call. */
int beam_moe_pack_weights(const beam_moe_dims* dims, const void* w_down_bf16, void* w_down_packed, void* stream);

/* beam_moe_forward with W_down given as beam_moe_pack_weights made it (fp16
 * [E, H, I]); all other arguments, outputs and results as beam_moe_forward, bit
 * for bit.  The down projection then copies its weights into LDS unconverted,
 * as the gate/up projection does, instead of converting each stage in
 * registers. */
int beam_moe_forward_packed(const beam_moe_dims* dims, int32_t T, const void* x_bf16, const float* w_router,
                            const float* logit_bias, const float* select_bias, const void* w_gate, const void* w_up,
                            const void* w_down_packed, float* out, int32_t* topk_ids, float* topk_w,
                            int32_t* expert_counts, int32_t* expert_offsets, int32_t* sorted_slots, void* ws,
                            size_t ws_bytes, void* stream);

/* beam_moe_forward without the workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  It allocates nothing: the scratch that
 * beam_moe_forward takes from `ws` (router partials, dispatch histograms, tile
 * table, SwiGLU activations, expert outputs) lives in a static device array of
 * BEAM_MOE_SCRATCH_BYTES (64 MiB) built into the library, one copy per GPU,
 * held until the process ends; its address is looked up once per device on the
 * first call there.
 *   - A batch fits when beam_moe_workspace_bytes(dims, T) <= BEAM_MOE_SCRATCH_BYTES
 *     (at Beam dims: T <= 471 tokens); larger ones return BEAM_MOE_ERR_SCRATCH
 *     before any launch.
 *   - Every call on one GPU uses that GPU's single array, which keeps what the
 *     last call left there: calls that overlap on one GPU (other streams, other
 *     threads) race and must be ordered by the caller.  Nothing in the array
 *     has to start at zero: a call writes every byte it reads before reading it.
 *   - `stream` must belong to the current device (BEAM_MOE_ERR_INVALID_ARG
 *     otherwise); the stage-timing diagnostics record nothing for this call.
 * Arguments, outputs and results are those of beam_moe_forward, bit for bit. */
int beam_moe_forward_noalloc(const beam_moe_dims* dims, int32_t T, const void* x_bf16, const float* w_router,
                             const float* logit_bias, const float* select_bias, const void* w_gate,
                             const void* w_up, const void* w_down, float* out, int32_t* topk_ids, float* topk_w,
                             int32_t* expert_counts, int32_t* expert_offsets, int32_t* sorted_slots,
                             void* stream);

/* The whole block with FP8 expert weights (steps 1-5 as beam_moe_forward).
 * The FP8 checkpoint of the model stores every expert weight as E4M3 and keeps
 * the router out of the quantisation (「Reflection 放出 501B 的 Beam 权重：四套
 * 精度、滑动窗口和一场榜单落差」, its parameter-precision listing of the FP8
 * repository); the scale granularity is not given there and is taken as one
 * fp32 scale per output row:  W[e][r, :] = e4m3(q[e][r, :]) * scale[e][r].
 *   w_gate_fp8, w_up_fp8  [E, I, H] uint8 E4M3 codes (OCP FP8 E4M3: bias 7,
 *                         no infinities, 0x7F / 0xFF are NaN and must not occur)
 *   gate_scale, up_scale  [E, I] fp32
 *   w_down_fp8            [E, H, I] uint8 E4M3 codes;  down_scale [E, H] fp32
 *   other arguments as in beam_moe_forward (the router stays FP32).
 * Precision: the codes are decoded exactly to bf16 (gate/up, against the bf16
 * x) or fp16 (down, against the fp16 activations) in registers; products
 * accumulate in FP32 and the row scale multiplies the accumulated sum; the
 * rest as in beam_moe_forward, whose choice between the few-rows-per-expert
 * kernels and the grouped GEMMs it shares.
 * Supported sizes additionally satisfy hidden % 256 == 0 and
 * intermediate % 256 == 0; the workspace is beam_moe_workspace_bytes(dims, T). */
int beam_moe_forward_fp8(const beam_moe_dims* dims, int32_t T, const void* x_bf16, const float* w_router,
                         const float* logit_bias, const float* select_bias, const uint8_t* w_gate_fp8,
                         const float* gate_scale, const uint8_t* w_up_fp8, const float* up_scale,
                         const uint8_t* w_down_fp8, const float* down_scale, float* out, int32_t* topk_ids,
                         float* topk_w, int32_t* expert_counts, int32_t* expert_offsets, int32_t* sorted_slots,
                         void* ws, size_t ws_bytes, void* stream);

/* The block as a residual sublayer at step `step` of the stream
 * (「Reflection 发布 Beam 501B 开源模型，支持 1M tokens 上下文」, section 残差流:
 * the input embedding is step 1; at step k a sublayer's output enters with
 * weight 1/sqrt(k) and the stream is kept with weight sqrt((k-1)/k); every
 * sublayer is normalised before and after, in FP32):
 *   x          = bf16(norm(stream_in) * norm_in_weight)          (RNE)
 *   out        = the block on x, as beam_moe_forward
 *   stream_out = sqrt((step-1)/step) * stream_in + 1/sqrt(step) * norm(out) * norm_out_weight
 * norm(v) = v / sqrt(mean(v^2) + norm_eps) over the H columns of a token (RMSNorm;
 * the pages name neither form, weights nor eps).  The norm statistics are taken in
 * FP64, the rest in FP32.
 *   stream_in        [T, H] fp32
 *   step             >= 2
 *   norm_in_weight, norm_out_weight   [H] fp32, NULL = ones
 *   norm_eps         >= 0, finite
 *   stream_out       [T, H] fp32 out; may be stream_in itself (in-place update)
 *   other arguments as in beam_moe_forward.  The workspace also holds x.
 * Supported hidden sizes additionally satisfy hidden <= 8192. */
int beam_moe_residual_forward(const beam_moe_dims* dims, int32_t T, const float* stream_in, int32_t step,
                              const float* norm_in_weight, const float* norm_out_weight, float norm_eps,
                              const float* w_router, const float* logit_bias, const float* select_bias,
                              const void* w_gate, const void* w_up, const void* w_down, float* stream_out,
                              int32_t* topk_ids, float* topk_w, int32_t* expert_counts, int32_t* expert_offsets,
                              int32_t* sorted_slots, void* ws, size_t ws_bytes, void* stream);

/* beam_moe_residual_forward with FP8 expert weights: the arguments of
 * beam_moe_residual_forward, with the expert weights given as in
 * beam_moe_forward_fp8 (E4M3 codes and fp32 per-row scales) and the same size
 * requirements as both. */
int beam_moe_residual_forward_fp8(const beam_moe_dims* dims, int32_t T, const float* stream_in, int32_t step,
                                  const float* norm_in_weight, const float* norm_out_weight, float norm_eps,
                                  const float* w_router, const float* logit_bias, const float* select_bias,
                                  const uint8_t* w_gate_fp8, const float* gate_scale, const uint8_t* w_up_fp8,
                                  const float* up_scale, const uint8_t* w_down_fp8, const float* down_scale,
                                  float* stream_out, int32_t* topk_ids, float* topk_w, int32_t* expert_counts,
                                  int32_t* expert_offsets, int32_t* sorted_slots, void* ws, size_t ws_bytes,
                                  void* stream);

/* Diagnostics: device time of the stages of beam_moe_forward,
 * beam_moe_forward_fp8 and both residual entry points ("prenorm" is empty
 * except in the last two).
 * beam_moe_timing_enable(1) makes later calls of any of them record HIP
 * events between their stages on the caller's stream (a marker per stage,
 * no synchronisation; the events are created by the library on first use and
 * kept for reuse). beam_moe_timing_read waits for the last recorded call,
 * writes for each stage the milliseconds summed over the calls recorded since
 * the previous read (stage_ms[s], s < *n_stages <= max_stages) and the number
 * of calls, then starts a new recording window. Stage names come from
 * beam_moe_stage_name. Not meant for concurrent calls from several threads. */
int beam_moe_timing_enable(int enable);
int beam_moe_timing_read(float* stage_ms, int32_t max_stages, int32_t* n_stages, int32_t* calls);
const char* beam_moe_stage_name(int32_t stage);

/* Diagnostics: which expert kernels the forward entry points run for T tokens.
 * Returns R > 0 when they take the stream kernels on tiles of at most R rows of
 * one expert (8, 16, 32 or 64: the smallest at least twice the average rows per
 * expert, T * topk / num_experts), 0 when they take the grouped GEMMs (256-row
 * tiles; from 32 average rows per expert, or where the stream kernels do not
 * fit the shape), or a negative status for invalid or unsupported dims.
 * fp8 != 0 asks about beam_moe_forward_fp8. */
int beam_moe_stream_rows(const beam_moe_dims* dims, int32_t T, int fp8);

/* Static string for a status code. */
const char* beam_moe_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* BEAM_MOE_H */
