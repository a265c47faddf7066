/*
 * fq.h -- C ABI of libfq: scale-only fake-quant MoE grouped GEMM on gfx950.
 *
 * The method (AngelSlim mcore_qad article, hnwysp.cn news 88453):
 *   section 一   BF16 weights are frozen; the forward fake-quantizes weights
 *               and activations (quantize -> dequantize); only the quantizer
 *               scales are trained.
 *   section 二.3 weights are fake-quantized transparently (parametrization)
 *               and each linear's input by a forward pre-hook; the gradient
 *               reaches the scales through autograd; router and output layer
 *               stay unquantized.
 *   section 二.4 each MoE layer's experts become one 3D weight stack
 *               [E, N, K]; the whole stack is fake-quantized in one
 *               vectorized pass and all experts run as one grouped GEMM.
 *   section 三   formats nvfp4 (W4A4), fp8 (W8A8), w4a16 (int4), w8a8 (int8).
 * The QAT + DeepSpeed ZeRO-3 page of the AngelSlim docs fixes that the
 * fake-quant output is cast back to the input dtype (bf16) and that the
 * matmul runs on bf16 operands ("Quantizer 的变更"), and that weight scales
 * are learnable while activation scales are not (example yaml).
 *
 * Numerics shared by every entry point (fp32, round-to-nearest-even, no
 * fused multiply-add in codec arithmetic):
 *   r = 1/s (one correctly rounded fp32 division per scale), z = x * r,
 *   c = Q(clamp(z, lo, hi)) on the format's grid (ties to even),
 *   v = fp32(value(c) * s), output bf16 = RNE(v).
 *   int8  : symmetric, lo/hi = -128/127, value(c) = c, +0.0 for c = 0.
 *   int4  : asymmetric, codes 0..15, zp' = clamp(rne(zp), 0, 15),
 *           value = c - zp', +0.0 for a zero value.
 *   fp8   : OCP E4M3 (bias 7, max 448, subnormals kept, saturating); the
 *           sign of z is kept (-0.0 possible).
 *   nvfp4 : E2M1 values {0, .5, 1, 1.5, 2, 3, 4, 6} in blocks of 16 along K;
 *           block scale s_b = fp32(E4M3(clamp(theta_b, 0, 448)) * g), with
 *           theta_b the learnable fp32 block parameter and g an fp32 tensor
 *           scale (one per expert for weights, one scalar for activations);
 *           s_b == 0 makes the block +0.0. Activation blocks are dynamic:
 *           theta_b = E4M3(clamp(amax_b * (1/(6*g)), 0, 448)).
 * Backward (straight-through estimator): mask m = [lo <= z <= hi] on the
 * unrounded z (inclusive); dv/dx = m; dv/ds = value(c) - m*z; int4
 * dv/dzp = -s*(1-m); nvfp4 dv/dtheta = g*[0 <= theta <= 448]*(value(c)-m*z).
 *
 * Conventions for every call:
 *   - Tensor pointers are DEVICE memory owned by the caller (contiguous,
 *     row-major, 16-byte aligned). bf16 tensors are raw 16-bit storage.
 *   - The library keeps no state between calls and allocates nothing inside
 *     a call; scratch memory comes from the caller's workspace (`ws`,
 *     `ws_bytes`, sized by fq_workspace_bytes). Calls enqueue work on
 *     `stream` (a hipStream_t; NULL = the default stream) and never
 *     synchronize it. Row counts of routed tensors are read on the device
 *     from seg_offsets[E], so no device-to-host copy happens.
 *   - Host-checkable problems return a status before any launch: NULL
 *     required pointer, non-positive or unsupported sizes, misalignment,
 *     an unsupported format, a workspace that is too small. A launch failure
 *     returns FQ_ERR_HIP. fq_last_error() gives a thread-local message for
 *     the last non-OK status. On error, outputs are undefined.
 *   - Device-data preconditions are NOT checked: scales finite and > 0
 *     (nvfp4 theta >= 0 and g > 0), expert ids valid, seg_offsets
 *     non-decreasing with seg_offsets[E] <= R_max.
 *   - Results are deterministic (bitwise reproducible run to run).
 */
#ifndef FQ_H
#define FQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FQ_ABI_VERSION 2

typedef enum {
  FQ_OK = 0,
  FQ_ERR_INVALID_ARGUMENT = 1,
  FQ_ERR_UNSUPPORTED = 2,
  FQ_ERR_WORKSPACE_TOO_SMALL = 3,
  FQ_ERR_HIP = 4
} fq_status;

typedef enum {
  FQ_FMT_NONE = 0,      /* no fake-quant (identity, mask 1)              */
  FQ_FMT_INT8 = 1,      /* int8 symmetric                                 */
  FQ_FMT_INT4 = 2,      /* int4 asymmetric with integer zero point        */
  FQ_FMT_FP8_E4M3 = 3,  /* OCP FP8 E4M3                                   */
  FQ_FMT_NVFP4 = 4      /* E2M1 + block-16 E4M3 scale + fp32 tensor scale */
} fq_format;

/* A stacked weight [E, N, K] (E experts, N output channels, K inputs; K
 * contiguous). A dense linear is E = 1. */
typedef struct {
  int32_t E, N, K;
} fq_shape;

/* Weight quantizer (learnable scales).
 *   group       : elements per scale along K. int8 / fp8: K (per output
 *                 channel) or a divisor of K that is a multiple of 16;
 *                 int4: 128 (any multiple of 16 dividing K); nvfp4: 16.
 *                 int8 / fp8 also FQ_GROUP_TENSOR: one scale per expert
 *                 matrix [N, K] (the per-tensor weights of the fp8_static
 *                 preset, QAT + ZeRO-3 page, example configs); scale and
 *                 dscale are then [E].
 *   scale       : [E, N, K/group] fp32. nvfp4: the block parameter theta.
 *   zero_point  : [E, N, K/group] fp32 holding integers; int4 only, else NULL.
 *   global_scale: [E] fp32 tensor scale g; nvfp4 only, else NULL. */
#define FQ_GROUP_TENSOR (-1)

typedef struct {
  int32_t fmt;
  int32_t group;
  const float *scale;
  const float *zero_point;
  const float *global_scale;
} fq_weight_q;

/* Activation quantizer. fmt NONE, FP8_E4M3 (scale = per-tensor s_a, one
 * device float), NVFP4 (scale = g_a, one device float; block scales dynamic
 * per 16 elements along K), INT8 (per-tensor s_a). The scale is frozen
 * (calibrated) by default; for FP8 and INT8 it may be learnable, and then
 * fq_swiglu_bwd / fq_moe_unpermute_reduce also return its gradient. */
typedef struct {
  int32_t fmt;
  const float *scale;
} fq_act_q;

typedef void *fq_stream; /* hipStream_t */

/* ------------------------------------------------------------------------
 * observer_absmax_init -- initial scales from observed statistics.
 * Sources: the PTQ weight scale max|W|/448 (QAT + ZeRO-3 page, "Quantizer
 * 初始值"); activation scales from a calibration forward (same page,
 * overview); per-channel min/max turned into quantization parameters
 * (msmodelslim multi-card page, FA3 observer section).
 *
 * per_tensor == 0 (weights): x is a stack [E, N, K] and
 *   int8 : scale[e,n,g] = amax_g / 127
 *   fp8  : scale[e,n,g] = amax_g / 448
 *   int4 : lo = min(0, min_g), hi = max(0, max_g), scale = (hi-lo)/15,
 *          zero_point = clamp(rne(-lo * (1/scale)), 0, 15)
 *   nvfp4: global_scale[e] = amax_e / 2688,
 *          scale[e,n,b] = E4M3(clamp(amax_b * (1/(6*g_e)), 0, 448))
 *   group FQ_GROUP_TENSOR (int8 / fp8): scale[e] = amax over expert e's
 *          matrix / 127 resp. 448
 * per_tensor == 1 (activations): x is any tensor of E*N*K elements and
 *   scale[0] = amax / D with D = 448 (fp8), 2688 (nvfp4), 127 (int8).
 * Each division is one IEEE fp32 division; a zero amax gives scale 1.0.
 * Outputs (device, caller-owned) are overwritten. ws may be NULL
 * (needs 0 bytes). Requires K % 8 == 0 and K % group == 0 (weights).
 * ---------------------------------------------------------------------- */
fq_status observer_absmax_init(const uint16_t *x_bf16, fq_shape shape, int32_t fmt,
                               int32_t group, int32_t per_tensor, float *scale,
                               float *zero_point, float *global_scale, void *ws,
                               size_t ws_bytes, fq_stream stream);

/* ------------------------------------------------------------------------
 * fq_quantize_stacked -- one vectorized fake-quant pass over a whole
 * weight stack [E, N, K] (mcore_qad article, section 二.4).
 *   w_fq_bf16 : [E, N, K] bf16 dequantized values, or NULL.
 *   codes     : integer codes, or NULL. int8 / fp8: one byte per element
 *               (int8 two's complement, E4M3 byte); int4 / nvfp4: two
 *               4-bit codes per byte, even k in the low nibble (int4 codes
 *               0..15, E2M1 nibble with the sign in bit 3).
 * At least one output must be non-NULL. Requires K % 8 == 0.
 * ---------------------------------------------------------------------- */
fq_status fq_quantize_stacked(const uint16_t *w_bf16, fq_shape shape, const fq_weight_q *q,
                              uint16_t *w_fq_bf16, uint8_t *codes, fq_stream stream);

/* ------------------------------------------------------------------------
 * Real-quantized export (QAT + ZeRO-3 page, convert / save_format=real: each
 * quantized linear keeps its codes with its weight scale; mcore_qad article,
 * section 三: the formats' stored layouts are the deployment side's).
 * The codes are fq_quantize_stacked's `codes` output. The stored tensors:
 *   int8 : codes int8 [E,N,K]; scale fp32 [E,N,K/group] (or [E] per tensor)
 *   fp8  : codes E4M3 bytes [E,N,K]; scale fp32 as int8
 *   int4 : codes [E,N,K/2] (even k in the low nibble); scale fp32
 *          [E,N,K/group]; zero point uint8 [E,N,K/group]
 *   nvfp4: codes [E,N,K/2] (E2M1, sign in bit 3, even k low); block scale
 *          E4M3 bytes [E,N,K/16]; tensor scale fp32 [E] (global_scale)
 *
 * fq_export_scales: the parameters that change form.
 *   nvfp4: scale_bytes[e,n,b] = E4M3 code of clamp(theta, 0, 448) (the
 *          rounding the forward applies to theta); theta 16-byte aligned,
 *          scale_bytes 4-byte aligned.
 *   int4 : zero_point_bytes[e,n,g] = clamp(rne(zp), 0, 15).
 *   int8 / fp8 store their fp32 scale unchanged: FQ_ERR_INVALID_ARGUMENT.
 * fq_dequantize_stacked: w_bf16[e,n,k] = bf16(fp32(value(code) * s)) with s
 *   the group scale (int4: value = code - zero point, +0.0 for 0; nvfp4:
 *   s = fp32(E4M3 value(scale byte) * global_scale[e])), the FQ pass's own
 *   arithmetic: decoding an export gives exactly the fake-quant values.
 *   group as in fq_weight_q (FQ_GROUP_TENSOR for int8 / fp8 per tensor);
 *   unused pointers may be NULL. Requires K % 16 == 0, codes 8-byte and
 *   w_bf16 16-byte aligned.
 * ---------------------------------------------------------------------- */
fq_status fq_export_scales(fq_shape shape, const fq_weight_q *q, uint8_t *scale_bytes,
                           uint8_t *zero_point_bytes, fq_stream stream);
fq_status fq_dequantize_stacked(const uint8_t *codes, fq_shape shape, int32_t fmt, int32_t group,
                                const float *scale, const uint8_t *scale_bytes,
                                const uint8_t *zero_point_bytes, const float *global_scale,
                                uint16_t *w_bf16, fq_stream stream);

/* ------------------------------------------------------------------------
 * fq_topk_kl -- top-K KL distillation between student and teacher logits
 * (mcore_qad article, section 二.5: the KL only over the teacher's top-k
 * tokens, so the [tokens, vocab] probabilities are never formed; QAT +
 * ZeRO-3 page, loss table: kl_top_K forward, r_kl_top_K reverse, averaged
 * over the valid tokens). Per token t:
 *   S    = the K largest teacher logits (equal logits: lower index first),
 *          written to topk_idx[t, 0:K] in increasing vocabulary order;
 *   p, q = softmax of the teacher's / student's logits restricted to S;
 *   loss_tok[t] = sum_S p (log p - log q)   (reverse != 0: sum_S q (log q -
 *                 log p)); 0 for an invalid token;
 *   grad[t, i]  = d loss_mean / d student logit at topk_idx[t, i]:
 *                 (q - p) / n (reverse: q ((log q - log p) - loss_tok) / n),
 *                 0 for an invalid token; every other logit's gradient is 0;
 *   loss_mean[0] = sum_t loss_tok[t] / n, n = number of valid tokens
 *                 (valid[t] != 0; valid NULL = all; n = 0 counts as 1).
 * student_bf16, teacher_bf16 [T, V] bf16 (16-byte aligned); topk_idx
 * [T, K] int32; grad [T, K] fp32; loss_tok [T] fp32; loss_mean one float.
 * Requires V % 8 == 0 and 1 <= K <= min(V, 4096). Workspace:
 * fq_workspace_bytes(FQ_OP_TOPK_KL, ...) bytes (one float). Sums are
 * taken in a fixed order (bitwise reproducible); exp / log are the
 * hardware's (relative error a few 2^-24).
 * ---------------------------------------------------------------------- */
fq_status fq_topk_kl(const uint16_t *student_bf16, const uint16_t *teacher_bf16, int32_t T,
                     int32_t V, int32_t K, int32_t reverse, const uint8_t *valid,
                     int32_t *topk_idx, float *grad, float *loss_tok, float *loss_mean, void *ws,
                     size_t ws_bytes, fq_stream stream);

/* ------------------------------------------------------------------------
 * fq_moe_permute -- routed-token permutation for one grouped GEMM over all
 * local experts (mcore_qad article, section 二.4: one GEMM over routed
 * tokens needs each expert's rows contiguous).
 *   expert_ids [T, topk] int32 global expert ids. Pair f = t*topk + j.
 *   Local pairs have expert in [expert_begin, expert_begin + E_local).
 *   perm[r]        (r < R): the local pairs sorted by (local expert, f),
 *                  a stable counting sort; perm has room for T*topk.
 *   row_of[t, j]   position of pair f in perm, -1 if not local.
 *   seg_offsets    [E_local + 1]: exclusive prefix sum of per-expert
 *                  counts; seg_offsets[E_local] = R.
 * Workspace: fq_workspace_bytes(FQ_OP_PERMUTE, {E_local, 0, 0}, T*topk, 0).
 * T == 0 is valid (all offsets 0).
 * ---------------------------------------------------------------------- */
fq_status fq_moe_permute(const int32_t *expert_ids, int32_t T, int32_t topk,
                         int32_t expert_begin, int32_t E_local, int32_t *perm,
                         int32_t *row_of, int32_t *seg_offsets, void *ws, size_t ws_bytes,
                         fq_stream stream);

/* ------------------------------------------------------------------------
 * fq_moe_permute_noalloc -- fq_moe_permute for callers that cannot allocate
 * or pass device memory of their own (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): the same arguments and
 * results, bit for bit, without a workspace. Its scratch (the per-chunk
 * counts and expert totals) is a static 4 MiB device array inside the
 * library; each GPU holds its own copy from the first call on it until the
 * process ends. The call allocates nothing.
 *   Limit: 4 * E_local * (ceil(T*topk / 256) + 1) <= 4 MiB, e.g. T*topk up
 *   to 2,096,896 pairs at E_local = 128. Larger requests return
 *   FQ_ERR_WORKSPACE_TOO_SMALL before anything is enqueued.
 *   Every call on one GPU shares that GPU's array: calls that can overlap
 *   on the device (other streams, other host threads) race; serialize them
 *   on one stream. A call overwrites what the last one left there.
 * ---------------------------------------------------------------------- */
fq_status fq_moe_permute_noalloc(const int32_t *expert_ids, int32_t T, int32_t topk,
                                 int32_t expert_begin, int32_t E_local, int32_t *perm,
                                 int32_t *row_of, int32_t *seg_offsets, fq_stream stream);

/* ------------------------------------------------------------------------
 * fq_validate -- debug check of the device-data preconditions that the other
 * calls assume and do not check (their host checks see only sizes and
 * pointers): the quantizer's parameters are scales of a fake-quant grid
 * (mcore_qad article, section 二.3) and must be usable as such, and the
 * routing feeds one grouped GEMM over per-expert segments (section 二.4).
 *   expert_ids [T, topk] (NULL: skipped): every id in [0, n_experts).
 *   seg_offsets [E+1] (NULL: skipped): seg[0] == 0, non-decreasing,
 *              0 <= seg[E] <= R_max.
 *   wq (NULL: skipped), with shape: scales finite and > 0 (INT8 / INT4 /
 *              FP8), NVFP4 theta finite and >= 0, zero points finite, NVFP4
 *              global scales finite and > 0.
 *   aq (NULL or fmt NONE: skipped): the activation scale finite and > 0.
 *   status     one device uint32, overwritten with the OR of the FQ_BAD_*
 *              bits of the failed conditions (0: all hold).
 * The kernels only read their inputs: a bad input is reported, never
 * faulted on. Enqueued on `stream`; read status after synchronizing. Host
 * errors (NULL status, bad sizes) return before anything is enqueued.
 * ---------------------------------------------------------------------- */
#define FQ_BAD_EXPERT_ID 0x01u
#define FQ_BAD_SEG_START 0x02u
#define FQ_BAD_SEG_ORDER 0x04u
#define FQ_BAD_SEG_END 0x08u
#define FQ_BAD_SCALE 0x10u
#define FQ_BAD_ZERO_POINT 0x20u
#define FQ_BAD_GLOBAL_SCALE 0x40u
#define FQ_BAD_ACT_SCALE 0x80u
fq_status fq_validate(const int32_t *expert_ids, int32_t T, int32_t topk, int32_t n_experts,
                      const int32_t *seg_offsets, int32_t E, int32_t R_max, fq_shape shape,
                      const fq_weight_q *wq, const fq_act_q *aq, uint32_t *status,
                      fq_stream stream);

/* ------------------------------------------------------------------------
 * fq_grouped_gemm_fwd -- Y[r, :] = FQ_a(X)[r, :] . FQ_w(W[e])^T for every
 * routed row r in segment e = [seg_offsets[e], seg_offsets[e+1]), fp32
 * accumulation on bf16 MFMA, bf16 output (mcore_qad article, sections 二.3
 * and 二.4).
 *   x_bf16  [R_max, K] rows in expert order; rows >= seg_offsets[E] are
 *           ignored and the matching rows of y are left untouched.
 *   w_bf16  [E, N, K] raw frozen weights with quantizer wq.
 *   w_fq    NULL, or FQ_w(W) already materialized by fq_quantize_stacked
 *           with the same quantizer (then w_bf16 is not read). With NULL
 *           the call materializes it in the workspace. With wq NULL, w_fq
 *           is used as given: passing the raw weights there is the
 *           quantization-off forward of the self-teacher (mcore_qad
 *           article, section 一).
 *   aq      activation quantizer applied to x first (NULL = NONE).
 *   y_bf16  [R_max, N].
 * Requires N % 16 == 0 and K % 16 == 0. The kernels work on N % 256 == 0,
 * K % 64 == 0; other shapes run on zero-padded copies of W_fq, x and y in
 * the workspace (the padded K columns add nothing, the padded N rows are
 * not copied back), at the cost of those copies.
 * Workspace: fq_workspace_bytes(FQ_OP_GEMM_FWD, shape, R_max, wq->fmt | aq->fmt << 8).
 * A call whose 256 x 256 output tiles would leave half of the GPU's CUs or
 * more idle splits each tile's contraction into 2-8 parts and adds the
 * parts' fp32 sums in part order afterwards (S * R_max * N * 4 bytes of the
 * workspace). The split is optional: a workspace that holds everything
 * else but not these sums runs the call unsplit (so a tile-aligned shape
 * with w_fq given and no activation FQ may pass no workspace). Results are
 * deterministic for a given R_max, shape, workspace size and device.
 * ---------------------------------------------------------------------- */
fq_status fq_grouped_gemm_fwd(const uint16_t *x_bf16, int32_t R_max, const int32_t *seg_offsets,
                              fq_shape shape, const uint16_t *w_bf16, const uint16_t *w_fq,
                              const fq_weight_q *wq, const fq_act_q *aq, uint16_t *y_bf16,
                              void *ws, size_t ws_bytes, fq_stream stream);

/* ------------------------------------------------------------------------
 * fq_grouped_gemm_bwd_scale -- backward of fq_grouped_gemm_fwd with the
 * weights frozen: dX and the weight-quantizer gradients only (mcore_qad
 * article, section 一: only scales train; section 二.3: the gradient flows
 * to the scale).
 *   dx    = m_x * (dY_e . FQ_w(W[e]))                     [R_max, K] bf16
 *   dWq_e = dY_e^T . FQ_a(X)_e                            (never stored)
 *   dscale[e,n,g]     = sum_{k in g} dWq_e[n,k] * dv/ds(e,n,k)   fp32
 *   dzero_point[e,n,g]= sum_{k in g} dWq_e[n,k] * dv/dzp(e,n,k)  (int4)
 *   per-tensor scale  : dscale[e] = sum over n of the per-channel sums
 *                       (each channel's in the order above, the channels
 *                       in a fixed-order tree)
 * dx, dscale, dzero_point may each be NULL (not computed). dscale is
 * overwritten (not accumulated); experts without rows get 0. dScale is
 * reduced in a fixed order (no float atomics): an expert's rows are
 * contracted in chunks of at most 2048, each chunk's partial sums summed in
 * chunk order.
 *   dy_bf16 [R_max, N]; x_bf16 [R_max, K] raw (pre activation fake-quant).
 * Requires N % 16 == 0 and K % 16 == 0; for dScale a group of 16, 32, 64
 * or a multiple of 128 (a per-channel group may be any K), and (nvfp4) theta
 * 16-byte aligned. The kernels work on N % 256 == 0, K % 256 == 0; other
 * shapes run on zero-padded copies in the workspace (a padded weight element
 * is 0 with a neutral scale: 1 on the integer / FP8 grids, theta 0 for
 * NVFP4, zero point 0, so its straight-through factor is 0), and only the
 * call's own region of dx, dscale and dzero_point is written.
 * Workspace: fq_workspace_bytes(FQ_OP_GEMM_BWD, shape, R_max, wq->fmt | aq->fmt << 8);
 * dX of a small call splits its contraction as the forward does (optional
 * in the same way: S * R_max * K * 4 bytes).
 * ---------------------------------------------------------------------- */
fq_status fq_grouped_gemm_bwd_scale(const uint16_t *dy_bf16, const uint16_t *x_bf16,
                                    int32_t R_max, const int32_t *seg_offsets, fq_shape shape,
                                    const uint16_t *w_bf16, const uint16_t *w_fq,
                                    const fq_weight_q *wq, const fq_act_q *aq,
                                    uint16_t *dx_bf16, float *dscale, float *dzero_point,
                                    void *ws, size_t ws_bytes, fq_stream stream);

/* ------------------------------------------------------------------------
 * The expert input as token rows. The forward pre-hook fake-quantizes a
 * token's input once, however many experts it is routed to (mcore_qad
 * article, section 二.3). The grouped GEMM (section 二.4) can then read
 * routed row r as token row perm[r] / topk, and the [R, K] gathered copy is
 * never formed.
 *
 * fq_actfq: xq = FQ_a(x), row by row (NVFP4: 16-blocks along K).
 *   x, xq [rows, K] bf16, K % 16 == 0. aq NULL or FMT_NONE copies x.
 * fq_grouped_gemm_fwd_tokens: fq_grouped_gemm_fwd with, for every routed
 *   row r < seg_offsets[E], x_bf16[r] = x_tok[perm[r] / topk].
 *   x_tok [T, K] is already fake-quantized, so the call takes no
 *   activation quantizer. perm [>= seg_offsets[E]] is fq_moe_permute's
 *   (the (token, slot) pair index of each routed row), topk its slot count.
 * fq_grouped_gemm_wgrad_tokens: the dScale (and int4 dzero_point) part of
 *   fq_grouped_gemm_bwd_scale, with the same row map for x. dX does not
 *   read x, so it stays with fq_grouped_gemm_bwd_scale.
 * Results are bitwise those of the plain calls on the gathered rows.
 * Requirements and errors are the plain calls', plus T >= 0, topk > 0, and
 * perm / x_tok non-NULL unless R_max == 0.
 * Workspace: fq_workspace_bytes(FQ_OP_GEMM_FWD, shape, max(R_max, T),
 *   w_fq ? 0 : wq->fmt), resp. fq_workspace_bytes(FQ_OP_GEMM_BWD, shape,
 *   max(R_max, T), 0); the zero-padded path copies the T token rows. The
 *   forward splits its contraction (see fq_grouped_gemm_fwd) when the
 *   workspace also holds the parts' sums for R_max rows, which the size
 *   for max(R_max, T) = R_max does; the bits then equal the plain call's
 *   with the same workspace.
 * ---------------------------------------------------------------------- */
fq_status fq_actfq(const uint16_t *x_bf16, int32_t rows, int32_t K, const fq_act_q *aq,
                   uint16_t *xq_bf16, fq_stream stream);
fq_status fq_grouped_gemm_fwd_tokens(const uint16_t *x_tok_bf16, int32_t T, const int32_t *perm,
                                     int32_t topk, int32_t R_max, const int32_t *seg_offsets,
                                     fq_shape shape, const uint16_t *w_bf16, const uint16_t *w_fq,
                                     const fq_weight_q *wq, uint16_t *y_bf16, void *ws,
                                     size_t ws_bytes, fq_stream stream);
fq_status fq_grouped_gemm_wgrad_tokens(const uint16_t *dy_bf16, const uint16_t *x_tok_bf16,
                                       int32_t T, const int32_t *perm, int32_t topk,
                                       int32_t R_max, const int32_t *seg_offsets, fq_shape shape,
                                       const uint16_t *w_bf16, const fq_weight_q *wq,
                                       float *dscale, float *dzero_point, void *ws,
                                       size_t ws_bytes, fq_stream stream);

/* ------------------------------------------------------------------------
 * MoE-layer elementwise steps around the grouped GEMMs (the routed-expert
 * path of one layer: gather -> gate_up GEMM -> SwiGLU -> down GEMM ->
 * combine, and its backward). R = seg_offsets[E] is read on the device
 * through `n_rows` (= &seg_offsets[E]); rows >= R are not touched.
 *
 * fq_moe_gather_actfq: xq[row_of[t,j]] = FQ_a(x[t]) for every routed slot
 *   (row_of[t,j] >= 0; forward pre-hook on the expert input, mcore_qad
 *   article section 二.3). x [T, H]; row_of [T, topk] from fq_moe_permute;
 *   xq [R, H]. Each token row is read and fake-quantized once.
 * fq_swiglu_actfq: a = bf16(silu(h[:, :F]) * h[:, F:]), aq = FQ_a(a).
 *   h [R_max, 2F]; a_out may be NULL; aq_out [R_max, F]. The gate half is
 *   the first F columns. silu(g) = g / (1 + exp(-g)) in fp32.
 * fq_swiglu_bwd: da = m_a * daq (m_a the activation-FQ mask of a, recomputed
 *   from h), dh = [da*u*s*(1+g*(1-s)), da*g*s] with s = sigmoid(g).
 * fq_moe_combine: out[t] = bf16(sum_j p[t,j] * o[row_of[t,j]]) over local
 *   slots j ascending (fp32); tokens without local slots get 0.
 * fq_moe_combine_bwd: do[row_of[t,j]] = bf16(p[t,j] * dout[t]) for every
 *   routed slot; each dout row is read once.
 * fq_moe_unpermute_reduce: dx[t] = bf16(m_a(x[t]) * sum_j dxq[row_of[t,j]]).
 * All require H (resp. F) % 16 == 0 and T * H (resp. R_max * F) < 2^35.
 * T == 0 launches nothing (the token pointers may then be NULL).
 *
 * Learnable activation scale (fq_swiglu_bwd, fq_moe_unpermute_reduce): the
 * gradient reaches a quantizer scale through autograd (mcore_qad article,
 * section 二.3), here with the weights' straight-through factor dv/ds =
 * value(c) - m*z. dscale_a (one device float, or NULL = scale frozen, no
 * extra work) is OVERWRITTEN with
 *   swiglu_bwd       : dS_a2 = sum over rows < R and f of daq * dv/ds(a)
 *   unpermute_reduce : dS_a1 = sum over t, h of
 *                      (sum_j dxq[row_of[t,j], h]) * dv/ds(x[t, h])
 * (0 for an empty batch). Only FP8 and INT8 activations have such a scale
 * (else FQ_ERR_UNSUPPORTED). Each block's fp32 partial goes to the
 * workspace `ws` (at least fq_workspace_bytes(FQ_OP_ACT_SCALE_GRAD,
 * {1, rows, cols}, 0, 0) bytes with rows x cols = R_max x F, resp. T x H),
 * then one block sums them in a fixed order, so the result is bitwise
 * reproducible. ws / ws_bytes are ignored when dscale_a is NULL.
 * ---------------------------------------------------------------------- */
fq_status fq_moe_gather_actfq(const uint16_t *x_bf16, int32_t T, int32_t H, const int32_t *row_of,
                              int32_t topk, const fq_act_q *aq, uint16_t *xq_bf16,
                              fq_stream stream);
fq_status fq_swiglu_actfq(const uint16_t *h_bf16, int32_t R_max, const int32_t *n_rows, int32_t F,
                          const fq_act_q *aq, uint16_t *a_bf16, uint16_t *aq_bf16,
                          fq_stream stream);
fq_status fq_swiglu_bwd(const uint16_t *daq_bf16, const uint16_t *h_bf16, int32_t R_max,
                        const int32_t *n_rows, int32_t F, const fq_act_q *aq, uint16_t *dh_bf16,
                        float *dscale_a, void *ws, size_t ws_bytes, fq_stream stream);
fq_status fq_moe_combine(const uint16_t *o_bf16, const float *probs, const int32_t *row_of,
                         int32_t T, int32_t topk, int32_t H, uint16_t *out_bf16,
                         fq_stream stream);
fq_status fq_moe_combine_bwd(const uint16_t *dout_bf16, const float *probs, const int32_t *row_of,
                             int32_t T, int32_t topk, int32_t H, uint16_t *do_bf16,
                             fq_stream stream);
fq_status fq_moe_unpermute_reduce(const uint16_t *dxq_bf16, const int32_t *row_of,
                                  const uint16_t *x_bf16, int32_t T, int32_t topk, int32_t H,
                                  const fq_act_q *aq, uint16_t *dx_bf16, float *dscale_a,
                                  void *ws, size_t ws_bytes, fq_stream stream);

/* Workspace sizing. op: one of FQ_OP_*. fmts = weight fmt | act fmt << 8. */
#define FQ_OP_PERMUTE 1
#define FQ_OP_GEMM_FWD 2
#define FQ_OP_GEMM_BWD 3
#define FQ_OP_ACT_SCALE_GRAD 4 /* shape = {1, rows, cols}; R_max, fmts unused */
#define FQ_OP_TOPK_KL 5        /* shape, R_max, fmts unused */
size_t fq_workspace_bytes(int32_t op, fq_shape shape, int32_t R_max, int32_t fmts);

const char *fq_last_error(void);
int32_t fq_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* FQ_H */
