// Internal launchers of libfq (not part of the C ABI).
#pragma once

#include "codec.hpp"
#include "common.hpp"

namespace fq {

void launch_fill_u32(uint32_t *p, uint32_t v, long n, hipStream_t st);
// [E, rows_s, cols_s] -> [E, rows_d, cols_d], zero fill outside the source (pad) or
// crop; n_rows (device, may be NULL): only dst rows below n_rows[0] are written
void launch_reshape_u16(const uint16_t *src, int E, int rows_s, int cols_s, uint16_t *dst,
                        int rows_d, int cols_d, const int32_t *n_rows, hipStream_t st);
void launch_reshape_f32(const float *src, int E, int rows_s, int cols_s, float *dst, int rows_d,
                        int cols_d, float fill, hipStream_t st);
// out[r * n + i] = v[r] for r < rows, i < n
void launch_repeat_rows(const float *v, int rows, int n, float *out, hipStream_t st);
// out[r] = sum over i < n of in[r * n + i], in a fixed order (bitwise reproducible)
void launch_sum_rows(const float *in, int rows, int n, float *out, hipStream_t st);
void launch_quantize_stacked(const uint16_t *w, fq_shape s, const fq_weight_q &q, uint16_t *out,
                             uint8_t *codes, hipStream_t st);
void launch_observer_weight(const uint16_t *w, fq_shape s, int fmt, int group, float *scale,
                            float *zero_point, float *gscale, hipStream_t st);
void launch_observer_tensor(const uint16_t *x, size_t n, int fmt, float *scale, hipStream_t st);
// n_rows (device, may be NULL): only the first n_rows[0] of the M rows are processed
void launch_act_fq(const uint16_t *x, size_t M, int K, const int32_t *n_rows, int afmt,
                   const float *ascale, uint16_t *xq, hipStream_t st);
void launch_act_mask(uint16_t *dx, const uint16_t *x, size_t M, int K, const int32_t *n_rows,
                     int afmt, const float *ascale, hipStream_t st);
void launch_gather_actfq(const uint16_t *x, int T, int H, const int32_t *row_of, int topk,
                         int afmt, const float *ascale, uint16_t *xq, hipStream_t st);
void launch_swiglu_actfq(const uint16_t *h, int R_max, const int32_t *n_rows, int F, int afmt,
                         const float *ascale, uint16_t *a, uint16_t *aq, hipStream_t st);
// Block partials of a learnable activation scale's gradient over a
// rows x cols tensor (one float each, summed into dscale_a[0] in a fixed order).
long act_grad_partials(long rows, int cols);
// dscale_a (may be NULL): overwritten with dS_a; part: act_grad_partials floats
void launch_swiglu_bwd(const uint16_t *daq, const uint16_t *h, int R_max, const int32_t *n_rows,
                       int F, int afmt, const float *ascale, uint16_t *dh, float *dscale_a,
                       float *part, hipStream_t st);
void launch_combine(const uint16_t *o, const float *probs, const int32_t *row_of, int T, int topk,
                    int H, uint16_t *out, hipStream_t st);
void launch_combine_bwd(const uint16_t *dout, const float *probs, const int32_t *row_of, int T,
                        int topk, int H, uint16_t *dO, hipStream_t st);
void launch_unpermute_reduce(const uint16_t *dxq, const int32_t *row_of, const uint16_t *x, int T,
                             int topk, int H, int afmt, const float *ascale, uint16_t *dx,
                             float *dscale_a, float *part, hipStream_t st);

// real-quantized export: E4M3 bytes of clamp(theta, 0, 448); zero-point bytes;
// decode of stored codes + scales to bf16 (group = N*K for one scale per matrix)
void launch_export_theta(const float *theta, size_t n, uint8_t *out, hipStream_t st);
void launch_export_zp(const float *zp, size_t n, uint8_t *out, hipStream_t st);
void launch_dequantize(const uint8_t *codes, fq_shape s, int fmt, int group, const float *scale,
                       const uint8_t *scale_bytes, const uint8_t *zp_bytes, const float *gscale,
                       uint16_t *out, hipStream_t st);

// top-K KL distillation: K <= kTopKMax (the selected entries live in LDS);
// inv_n: one device float of scratch (1 / number of valid tokens)
constexpr int kTopKMax = 4096;
void launch_topk_kl(const uint16_t *student, const uint16_t *teacher, int T, int V, int K,
                    bool reverse, const uint8_t *valid, int32_t *idx, float *grad, float *loss_tok,
                    float *loss_mean, float *inv_n, hipStream_t st);

// device-data precondition checks: status = OR of FQ_BAD_* bits (cleared first)
void launch_validate(const int32_t *ids, long n_ids, int n_experts, const int32_t *seg, int E,
                     int R_max, const float *scale, long n_scale, int scale_mode,
                     const float *zero_point, const float *gscale, int n_g, const float *act_scale,
                     uint32_t *status, hipStream_t st);

size_t permute_workspace_bytes(int E, long P);
// Size of the permute scratch array the allocation-free entry point uses.
constexpr size_t kPermuteScratchBytes = size_t(4) << 20;
// Device address of that array on the current device (resolved once per device).
fq_status permute_scratch(int32_t **out);
void launch_permute(const int32_t *ids, int T, int topk, int ebegin, int E, int32_t *perm,
                    int32_t *row_of, int32_t *seg, void *ws, hipStream_t st);

// xperm / topk: routed row r of X is row xperm[r] / topk of a token-indexed
// xq (FWD's X operand, WGRAD's X operand); NULL = xq indexed by routed row.
// part: fp32 scratch of gemm_ksplit_bytes for a call small enough to split
// along the contraction; NULL = never split.
void launch_gemm_fwd(const uint16_t *xq, int R_max, const int32_t *seg, fq_shape s,
                     const uint16_t *wfq, uint16_t *y, float *part, hipStream_t st,
                     const int32_t *xperm = nullptr, int topk = 1);
void launch_gemm_dgrad(const uint16_t *dy, int R_max, const int32_t *seg, fq_shape s,
                       const uint16_t *wfq, uint16_t *dx, float *part, hipStream_t st);
// scratch bytes of the FWD (fwd) or DGRAD contraction split of a call of
// R_max routed rows on the current device (0: the call does not split)
size_t gemm_ksplit_bytes(bool fwd, fq_shape s, int R_max);
// The wgrad contraction over an expert's rows runs in chunks of at most this
// many rows, so that one hot expert cannot serialize the grid.
constexpr int kWgradChunkRows = 2048;
// chunks over all experts for at most R_max routed rows
size_t wgrad_max_chunks(int E, int R_max);
// part_s / part_z: [wgrad_max_chunks, N, K / min(group, 128)] fp32 scratch;
// chunk_start: [E+1] int scratch. dzp / part_z only for int4.
void launch_gemm_wgrad_dscale(const uint16_t *dy, const uint16_t *xq, int R_max, const int32_t *seg,
                              fq_shape s,
                              const uint16_t *w, const fq_weight_q &q, float *dscale, float *dzp,
                              float *part_s, float *part_z, int *chunk_start, hipStream_t st,
                              const int32_t *xperm = nullptr, int topk = 1);

}  // namespace fq
