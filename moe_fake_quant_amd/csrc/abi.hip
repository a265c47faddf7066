// The C ABI of libfq: argument checks, workspace carving and launches.
// Every entry point validates what the host can see before enqueuing
// anything, launches on the caller's stream and never synchronizes it.
#include <stdarg.h>
#include <stdio.h>

#include <string>

#include "internal.hpp"

namespace fq {

static thread_local std::string g_last_error;

void set_error(const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
}

fq_status hip_status(hipError_t e, const char *what) {
  set_error("%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
  return FQ_ERR_HIP;
}

namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Carver {
  char *base;
  size_t used = 0;
  explicit Carver(void *p) : base(static_cast<char *>(p)) {}
  template <class T>
  T *take(size_t bytes) {
    T *p = reinterpret_cast<T *>(base + used);
    used += align_up(bytes);
    return p;
  }
};

bool valid_weight_fmt(int f) {
  return f == FQ_FMT_INT8 || f == FQ_FMT_INT4 || f == FQ_FMT_FP8_E4M3 || f == FQ_FMT_NVFP4;
}
bool valid_act_fmt(int f) {
  return f == FQ_FMT_NONE || f == FQ_FMT_INT8 || f == FQ_FMT_FP8_E4M3 || f == FQ_FMT_NVFP4;
}

// group sizes the fused dScale epilogue reduces: 16/32/64 inside a sub-tile,
// multiples of 128 per wave (and across tiles through partials)
bool group_ok_for_dscale(int g) { return g == 16 || g == 32 || g == 64 || (g % 128 == 0); }

fq_status check_shape(fq_shape s) {
  FQ_CHECK_ARG(s.E > 0 && s.N > 0 && s.K > 0, "shape must be positive (E=%d N=%d K=%d)", s.E, s.N,
               s.K);
  FQ_CHECK_ARG((size_t)s.E * s.N * s.K < (1ull << 32), "stack too large for 32-bit indexing");
  return FQ_OK;
}

fq_status check_weight_q(const fq_weight_q *q, fq_shape s, bool need_scales) {
  FQ_CHECK_ARG(q != nullptr, "weight quantizer is NULL");
  FQ_CHECK_ARG(valid_weight_fmt(q->fmt), "unsupported weight format %d", q->fmt);
  if (q->group == FQ_GROUP_TENSOR) {
    FQ_CHECK_ARG(q->fmt == FQ_FMT_INT8 || q->fmt == FQ_FMT_FP8_E4M3,
                 "a per-tensor weight scale needs int8 or fp8 (fmt %d)", q->fmt);
    FQ_CHECK_ARG(s.K % 16 == 0, "K must be a multiple of 16 (K=%d)", s.K);
    FQ_CHECK_ARG((size_t)s.N * s.K < (1ull << 31), "matrix too large for a per-tensor scale");
    FQ_CHECK_ARG(!need_scales || q->scale != nullptr, "scale is NULL");
    return FQ_OK;
  }
  FQ_CHECK_ARG(q->group > 0 && s.K % q->group == 0, "group %d must divide K=%d", q->group, s.K);
  FQ_CHECK_ARG(q->group % 16 == 0, "group %d must be a multiple of 16", q->group);
  if (q->fmt == FQ_FMT_NVFP4) FQ_CHECK_ARG(q->group == 16, "nvfp4 blocks are 16 elements");
  if (need_scales) {
    FQ_CHECK_ARG(q->scale != nullptr, "scale is NULL");
    if (q->fmt == FQ_FMT_INT4) FQ_CHECK_ARG(q->zero_point != nullptr, "int4 needs zero_point");
    if (q->fmt == FQ_FMT_NVFP4) FQ_CHECK_ARG(q->global_scale != nullptr, "nvfp4 needs global_scale");
  }
  return FQ_OK;
}

fq_status check_act_q(const fq_act_q *aq, int K) {
  if (!aq) return FQ_OK;
  FQ_CHECK_ARG(valid_act_fmt(aq->fmt), "unsupported activation format %d", aq->fmt);
  if (aq->fmt != FQ_FMT_NONE) {
    FQ_CHECK_ARG(aq->scale != nullptr, "activation scale is NULL");
    FQ_CHECK_ARG(K % 16 == 0, "activation fake-quant needs K %% 16 == 0 (K=%d)", K);
  }
  return FQ_OK;
}

// The elementwise kernels see a per-tensor weight quantizer as one group
// spanning the whole expert matrix (scale index = expert).
fq_weight_q as_groups(const fq_weight_q &q, fq_shape s) {
  fq_weight_q g = q;
  if (q.group == FQ_GROUP_TENSOR) g.group = s.N * s.K;
  return g;
}

inline int act_fmt(const fq_act_q *aq) { return aq ? aq->fmt : FQ_FMT_NONE; }
inline hipStream_t S(fq_stream s) { return reinterpret_cast<hipStream_t>(s); }

#define FQ_TRY(x)                    \
  do {                               \
    fq_status st_ = (x);             \
    if (st_ != FQ_OK) return st_;    \
  } while (0)

// The shape the GEMM kernels run on: N a multiple of 256, K of 64 (forward)
// or 256 (backward). Other shapes (multiples of 16) run zero-padded to it.
fq_shape gemm_pad_shape(int op, fq_shape s) {
  fq_shape p = s;
  p.N = (s.N + 255) / 256 * 256;
  const int kq = op == FQ_OP_GEMM_FWD ? 64 : 256;
  p.K = (s.K + kq - 1) / kq * kq;
  return p;
}
bool gemm_needs_pad(int op, fq_shape s) {
  const fq_shape p = gemm_pad_shape(op, s);
  return p.N != s.N || p.K != s.K;
}
// a per-channel scale (group = K) spans the padded row
int padded_group(int group, fq_shape s, fq_shape p) {
  return group == s.K ? p.K : group;
}

// split_rows: with the scratch of the contraction split of a small call of
// that many routed rows (FWD, or the backward's DGRAD), which a call uses only
// when its workspace holds it; 0 = without
size_t gemm_ws_core(int op, fq_shape s, int R_max, int fmts, int split_rows) {
  int wfmt = fmts & 0xFF, afmt = (fmts >> 8) & 0xFF;
  size_t b = 0;
  if (wfmt != FQ_FMT_NONE) b += align_up((size_t)s.E * s.N * s.K * 2);
  if (afmt != FQ_FMT_NONE) b += align_up((size_t)R_max * s.K * 2);
  b += align_up(gemm_ksplit_bytes(op == FQ_OP_GEMM_FWD, s, split_rows));
  if (op == FQ_OP_GEMM_BWD) {
    // dScale partials per row chunk and 16-block (the finest group), for the
    // scale and the zero point, and the chunk prefix
    b += 2 * align_up(wgrad_max_chunks(s.E, R_max) * s.N * (s.K / 16) * 4);
    b += align_up((size_t)(s.E + 1) * 4);
    // per-tensor weight scales: the scale repeated per channel, and the
    // per-channel dScale before its sum over channels
    b += 2 * align_up((size_t)s.E * s.N * 4);
  }
  return b;
}

// Padded shapes: the call's own W_fq (if materialized), the zero-padded
// operands, outputs and scales, then the padded problem's own workspace.
size_t gemm_ws(int op, fq_shape s, int R_max, int fmts, int split_rows) {
  if (!gemm_needs_pad(op, s)) return gemm_ws_core(op, s, R_max, fmts, split_rows);
  const fq_shape p = gemm_pad_shape(op, s);
  const int wfmt = fmts & 0xFF, afmt = (fmts >> 8) & 0xFF;
  const size_t E = (size_t)s.E, Rm = (size_t)(R_max > 0 ? R_max : 0);
  size_t b = 0;
  if (wfmt != FQ_FMT_NONE) b += align_up(E * s.N * s.K * 2);   // W_fq at the call's shape
  b += align_up(E * p.N * p.K * 2);                             // padded W_fq
  b += align_up(Rm * p.K * 2);                                  // padded x
  b += align_up(Rm * p.N * 2);                                  // padded y / dy
  if (op == FQ_OP_GEMM_BWD) {
    b += align_up(E * p.N * p.K * 2);                           // padded raw w
    b += align_up(Rm * p.K * 2);                                // padded dx
    b += 4 * align_up(E * p.N * (p.K / 16) * 4);                // scale, zp, dscale, dzp
  }
  return b + gemm_ws_core(op, p, R_max, wfmt | (afmt << 8), split_rows);
}

// A learnable activation scale's gradient: only the static per-tensor formats
// have one; the block partials live in the caller's workspace.
fq_status check_dscale_a(const char *fn, const fq_act_q *aq, long rows, int cols, void *ws,
                         size_t ws_bytes) {
  FQ_CHECK_SUPPORTED(act_fmt(aq) == FQ_FMT_FP8_E4M3 || act_fmt(aq) == FQ_FMT_INT8,
                     "%s: a learnable activation scale needs fp8 or int8 activations (fmt %d)", fn,
                     act_fmt(aq));
  const size_t need = align_up((size_t)act_grad_partials(rows, cols) * sizeof(float));
  if (!ws || ws_bytes < need) {
    set_error("%s: workspace %zu bytes < %zu needed", fn, ws_bytes, need);
    return FQ_ERR_WORKSPACE_TOO_SMALL;
  }
  return FQ_OK;
}

}  // namespace
}  // namespace fq

using namespace fq;

extern "C" {

int32_t fq_abi_version(void) { return FQ_ABI_VERSION; }

const char *fq_last_error(void) { return g_last_error.c_str(); }

size_t fq_workspace_bytes(int32_t op, fq_shape shape, int32_t R_max, int32_t fmts) {
  if (op == FQ_OP_PERMUTE) return permute_workspace_bytes(shape.E > 0 ? shape.E : 1, R_max);
  if (op == FQ_OP_GEMM_FWD || op == FQ_OP_GEMM_BWD) return gemm_ws(op, shape, R_max, fmts, R_max);
  if (op == FQ_OP_TOPK_KL) return kAlign;
  if (op == FQ_OP_ACT_SCALE_GRAD) {
    if (shape.N < 0 || shape.K <= 0) return 0;
    return align_up((size_t)act_grad_partials(shape.N, shape.K) * sizeof(float));
  }
  return 0;
}

fq_status observer_absmax_init(const uint16_t *x, fq_shape s, int32_t fmt, int32_t group,
                               int32_t per_tensor, float *scale, float *zero_point,
                               float *global_scale, void *ws, size_t ws_bytes, fq_stream stream) {
  (void)ws;
  (void)ws_bytes;
  FQ_TRY(check_shape(s));
  FQ_CHECK_ARG(x && scale, "x and scale must be non-NULL");
  FQ_CHECK_ARG(aligned16(x), "x must be 16-byte aligned");
  FQ_CHECK_ARG(s.K % 8 == 0, "K must be a multiple of 8 (K=%d)", s.K);
  if (per_tensor) {
    FQ_CHECK_ARG(fmt == FQ_FMT_INT8 || fmt == FQ_FMT_FP8_E4M3 || fmt == FQ_FMT_NVFP4,
                 "unsupported activation format %d", fmt);
    launch_observer_tensor(x, (size_t)s.E * s.N * s.K, fmt, scale, S(stream));
    FQ_CHECK_LAUNCH("observer_absmax_init");
    return FQ_OK;
  }
  fq_weight_q q{fmt, group, scale, zero_point, global_scale};
  FQ_TRY(check_weight_q(&q, s, true));
  launch_observer_weight(x, s, fmt, as_groups(q, s).group, scale, zero_point, global_scale,
                         S(stream));
  FQ_CHECK_LAUNCH("observer_absmax_init");
  return FQ_OK;
}

fq_status fq_quantize_stacked(const uint16_t *w, fq_shape s, const fq_weight_q *q, uint16_t *w_fq,
                              uint8_t *codes, fq_stream stream) {
  FQ_TRY(check_shape(s));
  FQ_TRY(check_weight_q(q, s, true));
  FQ_CHECK_ARG(w != nullptr, "w is NULL");
  FQ_CHECK_ARG(w_fq || codes, "at least one of w_fq and codes must be non-NULL");
  FQ_CHECK_ARG(aligned16(w) && (!w_fq || aligned16(w_fq)), "bf16 tensors must be 16-byte aligned");
  FQ_CHECK_ARG(!codes || ((uintptr_t)codes & 7) == 0, "codes must be 8-byte aligned");
  launch_quantize_stacked(w, s, as_groups(*q, s), w_fq, codes, S(stream));
  FQ_CHECK_LAUNCH("fq_quantize_stacked");
  return FQ_OK;
}

fq_status fq_export_scales(fq_shape s, const fq_weight_q *q, uint8_t *scale_bytes,
                           uint8_t *zero_point_bytes, fq_stream stream) {
  FQ_TRY(check_shape(s));
  FQ_TRY(check_weight_q(q, s, true));
  FQ_CHECK_ARG(q->fmt == FQ_FMT_NVFP4 || q->fmt == FQ_FMT_INT4,
               "only nvfp4 (block scale bytes) and int4 (zero-point bytes) have parameters to "
               "convert (fmt %d)", q->fmt);
  const size_t ng = (size_t)s.E * s.N * (s.K / q->group);
  if (q->fmt == FQ_FMT_NVFP4) {
    FQ_CHECK_ARG(scale_bytes != nullptr, "scale_bytes is NULL");
    FQ_CHECK_ARG(aligned16(q->scale) && ((uintptr_t)scale_bytes & 3) == 0,
                 "theta must be 16-byte and scale_bytes 4-byte aligned");
    launch_export_theta(q->scale, ng, scale_bytes, S(stream));
  } else {
    FQ_CHECK_ARG(zero_point_bytes != nullptr, "zero_point_bytes is NULL");
    launch_export_zp(q->zero_point, ng, zero_point_bytes, S(stream));
  }
  FQ_CHECK_LAUNCH("fq_export_scales");
  return FQ_OK;
}

fq_status fq_dequantize_stacked(const uint8_t *codes, fq_shape s, int32_t fmt, int32_t group,
                                const float *scale, const uint8_t *scale_bytes,
                                const uint8_t *zero_point_bytes, const float *global_scale,
                                uint16_t *w_bf16, fq_stream stream) {
  FQ_TRY(check_shape(s));
  FQ_CHECK_ARG(codes && w_bf16, "codes and w_bf16 must be non-NULL");
  FQ_CHECK_ARG(s.K % 16 == 0, "K must be a multiple of 16 (K=%d)", s.K);
  FQ_CHECK_ARG(((uintptr_t)codes & 7) == 0 && aligned16(w_bf16),
               "codes must be 8-byte and w_bf16 16-byte aligned");
  FQ_CHECK_ARG(valid_weight_fmt(fmt), "unsupported weight format %d", fmt);
  int g = group;
  if (fmt == FQ_FMT_NVFP4) {
    FQ_CHECK_ARG(group == 16, "nvfp4 blocks are 16 elements");
    FQ_CHECK_ARG(scale_bytes && global_scale, "nvfp4 needs scale_bytes and global_scale");
  } else if (group == FQ_GROUP_TENSOR) {
    FQ_CHECK_ARG(fmt == FQ_FMT_INT8 || fmt == FQ_FMT_FP8_E4M3,
                 "a per-tensor weight scale needs int8 or fp8 (fmt %d)", fmt);
    FQ_CHECK_ARG((size_t)s.N * s.K < (1ull << 31), "matrix too large for a per-tensor scale");
    FQ_CHECK_ARG(scale != nullptr, "scale is NULL");
    g = s.N * s.K;
  } else {
    FQ_CHECK_ARG(group > 0 && s.K % group == 0 && group % 16 == 0,
                 "group %d must divide K=%d and be a multiple of 16", group, s.K);
    FQ_CHECK_ARG(scale != nullptr, "scale is NULL");
    FQ_CHECK_ARG(fmt != FQ_FMT_INT4 || zero_point_bytes, "int4 needs zero_point_bytes");
  }
  launch_dequantize(codes, s, fmt, g, scale, scale_bytes, zero_point_bytes, global_scale, w_bf16,
                    S(stream));
  FQ_CHECK_LAUNCH("fq_dequantize_stacked");
  return FQ_OK;
}

fq_status fq_topk_kl(const uint16_t *student, const uint16_t *teacher, int32_t T, int32_t V,
                     int32_t K, int32_t reverse, const uint8_t *valid, int32_t *topk_idx,
                     float *grad, float *loss_tok, float *loss_mean, void *ws, size_t ws_bytes,
                     fq_stream stream) {
  FQ_CHECK_ARG(T >= 0 && V > 0 && V % 8 == 0, "bad sizes T=%d V=%d (V must be a multiple of 8)",
               T, V);
  FQ_CHECK_ARG(K >= 1 && K <= V, "K=%d must be in [1, V]", K);
  FQ_CHECK_SUPPORTED(K <= kTopKMax, "K=%d above the supported %d", K, kTopKMax);
  FQ_CHECK_ARG(loss_mean != nullptr, "loss_mean is NULL");
  FQ_CHECK_ARG(T == 0 || (student && teacher && topk_idx && grad && loss_tok), "NULL pointer");
  FQ_CHECK_ARG((!student || aligned16(student)) && (!teacher || aligned16(teacher)),
               "logits must be 16-byte aligned");
  if (!ws || ws_bytes < kAlign) {
    set_error("fq_topk_kl: workspace %zu bytes < %zu needed", ws_bytes, (size_t)kAlign);
    return FQ_ERR_WORKSPACE_TOO_SMALL;
  }
  launch_topk_kl(student, teacher, T, V, K, reverse != 0, valid, topk_idx, grad, loss_tok,
                 loss_mean, static_cast<float *>(ws), S(stream));
  FQ_CHECK_LAUNCH("fq_topk_kl");
  return FQ_OK;
}

fq_status fq_moe_permute(const int32_t *ids, int32_t T, int32_t topk, int32_t ebegin, int32_t E,
                         int32_t *perm, int32_t *row_of, int32_t *seg, void *ws, size_t ws_bytes,
                         fq_stream stream) {
  FQ_CHECK_ARG(T >= 0 && topk > 0 && E > 0 && ebegin >= 0, "bad sizes T=%d topk=%d E=%d", T, topk, E);
  FQ_CHECK_ARG(seg != nullptr, "seg_offsets is NULL");
  FQ_CHECK_ARG(T == 0 || (ids && perm && row_of), "expert_ids, perm and row_of must be non-NULL");
  FQ_CHECK_ARG((long)T * topk < (1l << 31), "too many pairs");
  size_t need = permute_workspace_bytes(E, (long)T * topk);
  if (ws_bytes < need || !ws) {
    set_error("fq_moe_permute: workspace %zu bytes < %zu needed", ws_bytes, need);
    return FQ_ERR_WORKSPACE_TOO_SMALL;
  }
  launch_permute(ids, T, topk, ebegin, E, perm, row_of, seg, ws, S(stream));
  FQ_CHECK_LAUNCH("fq_moe_permute");
  return FQ_OK;
}

fq_status fq_validate(const int32_t *ids, int32_t T, int32_t topk, int32_t n_experts,
                      const int32_t *seg, int32_t E, int32_t R_max, fq_shape s,
                      const fq_weight_q *wq, const fq_act_q *aq, uint32_t *status,
                      fq_stream stream) {
  FQ_CHECK_ARG(status != nullptr, "status is NULL");
  if (ids) FQ_CHECK_ARG(T >= 0 && topk > 0 && n_experts > 0, "bad routing sizes T=%d topk=%d n=%d",
                        T, topk, n_experts);
  if (seg) FQ_CHECK_ARG(E > 0 && R_max >= 0, "bad segment sizes E=%d R_max=%d", E, R_max);
  long n_scale = 0;
  int scale_mode = 0;
  if (wq) {
    FQ_TRY(check_shape(s));
    FQ_TRY(check_weight_q(wq, s, true));
    n_scale = wq->group == FQ_GROUP_TENSOR ? (long)s.E : (long)s.E * s.N * (s.K / wq->group);
    scale_mode = wq->fmt == FQ_FMT_NVFP4 ? 1 : 0;
  }
  const bool act = aq && aq->fmt != FQ_FMT_NONE;
  if (act) FQ_TRY(check_act_q(aq, 16));
  launch_validate(ids, ids ? (long)T * topk : 0, n_experts, seg, E, R_max,
                  wq ? wq->scale : nullptr, n_scale, scale_mode,
                  wq && wq->fmt == FQ_FMT_INT4 ? wq->zero_point : nullptr,
                  wq && wq->fmt == FQ_FMT_NVFP4 ? wq->global_scale : nullptr, wq ? s.E : 0,
                  act ? aq->scale : nullptr, status, S(stream));
  FQ_CHECK_LAUNCH("fq_validate");
  return FQ_OK;
}

fq_status fq_moe_permute_noalloc(const int32_t *ids, int32_t T, int32_t topk, int32_t ebegin,
                                 int32_t E, int32_t *perm, int32_t *row_of, int32_t *seg,
                                 fq_stream stream) {
  FQ_CHECK_ARG(T >= 0 && topk > 0 && E > 0 && ebegin >= 0, "bad sizes T=%d topk=%d E=%d", T, topk, E);
  FQ_CHECK_ARG(seg != nullptr, "seg_offsets is NULL");
  FQ_CHECK_ARG(T == 0 || (ids && perm && row_of), "expert_ids, perm and row_of must be non-NULL");
  FQ_CHECK_ARG((long)T * topk < (1l << 31), "too many pairs");
  size_t need = permute_workspace_bytes(E, (long)T * topk);
  if (need > kPermuteScratchBytes) {
    set_error("fq_moe_permute_noalloc: E_local=%d and T*topk=%ld need %zu bytes of scratch, the "
              "static scratch holds %zu (use fq_moe_permute with a workspace)",
              E, (long)T * topk, need, kPermuteScratchBytes);
    return FQ_ERR_WORKSPACE_TOO_SMALL;
  }
  int32_t *scr = nullptr;
  FQ_TRY(permute_scratch(&scr));
  launch_permute(ids, T, topk, ebegin, E, perm, row_of, seg, scr, S(stream));
  FQ_CHECK_LAUNCH("fq_moe_permute_noalloc");
  return FQ_OK;
}

namespace {

// The forward on a shape the kernels take (N % 256 == 0, K % 64 == 0);
// arguments already checked, workspace large enough.
void gemm_fwd_core(const uint16_t *x, int R_max, const int32_t *seg, fq_shape s, const uint16_t *w,
                   const uint16_t *w_fq, const fq_weight_q *wq, const fq_act_q *aq, uint16_t *y,
                   void *ws, bool split, hipStream_t st, const int32_t *xperm, int topk) {
  const int afmt = act_fmt(aq);
  Carver c(ws);
  const uint16_t *wfq = w_fq;
  if (!wfq) {
    uint16_t *t = c.take<uint16_t>((size_t)s.E * s.N * s.K * 2);
    launch_quantize_stacked(w, s, as_groups(*wq, s), t, nullptr, st);
    wfq = t;
  }
  const uint16_t *xq = x;
  if (afmt != FQ_FMT_NONE && R_max > 0) {
    uint16_t *t = c.take<uint16_t>((size_t)R_max * s.K * 2);
    launch_act_fq(x, R_max, s.K, seg + s.E, afmt, aq->scale, t, st);
    xq = t;
  }
  const size_t part_bytes = split ? gemm_ksplit_bytes(true, s, R_max) : 0;
  float *part = part_bytes ? c.take<float>(part_bytes) : nullptr;
  launch_gemm_fwd(xq, R_max, seg, s, wfq, y, part, st, xperm, topk);
}

// fq_grouped_gemm_fwd and its routed-X form: x has x_rows rows; with xperm
// routed row r reads row xperm[r] / topk of x (then aq is NULL)
fq_status gemm_fwd_call(const char *fn, const uint16_t *x, int32_t x_rows, const int32_t *xperm,
                        int32_t topk, int32_t R_max, const int32_t *seg, fq_shape s,
                        const uint16_t *w, const uint16_t *w_fq, const fq_weight_q *wq,
                        const fq_act_q *aq, uint16_t *y, void *ws, size_t ws_bytes,
                        fq_stream stream) {
  FQ_TRY(check_shape(s));
  FQ_CHECK_ARG(R_max >= 0, "R_max < 0");
  FQ_CHECK_ARG(seg && y && (x || R_max == 0), "x, seg_offsets and y must be non-NULL");
  FQ_CHECK_ARG(w || w_fq, "w or w_fq must be non-NULL");
  FQ_CHECK_ARG(wq || w_fq, "wq may be NULL only with w_fq (weights used as given)");
  if (wq) FQ_TRY(check_weight_q(wq, s, w_fq == nullptr));
  FQ_TRY(check_act_q(aq, s.K));
  FQ_CHECK_SUPPORTED(s.N % 16 == 0 && s.K % 16 == 0,
                     "grouped GEMM needs N %% 16 == 0 and K %% 16 == 0 (N=%d K=%d)", s.N, s.K);
  FQ_CHECK_SUPPORTED(s.E <= 1024, "grouped GEMM supports up to 1024 experts per stack (E=%d)", s.E);
  const fq_shape p = gemm_pad_shape(FQ_OP_GEMM_FWD, s);
  const int32_t rows_ws = x_rows > R_max ? x_rows : R_max;
  FQ_CHECK_SUPPORTED((size_t)rows_ws * p.K * 2 < (1ull << 32) && (size_t)p.N * p.K * 2 < (1ull << 32),
                     "operands must stay below 4 GiB (32-bit tile offsets)");
  FQ_CHECK_ARG((!x || aligned16(x)) && aligned16(y) && (!w || aligned16(w)) &&
                   (!w_fq || aligned16(w_fq)),
               "bf16 tensors must be 16-byte aligned");
  const int afmt = act_fmt(aq);
  const int fmts = (w_fq ? 0 : wq->fmt) | (afmt << 8);
  const size_t need = gemm_ws(FQ_OP_GEMM_FWD, s, rows_ws, fmts, R_max);
  const size_t need_min = gemm_ws(FQ_OP_GEMM_FWD, s, rows_ws, fmts, 0);
  if (need_min > 0 && (ws_bytes < need_min || !ws)) {
    set_error("%s: workspace %zu bytes < %zu needed", fn, ws_bytes, need);
    return FQ_ERR_WORKSPACE_TOO_SMALL;
  }
  const bool split = ws && ws_bytes >= need;
  hipStream_t st = S(stream);
  if (!gemm_needs_pad(FQ_OP_GEMM_FWD, s)) {
    gemm_fwd_core(x, R_max, seg, s, w, w_fq, wq, aq, y, ws, split, st, xperm, topk);
    FQ_CHECK_LAUNCH(fn);
    return FQ_OK;
  }
  // zero-padded to the kernels' shape: padded K columns add nothing, padded
  // N rows give outputs that are not copied back
  Carver c(ws);
  const uint16_t *wfq = w_fq;
  if (!wfq) {
    uint16_t *t = c.take<uint16_t>((size_t)s.E * s.N * s.K * 2);
    launch_quantize_stacked(w, s, as_groups(*wq, s), t, nullptr, st);
    wfq = t;
  }
  uint16_t *wfq_p = c.take<uint16_t>((size_t)s.E * p.N * p.K * 2);
  launch_reshape_u16(wfq, s.E, s.N, s.K, wfq_p, p.N, p.K, nullptr, st);
  uint16_t *x_p = c.take<uint16_t>((size_t)x_rows * p.K * 2);
  uint16_t *y_p = c.take<uint16_t>((size_t)R_max * p.N * 2);
  // routed X: every token row is copied (rows are not in segment order)
  if (x_rows > 0)
    launch_reshape_u16(x, 1, x_rows, s.K, x_p, x_rows, p.K, xperm ? nullptr : seg + s.E, st);
  gemm_fwd_core(x_p, R_max, seg, p, nullptr, wfq_p, nullptr, aq, y_p, c.base + c.used, split, st,
                xperm, topk);
  if (R_max > 0) launch_reshape_u16(y_p, 1, R_max, p.N, y, R_max, s.N, seg + s.E, st);
  FQ_CHECK_LAUNCH(fn);
  return FQ_OK;
}

}  // namespace

fq_status fq_grouped_gemm_fwd(const uint16_t *x, int32_t R_max, const int32_t *seg, fq_shape s,
                              const uint16_t *w, const uint16_t *w_fq, const fq_weight_q *wq,
                              const fq_act_q *aq, uint16_t *y, void *ws, size_t ws_bytes,
                              fq_stream stream) {
  return gemm_fwd_call("fq_grouped_gemm_fwd", x, R_max, nullptr, 1, R_max, seg, s, w, w_fq, wq, aq,
                       y, ws, ws_bytes, stream);
}

fq_status fq_grouped_gemm_fwd_tokens(const uint16_t *x_tok, int32_t T, const int32_t *perm,
                                     int32_t topk, int32_t R_max, const int32_t *seg, fq_shape s,
                                     const uint16_t *w, const uint16_t *w_fq,
                                     const fq_weight_q *wq, uint16_t *y, void *ws, size_t ws_bytes,
                                     fq_stream stream) {
  FQ_CHECK_ARG(T >= 0 && topk > 0, "bad sizes (T=%d topk=%d)", T, topk);
  FQ_CHECK_ARG(R_max == 0 || (perm && x_tok), "perm and x_tok must be non-NULL");
  return gemm_fwd_call("fq_grouped_gemm_fwd_tokens", x_tok, T, perm, topk, R_max, seg, s, w, w_fq,
                       wq, nullptr, y, ws, ws_bytes, stream);
}

namespace {

// The backward on a shape the kernels take (N % 256 == 0, K % 256 == 0);
// arguments already checked, workspace large enough.
void gemm_bwd_core(const uint16_t *dy, const uint16_t *x, int R_max, const int32_t *seg, fq_shape s,
                   const uint16_t *w, const uint16_t *w_fq, const fq_weight_q *wq,
                   const fq_act_q *aq, uint16_t *dx, float *dscale, float *dzp, void *ws,
                   bool split, hipStream_t st, const int32_t *xperm, int topk) {
  const bool want_ds = dscale || dzp;
  const bool per_tensor = wq->group == FQ_GROUP_TENSOR;
  const int afmt = act_fmt(aq);
  Carver c(ws);
  const uint16_t *wfq = w_fq;
  if (!wfq && dx) {
    uint16_t *t = c.take<uint16_t>((size_t)s.E * s.N * s.K * 2);
    launch_quantize_stacked(w, s, as_groups(*wq, s), t, nullptr, st);
    wfq = t;
  }
  if (dx && R_max > 0) {
    const size_t part_bytes = split ? gemm_ksplit_bytes(false, s, R_max) : 0;
    float *part = part_bytes ? c.take<float>(part_bytes) : nullptr;
    launch_gemm_dgrad(dy, R_max, seg, s, wfq, dx, part, st);
    if (afmt != FQ_FMT_NONE) launch_act_mask(dx, x, R_max, s.K, seg + s.E, afmt, aq->scale, st);
  }
  if (want_ds) {
    const uint16_t *xq = x;
    if (afmt != FQ_FMT_NONE && R_max > 0) {
      uint16_t *t = c.take<uint16_t>((size_t)R_max * s.K * 2);
      launch_act_fq(x, R_max, s.K, seg + s.E, afmt, aq->scale, t, st);
      xq = t;
    }
    const size_t part = wgrad_max_chunks(s.E, R_max) * s.N * (s.K / 16) * 4;
    float *ps = c.take<float>(part);
    float *pz = c.take<float>(part);
    int *cs = c.take<int>((size_t)(s.E + 1) * 4);
    if (per_tensor) {
      // per channel over the repeated scale, then the fixed-order sum over channels
      float *rep = c.take<float>((size_t)s.E * s.N * 4);
      float *dch = c.take<float>((size_t)s.E * s.N * 4);
      launch_repeat_rows(wq->scale, s.E, s.N, rep, st);
      fq_weight_q qc{wq->fmt, s.K, rep, nullptr, nullptr};
      launch_gemm_wgrad_dscale(dy, xq, R_max, seg, s, w, qc, dch, nullptr, ps, nullptr, cs, st,
                               xperm, topk);
      launch_sum_rows(dch, s.E, s.N, dscale, st);
    } else {
      launch_gemm_wgrad_dscale(dy, xq, R_max, seg, s, w, *wq, dscale, dzp, ps, dzp ? pz : nullptr, cs,
                               st, xperm, topk);
    }
  }
}

}  // namespace

namespace {

// fq_grouped_gemm_bwd_scale and its routed-X form (see gemm_fwd_call; with
// xperm, aq and dx are NULL)
fq_status gemm_bwd_call(const char *fn, const uint16_t *dy, const uint16_t *x, int32_t x_rows,
                        const int32_t *xperm, int32_t topk, int32_t R_max, const int32_t *seg,
                        fq_shape s, const uint16_t *w, const uint16_t *w_fq, const fq_weight_q *wq,
                        const fq_act_q *aq, uint16_t *dx, float *dscale, float *dzp, void *ws,
                        size_t ws_bytes, fq_stream stream) {
  FQ_TRY(check_shape(s));
  FQ_CHECK_ARG(R_max >= 0, "R_max < 0");
  FQ_CHECK_ARG(seg != nullptr, "seg_offsets is NULL");
  FQ_CHECK_ARG(dy || R_max == 0, "dy is NULL");
  const bool want_ds = dscale || dzp;
  FQ_TRY(check_weight_q(wq, s, true));
  FQ_TRY(check_act_q(aq, s.K));
  FQ_CHECK_ARG(w != nullptr, "w (raw weights) is NULL");
  FQ_CHECK_ARG(!want_ds || x || R_max == 0, "x is NULL");
  FQ_CHECK_ARG(!dzp || wq->fmt == FQ_FMT_INT4, "dzero_point only exists for int4");
  FQ_CHECK_ARG(!dzp || dscale, "dzero_point needs dscale too");
  FQ_CHECK_SUPPORTED(s.N % 16 == 0 && s.K % 16 == 0,
                     "grouped GEMM needs N %% 16 == 0 and K %% 16 == 0 (N=%d K=%d)", s.N, s.K);
  FQ_CHECK_SUPPORTED(s.E <= 1024, "grouped GEMM supports up to 1024 experts per stack (E=%d)", s.E);
  const fq_shape p = gemm_pad_shape(FQ_OP_GEMM_BWD, s);
  const int32_t rows_ws = x_rows > R_max ? x_rows : R_max;
  FQ_CHECK_SUPPORTED((size_t)rows_ws * (p.K > p.N ? p.K : p.N) * 2 < (1ull << 32) &&
                         (size_t)p.N * p.K * 2 < (1ull << 32),
                     "operands must stay below 4 GiB (32-bit tile offsets)");
  const bool per_tensor = wq->group == FQ_GROUP_TENSOR;
  const int group_p = per_tensor ? FQ_GROUP_TENSOR : padded_group(wq->group, s, p);
  FQ_CHECK_SUPPORTED(!want_ds || per_tensor || group_ok_for_dscale(group_p),
                     "dScale needs group 16, 32, 64 or a multiple of 128 (group=%d)", wq->group);
  FQ_CHECK_ARG(!want_ds || wq->fmt != FQ_FMT_NVFP4 || aligned16(wq->scale),
               "nvfp4 theta must be 16-byte aligned");
  FQ_CHECK_ARG((!dy || aligned16(dy)) && (!x || aligned16(x)) && aligned16(w) &&
                   (!w_fq || aligned16(w_fq)) && (!dx || aligned16(dx)),
               "bf16 tensors must be 16-byte aligned");
  const int afmt = act_fmt(aq);
  // FQ_w(W) is materialized only for dX
  const int fmts = ((w_fq || !dx) ? 0 : wq->fmt) | (afmt << 8);
  const size_t need = gemm_ws(FQ_OP_GEMM_BWD, s, rows_ws, fmts, dx ? R_max : 0);
  const size_t need_min = gemm_ws(FQ_OP_GEMM_BWD, s, rows_ws, fmts, 0);
  if (ws_bytes < need_min || !ws) {
    set_error("%s: workspace %zu bytes < %zu needed", fn, ws_bytes, need);
    return FQ_ERR_WORKSPACE_TOO_SMALL;
  }
  const bool split = ws_bytes >= need;
  hipStream_t st = S(stream);
  if (!gemm_needs_pad(FQ_OP_GEMM_BWD, s)) {
    gemm_bwd_core(dy, x, R_max, seg, s, w, w_fq, wq, aq, dx, dscale, dzp, ws, split, st, xperm,
                  topk);
    FQ_CHECK_LAUNCH(fn);
    return FQ_OK;
  }
  // Zero-padded to the kernels' shape. A padded weight element is 0 with a
  // neutral scale (1 for the integer / FP8 grids, theta 0 for NVFP4, zero
  // point 0), so its straight-through factor is 0; padded contraction
  // columns add nothing; only the call's own region is copied back.
  Carver c(ws);
  const int G = per_tensor ? 0 : s.K / wq->group, Gp = per_tensor ? 0 : p.K / group_p;
  uint16_t *wfq_p = nullptr;
  if (dx) {
    const uint16_t *wfq = w_fq;
    if (!wfq) {
      uint16_t *t = c.take<uint16_t>((size_t)s.E * s.N * s.K * 2);
      launch_quantize_stacked(w, s, as_groups(*wq, s), t, nullptr, st);
      wfq = t;
    }
    wfq_p = c.take<uint16_t>((size_t)s.E * p.N * p.K * 2);
    launch_reshape_u16(wfq, s.E, s.N, s.K, wfq_p, p.N, p.K, nullptr, st);
  }
  uint16_t *w_p = c.take<uint16_t>((size_t)s.E * p.N * p.K * 2);
  launch_reshape_u16(w, s.E, s.N, s.K, w_p, p.N, p.K, nullptr, st);
  uint16_t *x_p = c.take<uint16_t>((size_t)x_rows * p.K * 2);
  uint16_t *dy_p = c.take<uint16_t>((size_t)R_max * p.N * 2);
  uint16_t *dx_p = c.take<uint16_t>((size_t)R_max * p.K * 2);
  if (x && x_rows > 0)
    launch_reshape_u16(x, 1, x_rows, s.K, x_p, x_rows, p.K, xperm ? nullptr : seg + s.E, st);
  if (R_max > 0) launch_reshape_u16(dy, 1, R_max, s.N, dy_p, R_max, p.N, seg + s.E, st);
  const size_t nsc = (size_t)s.E * p.N * (p.K / 16) * 4;
  float *sc_p = c.take<float>(nsc), *zp_p = c.take<float>(nsc);
  float *ds_p = c.take<float>(nsc), *dzp_p = c.take<float>(nsc);
  fq_weight_q wq_p = *wq;
  wq_p.group = group_p;
  if (!per_tensor) {
    launch_reshape_f32(wq->scale, s.E, s.N, G, sc_p, p.N, Gp,
                       wq->fmt == FQ_FMT_NVFP4 ? 0.0f : 1.0f, st);
    wq_p.scale = sc_p;
    if (wq->fmt == FQ_FMT_INT4) {
      launch_reshape_f32(wq->zero_point, s.E, s.N, G, zp_p, p.N, Gp, 0.0f, st);
      wq_p.zero_point = zp_p;
    }
  }
  // per-tensor dScale is [E] already, written in place
  float *ds_out = dscale ? (per_tensor ? dscale : ds_p) : nullptr;
  float *dzp_out = dzp ? dzp_p : nullptr;
  gemm_bwd_core(dy_p, x ? x_p : nullptr, R_max, seg, p, w_p, wfq_p, &wq_p, aq,
                dx ? dx_p : nullptr, ds_out, dzp_out, c.base + c.used, split, st, xperm, topk);
  if (dx && R_max > 0) launch_reshape_u16(dx_p, 1, R_max, p.K, dx, R_max, s.K, seg + s.E, st);
  if (dscale && !per_tensor) launch_reshape_f32(ds_p, s.E, p.N, Gp, dscale, s.N, G, 0.0f, st);
  if (dzp) launch_reshape_f32(dzp_p, s.E, p.N, Gp, dzp, s.N, G, 0.0f, st);
  FQ_CHECK_LAUNCH(fn);
  return FQ_OK;
}

}  // namespace

fq_status fq_grouped_gemm_bwd_scale(const uint16_t *dy, const uint16_t *x, int32_t R_max,
                                    const int32_t *seg, fq_shape s, const uint16_t *w,
                                    const uint16_t *w_fq, const fq_weight_q *wq, const fq_act_q *aq,
                                    uint16_t *dx, float *dscale, float *dzp, void *ws,
                                    size_t ws_bytes, fq_stream stream) {
  return gemm_bwd_call("fq_grouped_gemm_bwd_scale", dy, x, R_max, nullptr, 1, R_max, seg, s, w, w_fq,
                       wq, aq, dx, dscale, dzp, ws, ws_bytes, stream);
}

fq_status fq_grouped_gemm_wgrad_tokens(const uint16_t *dy, const uint16_t *x_tok, int32_t T,
                                       const int32_t *perm, int32_t topk, int32_t R_max,
                                       const int32_t *seg, fq_shape s, const uint16_t *w,
                                       const fq_weight_q *wq, float *dscale, float *dzp, void *ws,
                                       size_t ws_bytes, fq_stream stream) {
  FQ_CHECK_ARG(T >= 0 && topk > 0, "bad sizes (T=%d topk=%d)", T, topk);
  FQ_CHECK_ARG(R_max == 0 || (perm && x_tok), "perm and x_tok must be non-NULL");
  return gemm_bwd_call("fq_grouped_gemm_wgrad_tokens", dy, x_tok, T, perm, topk, R_max, seg, s, w,
                       nullptr, wq, nullptr, nullptr, dscale, dzp, ws, ws_bytes, stream);
}

fq_status fq_actfq(const uint16_t *x, int32_t rows, int32_t K, const fq_act_q *aq, uint16_t *xq,
                   fq_stream stream) {
  FQ_CHECK_ARG(rows >= 0 && K > 0 && K % 16 == 0, "bad sizes (rows=%d K=%d; K %% 16 == 0)", rows, K);
  FQ_CHECK_ARG(rows == 0 || (x && xq), "NULL pointer");
  FQ_CHECK_ARG((!x || aligned16(x)) && (!xq || aligned16(xq)), "bf16 tensors must be 16-byte aligned");
  FQ_CHECK_ARG((long)rows * K < (1l << 35), "too many elements");
  FQ_TRY(check_act_q(aq, K));
  launch_act_fq(x, (size_t)rows, K, nullptr, act_fmt(aq), aq ? aq->scale : nullptr, xq, S(stream));
  FQ_CHECK_LAUNCH("fq_actfq");
  return FQ_OK;
}

fq_status fq_moe_gather_actfq(const uint16_t *x, int32_t T, int32_t H, const int32_t *row_of,
                              int32_t topk, const fq_act_q *aq, uint16_t *xq, fq_stream stream) {
  FQ_CHECK_ARG(T >= 0 && H > 0 && topk > 0, "bad sizes");
  FQ_CHECK_ARG(H % 16 == 0, "H must be a multiple of 16");
  FQ_CHECK_ARG(T == 0 || (x && row_of && xq), "NULL pointer");
  FQ_CHECK_ARG((!x || aligned16(x)) && (!xq || aligned16(xq)), "bf16 tensors must be 16-byte aligned");
  FQ_CHECK_ARG((long)T * H < (1l << 35), "too many elements");
  FQ_TRY(check_act_q(aq, H));
  launch_gather_actfq(x, T, H, row_of, topk, act_fmt(aq), aq ? aq->scale : nullptr, xq, S(stream));
  FQ_CHECK_LAUNCH("fq_moe_gather_actfq");
  return FQ_OK;
}

fq_status fq_swiglu_actfq(const uint16_t *h, int32_t R_max, const int32_t *n_rows, int32_t F,
                          const fq_act_q *aq, uint16_t *a, uint16_t *aqo, fq_stream stream) {
  FQ_CHECK_ARG(R_max >= 0 && F > 0 && F % 16 == 0, "bad sizes (F must be a multiple of 16)");
  FQ_CHECK_ARG((long)R_max * F < (1l << 35), "too many elements");
  FQ_CHECK_ARG(n_rows && (R_max == 0 || (h && aqo)), "NULL pointer");
  FQ_CHECK_ARG((!h || aligned16(h)) && (!a || aligned16(a)) && (!aqo || aligned16(aqo)),
               "bf16 tensors must be 16-byte aligned");
  FQ_TRY(check_act_q(aq, F));
  launch_swiglu_actfq(h, R_max, n_rows, F, act_fmt(aq), aq ? aq->scale : nullptr, a, aqo, S(stream));
  FQ_CHECK_LAUNCH("fq_swiglu_actfq");
  return FQ_OK;
}

fq_status fq_swiglu_bwd(const uint16_t *daq, const uint16_t *h, int32_t R_max, const int32_t *n_rows,
                        int32_t F, const fq_act_q *aq, uint16_t *dh, float *dscale_a, void *ws,
                        size_t ws_bytes, fq_stream stream) {
  FQ_CHECK_ARG(R_max >= 0 && F > 0 && F % 16 == 0, "bad sizes (F must be a multiple of 16)");
  FQ_CHECK_ARG((long)R_max * F < (1l << 35), "too many elements");
  FQ_CHECK_ARG(n_rows && (R_max == 0 || (h && daq && dh)), "NULL pointer");
  FQ_CHECK_ARG((!h || aligned16(h)) && (!daq || aligned16(daq)) && (!dh || aligned16(dh)),
               "bf16 tensors must be 16-byte aligned");
  FQ_TRY(check_act_q(aq, F));
  if (dscale_a) FQ_TRY(check_dscale_a("fq_swiglu_bwd", aq, R_max, F, ws, ws_bytes));
  launch_swiglu_bwd(daq, h, R_max, n_rows, F, act_fmt(aq), aq ? aq->scale : nullptr, dh, dscale_a,
                    static_cast<float *>(ws), S(stream));
  FQ_CHECK_LAUNCH("fq_swiglu_bwd");
  return FQ_OK;
}

fq_status fq_moe_combine(const uint16_t *o, const float *probs, const int32_t *row_of, int32_t T,
                         int32_t topk, int32_t H, uint16_t *out, fq_stream stream) {
  FQ_CHECK_ARG(T >= 0 && topk > 0 && H > 0 && H % 16 == 0, "bad sizes (H must be a multiple of 16)");
  FQ_CHECK_ARG((long)T * H < (1l << 35), "too many elements");
  FQ_CHECK_ARG(T == 0 || (o && probs && row_of && out), "NULL pointer");
  FQ_CHECK_ARG((!o || aligned16(o)) && (!out || aligned16(out)), "bf16 tensors must be 16-byte aligned");
  launch_combine(o, probs, row_of, T, topk, H, out, S(stream));
  FQ_CHECK_LAUNCH("fq_moe_combine");
  return FQ_OK;
}

fq_status fq_moe_combine_bwd(const uint16_t *dout, const float *probs, const int32_t *row_of,
                             int32_t T, int32_t topk, int32_t H, uint16_t *dO, fq_stream stream) {
  FQ_CHECK_ARG(T >= 0 && topk > 0 && H > 0 && H % 16 == 0, "bad sizes (H must be a multiple of 16)");
  FQ_CHECK_ARG((long)T * H < (1l << 35), "too many elements");
  FQ_CHECK_ARG(T == 0 || (dout && probs && row_of && dO), "NULL pointer");
  FQ_CHECK_ARG((!dout || aligned16(dout)) && (!dO || aligned16(dO)),
               "bf16 tensors must be 16-byte aligned");
  launch_combine_bwd(dout, probs, row_of, T, topk, H, dO, S(stream));
  FQ_CHECK_LAUNCH("fq_moe_combine_bwd");
  return FQ_OK;
}

fq_status fq_moe_unpermute_reduce(const uint16_t *dxq, const int32_t *row_of, const uint16_t *x,
                                  int32_t T, int32_t topk, int32_t H, const fq_act_q *aq,
                                  uint16_t *dx, float *dscale_a, void *ws, size_t ws_bytes,
                                  fq_stream stream) {
  FQ_CHECK_ARG(T >= 0 && topk > 0 && H > 0 && H % 16 == 0, "bad sizes (H must be a multiple of 16)");
  FQ_CHECK_ARG((long)T * H < (1l << 35), "too many elements");
  FQ_CHECK_ARG(T == 0 || (dxq && row_of && dx), "NULL pointer");
  FQ_TRY(check_act_q(aq, H));
  FQ_CHECK_ARG(act_fmt(aq) == FQ_FMT_NONE || T == 0 || x, "x is NULL");
  FQ_CHECK_ARG((!dxq || aligned16(dxq)) && (!dx || aligned16(dx)) && (!x || aligned16(x)),
               "bf16 tensors must be 16-byte aligned");
  if (dscale_a) FQ_TRY(check_dscale_a("fq_moe_unpermute_reduce", aq, T, H, ws, ws_bytes));
  launch_unpermute_reduce(dxq, row_of, x, T, topk, H, act_fmt(aq), aq ? aq->scale : nullptr, dx,
                          dscale_a, static_cast<float *>(ws), S(stream));
  FQ_CHECK_LAUNCH("fq_moe_unpermute_reduce");
  return FQ_OK;
}

}  // extern "C"
