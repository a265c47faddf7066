"""The routed-expert path of one MoE layer, forward and scale-only backward
(test infrastructure only).

Structure: the experts of a layer are one gate_up stack [E, 2F, H] and one
down stack [E, H, F] (mcore_qad article, section 二.4); inputs of each
projection are fake-quantised before the matmul (section 二.3); the activation
between them is SwiGLU (the experts' act_fn, QAT + ZeRO-3 page, architecture
notes on fused MoE experts). The router is unquantised and outside the path
(section 二.3): expert ids and routing weights are inputs (R-11, R-12).

Forward, per routed row r of expert e (token t = perm[r] // k):
  Xq[r] = FQ_a1(X[t])                                   gather + act FQ
  H     = Xq . FQ(W_gu[e])^T                            bf16
  A     = bf16(silu(H[:, :F]) * H[:, F:])               gate first (R-10)
  Aq    = FQ_a2(A)
  O     = Aq . FQ(W_d[e])^T                             bf16
  out[t] = bf16(sum_j p[t,j] * O[row_of[t,j]])           slots ascending
Backward (dX and the weight-scale gradients; activation scales frozen unless
learnable, R-23):
  dO[r]  = bf16(p[t,j] * dOut[t])
  dA     = bf16(m_a2 * (dO . FQ(W_d[e])))               + dS_d from dO^T . Aq
  dH     = bf16(SwiGLU'(H) applied to dA)
  dXq    = bf16(dH . FQ(W_gu[e]))                       + dS_gu from dH^T . Xq
  dX[t]  = bf16(m_a1(X[t]) * sum_j dXq[row_of[t,j]])
  dS_a1  = sum over t, h of (sum_j dXq[row_of[t,j], h]) * dv/ds(X[t, h])  (R-23)
  dS_a2  = sum over r, f of dAq[r, f] * dv/ds(A[r, f])
Float64 everywhere except where the GPU stores bf16.
"""
from __future__ import annotations

import numpy as np

from .codecs import FMT_FP8, FMT_INT8, FMT_NONE, fq_act
from .gemm import grouped_gemm_bwd, grouped_gemm_fwd
from .numerics import bf16_to_f32, f64_to_bf16
from .observer import observer_act, observer_weight
from .permute import moe_permute


def gather_actfq(x_bits, perm, topk: int, afmt: int, act_scale):
    """Xq[r] = FQ_a(X[perm[r] // topk]). Returns the FQ record of the gathered rows."""
    tok = np.asarray(perm, dtype=np.int64) // topk
    return fq_act(np.asarray(x_bits)[tok], afmt, act_scale)


def _sigmoid(g):
    # exp(-g) overflows to inf for g below about -709, and 1 / inf = 0 is the limit
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-g))


def swiglu_fwd(h_bits):
    """A = bf16(silu(gate) * up), gate = H[:, :F], up = H[:, F:] (R-10)."""
    h = bf16_to_f32(h_bits).astype(np.float64)
    F = h.shape[1] // 2
    g, u = h[:, :F], h[:, F:]
    return f64_to_bf16(g * _sigmoid(g) * u)


def swiglu_actfq(h_bits, afmt: int, act_scale):
    a = swiglu_fwd(h_bits)
    return a, fq_act(a, afmt, act_scale)


def swiglu_bwd(dq_bits, h_bits, afmt: int, act_scale, a_bits=None):
    """dH from dAq (the unmasked dgrad of the down projection).

    dA = m_a2 * dAq, m_a2 the activation-FQ mask of A (recomputed from H, or from
    ``a_bits`` when given); dgate = dA*up*s*(1 + g*(1-s)), dup = dA*g*s, s = sigmoid(g).
    """
    h = bf16_to_f32(h_bits).astype(np.float64)
    F = h.shape[1] // 2
    g, u = h[:, :F], h[:, F:]
    if a_bits is None:
        a_bits = swiglu_fwd(h_bits)
    m = fq_act(a_bits, afmt, act_scale).mask if afmt != FMT_NONE else 1.0
    da = bf16_to_f32(dq_bits).astype(np.float64) * m
    s = _sigmoid(g)
    dgate = da * u * s * (1.0 + g * (1.0 - s))
    dup = da * g * s
    return f64_to_bf16(np.concatenate([dgate, dup], axis=1))


def combine(o_bits, probs, row_of):
    """out[t] = bf16(sum over local slots j of p[t,j] * O[row_of[t,j]])."""
    o = bf16_to_f32(o_bits).astype(np.float64)
    row_of = np.asarray(row_of, dtype=np.int64)
    p = np.asarray(probs, dtype=np.float32).astype(np.float64)
    T, k = row_of.shape
    out = np.zeros((T, o.shape[1]), dtype=np.float64)
    for j in range(k):
        r = row_of[:, j]
        ok = r >= 0
        out[ok] += p[ok, j:j + 1] * o[r[ok]]
    return f64_to_bf16(out)


def combine_bwd(dout_bits, probs, perm, topk: int):
    """dO[r] = bf16(p[t,j] * dOut[t]) with f = perm[r], t = f // k, j = f % k."""
    perm = np.asarray(perm, dtype=np.int64)
    t, j = perm // topk, perm % topk
    d = bf16_to_f32(dout_bits).astype(np.float64)[t]
    p = np.asarray(probs, dtype=np.float32).astype(np.float64)[t, j]
    return f64_to_bf16(d * p[:, None])


def unpermute_sum(dxq_bits, row_of):
    """The gradient reaching FQ_a1(X[t]): sum over local slots of dXq[row_of[t,j]]
    (float64; tokens routed to no local expert get 0)."""
    dxq = bf16_to_f32(dxq_bits).astype(np.float64)
    row_of = np.asarray(row_of, dtype=np.int64)
    T, k = row_of.shape
    acc = np.zeros((T, dxq.shape[1]), dtype=np.float64)
    for j in range(k):
        r = row_of[:, j]
        ok = r >= 0
        acc[ok] += dxq[r[ok]]
    return acc


def unpermute_reduce(dxq_bits, row_of, x_bits, afmt: int, act_scale):
    """dX[t] = bf16(m_a1(X[t]) * sum over local slots of dXq[row_of[t,j]])."""
    acc = unpermute_sum(dxq_bits, row_of)
    m = fq_act(x_bits, afmt, act_scale).mask if afmt != FMT_NONE else 1.0
    return f64_to_bf16(acc * m)


def act_scale_grad(x_bits, g, afmt: int, act_scale) -> float:
    """Gradient of a learnable per-tensor activation scale s_a (R-23).

    FQ_a maps every element x of the tensor to v = q(x / s_a) * s_a; with the
    round passed straight through (R-13, R-14) dv/ds_a is the same factor as for
    a weight scale, q - z inside the range and the bound outside it. The chain
    rule sums it against ``g``, the gradient reaching FQ_a's output, over all
    elements (float64). Only the static per-tensor formats FP8 and INT8 have such
    a scale."""
    if afmt not in (FMT_FP8, FMT_INT8):
        raise ValueError(f"no learnable per-tensor scale for activation format {afmt}")
    fq = fq_act(x_bits, afmt, act_scale)
    return float(np.sum(np.asarray(g, dtype=np.float64) * fq.dv_ds))


def teacher_forward(case):
    """The self-teacher: the same layer with quantization off (mcore_qad article,
    section 一): plain gather, bf16 grouped GEMMs on the frozen weights,
    SwiGLU, combine. Returns out bits [T, H]."""
    E = case.w_gu.shape[0]
    k = case.expert_ids.shape[1]
    perm, row_of, seg = moe_permute(case.expert_ids, case.expert_begin, E)
    xg = np.asarray(case.x)[np.asarray(perm, dtype=np.int64) // k]
    h = grouped_gemm_fwd(xg, seg, case.w_gu, FMT_NONE, None, None)
    a = swiglu_fwd(h)
    o = grouped_gemm_fwd(a, seg, case.w_d, FMT_NONE, None, None)
    return combine(o, case.probs, row_of)


def moe_layer(case, wfmt: int, group, afmt: int, wq_gu=None, wq_d=None,
              act_scales=None):
    """Full forward + scale-only backward of one MoE layer's routed-expert path.

    group: elements per weight scale, or None for one scale per output
    channel (the K of each stack). wq_gu / wq_d: (scale, zero_point,
    global_scale) of each stack; observer init when None. act_scales: (s_a1,
    s_a2); calibrated on this batch when None (s_a1 from X, s_a2 from the
    calibration A). Returns a dict of every
    intermediate (bf16 bits unless noted); ds_a1 / ds_a2 are the gradients of
    the two activation scales (float, FP8 / INT8 activations only, else None).
    """
    E = case.w_gu.shape[0]
    k = case.expert_ids.shape[1]
    g_gu = group or case.w_gu.shape[2]
    g_d = group or case.w_d.shape[2]
    if wq_gu is None:
        wq_gu = observer_weight(case.w_gu, wfmt, g_gu)
    if wq_d is None:
        wq_d = observer_weight(case.w_d, wfmt, g_d)
    perm, row_of, seg = moe_permute(case.expert_ids, case.expert_begin, E)
    calibrated = act_scales is None
    if calibrated:
        s1 = observer_act(case.x, afmt) if afmt != FMT_NONE else np.float32(1.0)
    else:
        s1 = act_scales[0]
    xq = gather_actfq(case.x, perm, k, afmt, s1)
    h = grouped_gemm_fwd(xq.bits, seg, case.w_gu, wfmt, g_gu, *wq_gu)
    if calibrated:
        a_cal = swiglu_fwd(h)
        s2 = observer_act(a_cal, afmt) if afmt != FMT_NONE else np.float32(1.0)
    else:
        s2 = act_scales[1]
    a, aq = swiglu_actfq(h, afmt, s2)
    o = grouped_gemm_fwd(aq.bits, seg, case.w_d, wfmt, g_d, *wq_d)
    out = combine(o, case.probs, row_of)
    do = combine_bwd(case.dout, case.probs, perm, k)
    daq, ds_d, dzp_d = grouped_gemm_bwd(do, aq.bits, seg, case.w_d, wfmt, g_d, *wq_d)
    dh = swiglu_bwd(daq, h, afmt, s2, a_bits=a)
    dxq, ds_gu, dzp_gu = grouped_gemm_bwd(dh, xq.bits, seg, case.w_gu, wfmt, g_gu, *wq_gu)
    dx = unpermute_reduce(dxq, row_of, case.x, afmt, s1)
    ds_a1 = ds_a2 = None
    if afmt in (FMT_FP8, FMT_INT8):
        ds_a1 = act_scale_grad(case.x, unpermute_sum(dxq, row_of), afmt, s1)
        ds_a2 = act_scale_grad(a, bf16_to_f32(daq), afmt, s2)
    return dict(perm=perm, row_of=row_of, seg=seg, s_a1=np.float32(s1), s_a2=np.float32(s2),
                wq_gu=wq_gu, wq_d=wq_d, xq=xq.bits, h=h, a=a, aq=aq.bits, o=o, out=out,
                do=do, daq=daq, dh=dh, dxq=dxq, dx=dx, ds_gu=ds_gu, ds_d=ds_d,
                dzp_gu=dzp_gu, dzp_d=dzp_d, ds_a1=ds_a1, ds_a2=ds_a2)
