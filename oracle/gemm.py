"""Grouped GEMM with fake-quantised operands, forward and scale-only backward
(test infrastructure only).

Forward (mcore_qad article, section 二.4: one GEMM over all experts' routed
rows; section 二.3: weights and inputs fake-quantised before the matmul):
    Y[r, :] = FQ_a(X)[r, :] . FQ_w(W[e])^T      for r in segment e
computed per expert with float64 accumulation of the bf16 operand values and
rounded to bf16 (the stored dtype).

Backward (section 一: weights frozen, only scales trained; section 二.3:
gradient reaches the scale through autograd), with the STE factors of
``codecs``:
    dXq      = dY_e . FQ_w(W[e])            dX = bf16(m_x * dXq)
    dWq[e]   = dY_e^T . Xq_e                (never stored)
    dS[e,n,g] = sum_{k in g} dWq[e,n,k] * dv/ds(e,n,k)
    dZP[e,n,g] = sum_{k in g} dWq[e,n,k] * dv/dzp(e,n,k)   (int4 only)
    dS[e]     = sum_{n,k} dWq[e,n,k] * dv/ds(e,n,k)        (per-tensor scale)
An expert with no rows gets dS = 0.
"""
from __future__ import annotations

import numpy as np

from .codecs import FMT_INT4, GROUP_TENSOR, fq_act, fq_weight_stack
from .numerics import bf16_to_f32, f64_to_bf16


def grouped_gemm_fwd(x_bits, seg, w_bits, wfmt: int, group: int, scale, zero_point=None,
                     global_scale=None, afmt: int = 0, act_scale=None):
    """Returns y bits [R, N] for the R = seg[-1] routed rows."""
    seg = np.asarray(seg, dtype=np.int64)
    R = int(seg[-1])
    xq = fq_act(np.asarray(x_bits)[:R], afmt, act_scale)
    wq = fq_weight_stack(w_bits, wfmt, group, scale, zero_point, global_scale)
    a = bf16_to_f32(xq.bits).astype(np.float64)
    b = bf16_to_f32(wq.bits).astype(np.float64)
    E, N, K = b.shape
    y = np.zeros((R, N), dtype=np.float64)
    for e in range(E):
        lo, hi = seg[e], seg[e + 1]
        if hi > lo:
            y[lo:hi] = a[lo:hi] @ b[e].T
    return f64_to_bf16(y)


def grouped_gemm_bwd(dy_bits, x_bits, seg, w_bits, wfmt: int, group: int, scale,
                     zero_point=None, global_scale=None, afmt: int = 0, act_scale=None):
    """Returns (dx bits [R, K], dscale float64 [E, N, K/group] (per-tensor: [E]),
    dzp float64 or None)."""
    seg = np.asarray(seg, dtype=np.int64)
    R = int(seg[-1])
    xq = fq_act(np.asarray(x_bits)[:R], afmt, act_scale)
    wq = fq_weight_stack(w_bits, wfmt, group, scale, zero_point, global_scale)
    a = bf16_to_f32(xq.bits).astype(np.float64)
    b = bf16_to_f32(wq.bits).astype(np.float64)
    dy = bf16_to_f32(np.asarray(dy_bits)[:R]).astype(np.float64)
    E, N, K = b.shape
    per_tensor = group == GROUP_TENSOR
    G = 1 if per_tensor else K // group
    dx = np.zeros((R, K), dtype=np.float64)
    ds = np.zeros((E,) if per_tensor else (E, N, G), dtype=np.float64)
    dzp = np.zeros((E, N, G), dtype=np.float64) if wfmt == FMT_INT4 else None
    for e in range(E):
        lo, hi = seg[e], seg[e + 1]
        if hi <= lo:
            continue
        dx[lo:hi] = dy[lo:hi] @ b[e]
        dwq = dy[lo:hi].T @ a[lo:hi]                       # [N, K]
        if per_tensor:
            ds[e] = np.sum(dwq * wq.dv_ds[e])
        else:
            ds[e] = (dwq * wq.dv_ds[e]).reshape(N, G, group).sum(axis=-1)
        if dzp is not None:
            dzp[e] = (dwq * wq.dv_dzp[e]).reshape(N, G, group).sum(axis=-1)
    dx = dx * xq.mask
    return f64_to_bf16(dx), ds, dzp
