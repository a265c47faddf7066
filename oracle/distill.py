"""Self-distillation pieces of scale-only QAD (test infrastructure only).

What they are: with distillation on, the teacher is the same frozen model run
again with quantization switched off (AngelSlim mcore_qad article, section
一), and the loss between student and teacher logits is a KL divergence;
with a top-k setting the KL is taken only over the teacher's k most likely
tokens, so the [tokens, vocab] probabilities are never formed (same article,
section 二.5; the QAT + ZeRO-3 page's loss table lists the forward and reverse
top-K variants kl_top_K / r_kl_top_K, averaged over the valid tokens).

Readings (R-25): per token, S = the K vocabulary entries with the largest
teacher logits (equal logits: the lower index first); both distributions are
the softmax of the logits restricted to S; forward KL = sum over S of
p_t (log p_t - log p_s), reverse KL = sum over S of p_s (log p_s - log p_t);
the loss is the mean over valid tokens. Only the student's logits get a
gradient (the teacher is frozen and runs without autograd).
"""
from __future__ import annotations

import numpy as np

from .numerics import bf16_to_f32


def topk_set(teacher_bits, K: int) -> np.ndarray:
    """[T, K] vocabulary indices of each row's K largest teacher logits, ties
    to the lower index, listed in increasing index order."""
    t = bf16_to_f32(teacher_bits).astype(np.float64)
    T, V = t.shape
    assert 1 <= K <= V
    out = np.empty((T, K), dtype=np.int64)
    for r in range(T):
        # stable sort on -logit keeps equal logits in index order
        order = np.argsort(-t[r], kind="stable")
        out[r] = np.sort(order[:K])
    return out


def _log_softmax(z):
    m = z.max(axis=-1, keepdims=True)
    return z - m - np.log(np.exp(z - m).sum(axis=-1, keepdims=True))


def topk_kl(student_bits, teacher_bits, K: int, reverse: bool = False, valid=None):
    """Top-K KL distillation loss and its gradient on the student logits.

    Returns (idx [T, K] int64, grad [T, K] float64 = d(mean loss)/d student
    logit at idx, loss_tok [T] float64 (0 for invalid tokens), loss_mean)."""
    s = bf16_to_f32(student_bits).astype(np.float64)
    t = bf16_to_f32(teacher_bits).astype(np.float64)
    T, V = t.shape
    valid = np.ones(T, bool) if valid is None else np.asarray(valid).astype(bool)
    idx = topk_set(teacher_bits, K)
    zs = np.take_along_axis(s, idx, axis=1)
    zt = np.take_along_axis(t, idx, axis=1)
    ls, lt = _log_softmax(zs), _log_softmax(zt)
    ps, pt = np.exp(ls), np.exp(lt)
    if reverse:
        loss = (ps * (ls - lt)).sum(axis=1)
        # d/dz_s of sum p_s (log p_s - log p_t) = p_s * ((log p_s - log p_t) - loss)
        g = ps * ((ls - lt) - loss[:, None])
    else:
        loss = (pt * (lt - ls)).sum(axis=1)
        g = ps - pt
    n = int(valid.sum())
    loss = np.where(valid, loss, 0.0)
    g = np.where(valid[:, None], g, 0.0) / max(n, 1)
    mean = float(loss.sum() / max(n, 1))
    return idx, g, loss, mean
