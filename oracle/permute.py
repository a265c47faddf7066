"""Routed-token permutation (test infrastructure only).

One grouped GEMM over all experts needs the routed rows of each expert to be
contiguous (mcore_qad article, section 二.4). Pairs are indexed f = t*k + j
(token t, slot j). The local pairs (expert in [expert_begin,
expert_begin + E_local)) are ordered by (local expert, f): a stable counting
sort. This order is unique.
"""
import numpy as np


def moe_permute(expert_ids, expert_begin: int, E_local: int):
    """Returns (perm [R] int32, row_of [T,k] int32 (-1 if not local), seg [E_local+1] int32)."""
    ids = np.asarray(expert_ids, dtype=np.int64)
    T, k = ids.shape
    flat = ids.reshape(-1)
    local = (flat >= expert_begin) & (flat < expert_begin + E_local)
    f = np.nonzero(local)[0]
    le = flat[f] - expert_begin
    order = np.lexsort((f, le))          # primary key: local expert, then f
    perm = f[order]
    counts = np.bincount(le, minlength=E_local)
    seg = np.zeros(E_local + 1, dtype=np.int64)
    seg[1:] = np.cumsum(counts)
    row_of = np.full(T * k, -1, dtype=np.int64)
    row_of[perm] = np.arange(perm.size)
    return perm.astype(np.int32), row_of.reshape(T, k).astype(np.int32), seg.astype(np.int32)
