"""Seeded synthetic inputs for the fake-quant MoE hot path.

This module only draws random tensors; it holds none of the method's arithmetic
(no quantisation, no scales, no GEMMs). It is the one piece shared by the CPU
oracle, the HIP path's tests and the benchmark.

Every tensor is drawn on the CPU from a ``torch.Generator`` seeded per call, in
a fixed draw order, so the same call gives the same bits on any machine.
Normals are drawn in fp32 and cast to bfloat16 with round-to-nearest-even.
bfloat16 tensors are returned as ``numpy.uint16`` arrays holding the raw bits;
integer and fp32 tensors as ordinary numpy arrays.

Shapes follow the Qwen3-30B-A3B MoE layer (128 experts, hidden 2048, expert FFN
768, top-8 routing) that the AngelSlim mcore_qad article trains with stacked
3D expert weights (section "分组专家 Grouped Experts"); the dense cases follow
the single-linear QAT setting of the AngelSlim QAT + ZeRO-3 page.

Routing is an input of the path: the router stays unquantised and outside it
(mcore_qad article, fake-quant injection section). Routing weights are
softmax -> top-k (ties to the lower expert id) -> renormalised over the k
chosen experts, as Qwen3-MoE does; Zipf-skewed routing samples k experts
without replacement in proportion to w_e = (e+1)^-s via Gumbel-top-k.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import numpy as np
import torch

HIDDEN = 2048
FFN = 768
N_EXPERTS = 128
TOPK = 8

# Format tags for the five workloads (plain strings; the numeric enums live on
# each side of the boundary separately).
FMT_INT8 = "int8"
FMT_INT4 = "int4"
FMT_FP8 = "fp8"
FMT_NVFP4 = "nvfp4"


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def normal_bf16(gen: torch.Generator, shape: Sequence[int], std: float = 1.0) -> np.ndarray:
    """N(0, std^2) drawn in fp32, scaled in fp32, cast to bf16 (RNE); raw bits."""
    t = torch.randn(*shape, generator=gen, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bits_to_torch_bf16(a: np.ndarray) -> torch.Tensor:
    """View raw bf16 bits (uint16 numpy) as a torch bfloat16 CPU tensor (no copy)."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)


def softmax_topk_routing(logits: np.ndarray, k: int):
    """softmax -> top-k (ties to lower id) -> renormalise. Returns (ids int32, p fp32)."""
    lg = logits.astype(np.float64)
    # top-k of softmax == top-k of logits; a stable sort of -logits breaks ties
    # toward the lower expert id.
    order = np.argsort(-lg, axis=1, kind="stable")[:, :k]
    sel = np.take_along_axis(lg, order, axis=1)
    ex = np.exp(sel - sel.max(axis=1, keepdims=True))
    p = ex / ex.sum(axis=1, keepdims=True)
    return order.astype(np.int32), p.astype(np.float32)


def zipf_routing(gen: torch.Generator, T: int, n_experts: int, k: int, s: float,
                 zero_experts: Sequence[int] = ()):
    """Gumbel-top-k sampling without replacement with weights (e+1)^-s.

    Experts listed in ``zero_experts`` get weight 0 and are never chosen.
    p = softmax over the k chosen perturbed log-weights.
    """
    w = (np.arange(n_experts, dtype=np.float64) + 1.0) ** (-s)
    for e in zero_experts:
        w[e] = 0.0
    with np.errstate(divide="ignore"):
        logw = np.log(w)
    u = torch.rand(T, n_experts, generator=gen, dtype=torch.float64).numpy()
    with np.errstate(divide="ignore"):
        gumbel = -np.log(-np.log(u))
    score = logw[None, :] + gumbel
    order = np.argsort(-score, axis=1, kind="stable")[:, :k]
    sel = np.take_along_axis(score, order, axis=1)
    ex = np.exp(sel - sel.max(axis=1, keepdims=True))
    p = ex / ex.sum(axis=1, keepdims=True)
    return order.astype(np.int32), p.astype(np.float32)


@dataclasses.dataclass
class DenseCase:
    """One dense linear: Y = X . FQ(W)^T, with upstream gradient dY."""
    name: str
    fmt: str
    group: int          # K for per-channel, 128 for int4, 16 for nvfp4
    w: np.ndarray       # [N, K] bf16 bits
    x: np.ndarray       # [M, K] bf16 bits
    dy: np.ndarray      # [M, N] bf16 bits
    act_fmt: str = "none"


@dataclasses.dataclass
class MoECase:
    """One MoE layer's routed-expert path (gate_up -> SwiGLU -> down)."""
    name: str
    fmt: str
    n_experts_global: int
    expert_begin: int
    w_gu: np.ndarray        # [E_local, 2F, H] bf16 bits
    w_d: np.ndarray         # [E_local, H, F] bf16 bits
    x: np.ndarray           # [T, H] bf16 bits
    expert_ids: np.ndarray  # [T, k] int32 (global ids)
    probs: np.ndarray       # [T, k] fp32
    dout: np.ndarray        # [T, H] bf16 bits

    @property
    def E(self) -> int:
        return self.w_gu.shape[0]

    @property
    def T(self) -> int:
        return self.x.shape[0]

    @property
    def topk(self) -> int:
        return self.expert_ids.shape[1]


def dense_case(M: int, N: int, K: int, fmt: str, group: int, seed: int = 0,
               w_std: float = 0.02, outlier_frac: float = 0.0, outlier_mult: float = 20.0,
               name: str = "dense") -> DenseCase:
    """Draw order: W, outlier positions, X, dY."""
    g = _gen(seed)
    wt = torch.randn(N, K, generator=g, dtype=torch.float32).mul_(w_std)
    n_out = int(outlier_frac * N * K)
    if n_out > 0:
        pos = torch.randperm(N * K, generator=g)[:n_out]
        wt.view(-1)[pos] *= outlier_mult
    w = wt.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    x = normal_bf16(g, (M, K))
    dy = normal_bf16(g, (M, N))
    return DenseCase(name=name, fmt=fmt, group=group, w=w, x=x, dy=dy)


def moe_case(T: int, fmt: str, E_global: int = N_EXPERTS, H: int = HIDDEN, F: int = FFN,
             topk: int = TOPK, seed: int = 0, expert_begin: int = 0,
             E_local: Optional[int] = None, zipf_s: Optional[float] = None,
             zero_experts: Sequence[int] = (), w_std: float = 0.02,
             name: str = "moe") -> MoECase:
    """Draw order: W_gu, W_d (local experts only), X, routing, dOut."""
    if E_local is None:
        E_local = E_global - expert_begin
    g = _gen(seed)
    w_gu = normal_bf16(g, (E_local, 2 * F, H), std=w_std)
    w_d = normal_bf16(g, (E_local, H, F), std=w_std)
    x = normal_bf16(g, (T, H))
    if zipf_s is None:
        logits = torch.randn(T, E_global, generator=g, dtype=torch.float32).numpy()
        ids, p = softmax_topk_routing(logits, topk)
    else:
        ids, p = zipf_routing(g, T, E_global, topk, zipf_s, zero_experts)
    dout = normal_bf16(g, (T, H))
    return MoECase(name=name, fmt=fmt, n_experts_global=E_global, expert_begin=expert_begin,
                   w_gu=w_gu, w_d=w_d, x=x, expert_ids=ids, probs=p, dout=dout)


def kd_logits(T: int, V: int, seed: int = 0, device: str = "cpu", teacher_std: float = 2.0,
              peaks: int = 4, peak_boost: float = 8.0, student_noise: float = 0.3):
    """Synthetic teacher / student logits [T, V] (bf16) for the top-K KL
    distillation kernel: teacher ~ N(0, teacher_std^2) with `peaks` random
    vocabulary entries per token raised by peak_boost (a peaked next-token
    distribution); student = teacher + N(0, student_noise^2) (the quantized
    copy of the same model). Draw order: teacher, peak positions, student
    noise. On device "cpu" the draws are the CPU generator's; on "cuda" the
    device generator's (same seed, same bits on a given torch build).
    Returns two torch bfloat16 tensors on `device`."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    t = torch.randn(T, V, generator=g, device=device, dtype=torch.float32).mul_(teacher_std)
    if peaks > 0:
        pos = torch.randint(0, V, (T, peaks), generator=g, device=device)
        t.scatter_add_(1, pos, torch.full((T, peaks), peak_boost, device=device))
    s = torch.randn(T, V, generator=g, device=device, dtype=torch.float32).mul_(student_noise)
    s.add_(t)
    return s.to(torch.bfloat16), t.to(torch.bfloat16)


# Shape of the distillation kernel's workload: one 4096-token micro-batch over
# the Qwen3 vocabulary (151936 entries), teacher top-1000 (the kl_top_1000
# example of the QAT + ZeRO-3 page's loss table).
KD_TOKENS = 4096
KD_VOCAB = 151936
KD_TOPK = 1000
KD_NAME = "kd-topk1000-t4096-v151936"


# ---------------------------------------------------------------------------
# The five workloads, full size.
# ---------------------------------------------------------------------------
CONFIG_NAMES = {
    1: "dense-int8-w256x512-m64",
    2: "dense-int4g128-w4096x4096-m2048",
    3: "moe-fp8-e128-h2048-f768-t8192-top8",
    4: "moe-nvfp4-e128-h2048-f768-t16384-top8",
    5: "moe-nvfp4-local16of128-h2048-f768-t32768-top8-zipf1.2",
}

# Experts that get zero routing weight in the Zipf-skewed local-share workload,
# so that some local experts receive no tokens.
ZIPF_EMPTY_EXPERTS = (3, 7, 11, 15)


def config(cfg: int, seed: int = 0):
    """The full-size workload ``cfg`` (1..5)."""
    if cfg == 1:
        return dense_case(64, 256, 512, FMT_INT8, 512, seed=seed, name=CONFIG_NAMES[1])
    if cfg == 2:
        return dense_case(2048, 4096, 4096, FMT_INT4, 128, seed=seed, outlier_frac=0.001,
                          name=CONFIG_NAMES[2])
    if cfg == 3:
        return moe_case(8192, FMT_FP8, seed=seed, name=CONFIG_NAMES[3])
    if cfg == 4:
        return moe_case(16384, FMT_NVFP4, seed=seed, name=CONFIG_NAMES[4])
    if cfg == 5:
        return moe_case(32768, FMT_NVFP4, seed=seed, E_local=16, zipf_s=1.2,
                        zero_experts=ZIPF_EMPTY_EXPERTS, name=CONFIG_NAMES[5])
    raise ValueError(f"unknown workload {cfg}")
