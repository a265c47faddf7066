"""Scale initialisation from observed statistics (test infrastructure only).

Sources: the PTQ weight scale max|W|/448 for FP8 ("QAT + DeepSpeed ZeRO-3"
page, section "Quantizer 初始值"); activation scales set by a calibration
forward (same page, overview: lazy activation-scale init); per-channel min /
max turned into quantisation parameters (msmodelslim multi-card page, FA3
observer section). The same absmax rule, with each format's grid maximum, gives
int8 (127) and NVFP4 (6 * 448, the E2M1 max times the E4M3 max).

All divisions are single IEEE fp32 divisions; an all-zero row / group / tensor
gets scale 1.0 (R-4).
"""
from __future__ import annotations

import numpy as np

from .codecs import (E4M3_MAX, E2M1_MAX, FMT_FP8, FMT_INT4, FMT_INT8, FMT_NVFP4,
                     GROUP_TENSOR, NVFP4_BLOCK, e4m3_round)
from .numerics import bf16_to_f32

NVFP4_DIV = np.float32(E2M1_MAX * E4M3_MAX)   # 2688


def _safe_scale(s: np.ndarray) -> np.ndarray:
    s = np.asarray(s, dtype=np.float32)
    return np.where(s == 0, np.float32(1.0), s).astype(np.float32)


def observer_weight(w_bits, fmt: int, group: int):
    """Initial learnable parameters of a stacked weight [E, N, K].

    Returns (scale [E,N,K/group] fp32, zero_point or None, global_scale or None).
      int8 : s = amax_group / 127
      fp8  : s = amax_group / 448
      group GROUP_TENSOR (int8 / fp8): the amax of each expert matrix, scale [E]
      int4 : lo = min(0, min), hi = max(0, max); s = (hi - lo) / 15;
             zp = clamp(rne(-lo * (1/s)), 0, 15)                      (R-5)
      nvfp4: g_e = amax_expert / 2688;
             theta_b = e4m3(clamp(amax_b * (1/(6*g_e)), 0, 448))      (R-8)
    """
    w = bf16_to_f32(w_bits)
    E, N, K = w.shape
    if fmt in (FMT_INT8, FMT_FP8) and group == GROUP_TENSOR:
        amax = np.abs(w).reshape(E, -1).max(axis=-1).astype(np.float32)
        div = np.float32(127.0) if fmt == FMT_INT8 else np.float32(E4M3_MAX)
        return _safe_scale(amax / div), None, None
    if fmt in (FMT_INT8, FMT_FP8):
        amax = np.abs(w).reshape(E, N, K // group, group).max(axis=-1).astype(np.float32)
        div = np.float32(127.0) if fmt == FMT_INT8 else np.float32(E4M3_MAX)
        return _safe_scale(amax / div), None, None
    if fmt == FMT_INT4:
        blk = w.reshape(E, N, K // group, group)
        lo = np.minimum(blk.min(axis=-1), np.float32(0.0)).astype(np.float32)
        hi = np.maximum(blk.max(axis=-1), np.float32(0.0)).astype(np.float32)
        s = _safe_scale(((hi - lo).astype(np.float32) / np.float32(15.0)).astype(np.float32))
        r = (np.float32(1.0) / s).astype(np.float32)
        zp = np.clip(np.rint((-lo * r).astype(np.float32).astype(np.float64)), 0.0, 15.0)
        return s, zp.astype(np.float32), None
    if fmt == FMT_NVFP4:
        assert group == NVFP4_BLOCK
        amax_e = np.abs(w).reshape(E, -1).max(axis=-1).astype(np.float32)
        g = _safe_scale((amax_e / NVFP4_DIV).astype(np.float32))
        amax_b = np.abs(w).reshape(E, N, K // group, group).max(axis=-1).astype(np.float32)
        d = (np.float32(6.0) * g).astype(np.float32)
        rd = (np.float32(1.0) / d).astype(np.float32)
        t = (amax_b * rd[:, None, None]).astype(np.float32)
        _, th = e4m3_round(np.clip(t, np.float32(0.0), np.float32(E4M3_MAX)))
        return th.astype(np.float32), None, g
    raise ValueError(f"unsupported weight format {fmt}")


def observer_act(x_bits, fmt: int) -> np.float32:
    """Per-tensor activation scale from a calibration batch.

    fp8: s_a = amax / 448; nvfp4: g_a = amax / 2688; int8: amax / 127.
    """
    x = bf16_to_f32(x_bits)
    amax = np.float32(np.abs(x).max()) if x.size else np.float32(0.0)
    if fmt == FMT_FP8:
        div = np.float32(E4M3_MAX)
    elif fmt == FMT_NVFP4:
        div = NVFP4_DIV
    elif fmt == FMT_INT8:
        div = np.float32(127.0)
    else:
        raise ValueError(f"unsupported activation format {fmt}")
    return np.float32(_safe_scale(np.float32(amax / div)))
