"""The four fake-quant codecs of the oracle (test infrastructure only).

What is computed (AngelSlim mcore_qad article, sections 一 and 二.3): the
forward replaces a weight or activation tensor x by quantize->dequantize of it
with a scale, the backward lets the gradient reach x and the (learnable) scale.
The article lists the formats nvfp4 (W4A4), fp8 (W8A8), w4a16 (int4) and w8a8
(int8) in section 三; their definitions (grids, group sizes, scale shapes) are
the standard ones named there: int8 symmetric per output channel, int4
asymmetric with group 128 along K, FP8 E4M3 and NVFP4 = E2M1 values with one
E4M3 scale per 16-element block times one fp32 tensor scale.

All arithmetic is IEEE fp32, round-to-nearest-even, no fused multiply-add:
  r = 1/s once per scale (R-1), z = x*r per element, code c = Q(clamp(z)),
  dequantised v = fp32(value(c) * s), output = bf16_rne(v).
Integer formats give +0.0 for a zero code, minifloat formats keep the sign of
z (R-2).

Backward, straight-through estimator (R-13, R-14): with
  v = s * round_ste(clamp(z, lo, hi))   (minus zp inside for int4),
plain autograd gives
  dv/dx = m = [lo <= z <= hi]  (unrounded z, inclusive bounds)
  dv/ds = value(c) - m*z       (value in z units; minus zp for int4)
  dv/dzp = -s*(1-m)            (int4 only)
NVFP4: s_b = e4m3(clamp(theta_b, 0, 448)) * g with STE through that rounding
(R-8), so dv/dtheta_b = g * [0 <= theta_b <= 448] * (value(c) - m*z); a zero
s_b gives a +0.0 block with mask 0 and gradient 0 (R-9).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

from .numerics import bf16_to_f32, f32_to_bf16

FMT_NONE = 0
FMT_INT8 = 1
FMT_INT4 = 2
FMT_FP8 = 3
FMT_NVFP4 = 4
FMT_NAMES = {"none": FMT_NONE, "int8": FMT_INT8, "int4": FMT_INT4, "fp8": FMT_FP8,
             "nvfp4": FMT_NVFP4}

INT8_LO, INT8_HI = -128.0, 127.0      # full two's-complement range (R-3)
INT4_LO, INT4_HI = 0.0, 15.0          # unsigned codes, integer zero point
NVFP4_BLOCK = 16
# One weight scale per expert matrix [N, K] (the per-tensor weight preset of
# the QAT + ZeRO-3 page's fp8_static example; INT8 / FP8 only, R-24).
GROUP_TENSOR = -1
INT4_GROUP = 128


def _e4m3_table() -> np.ndarray:
    """Non-negative finite E4M3 values by code 0x00..0x7E (0x7F is NaN).

    OCP E4M3: 1 sign, 4 exponent bits (bias 7), 3 mantissa bits, no infinity;
    exponent field 0 holds the subnormals m * 2^-9.
    """
    vals = []
    for code in range(0x7F):
        e, m = code >> 3, code & 7
        if e == 0:
            vals.append(m * 2.0 ** -9)
        else:
            vals.append((1.0 + m / 8.0) * 2.0 ** (e - 7))
    return np.array(vals, dtype=np.float64)


E4M3_POS = _e4m3_table()          # increasing, E4M3_POS[126] == 448
E4M3_MAX = float(E4M3_POS[-1])
# E2M1: 1 sign, 2 exponent bits (bias 1), 1 mantissa bit; codes 0..7.
E2M1_POS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
E2M1_MAX = 6.0


def _nearest_index(a: np.ndarray, table: np.ndarray) -> np.ndarray:
    """Index of the table entry nearest to each a >= 0 (a <= table max).

    Ties go to the even index, which is the code with an even last mantissa
    bit (R-6, R-7).
    """
    a = np.asarray(a, dtype=np.float64)
    hi = np.searchsorted(table, a, side="left")
    hi = np.minimum(hi, len(table) - 1)
    lo = np.maximum(hi - 1, 0)
    dlo = a - table[lo]
    dhi = table[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    return np.where(pick_hi, hi, lo).astype(np.int64)


def e4m3_round(z) -> tuple:
    """Saturating RNE onto the E4M3 grid. Returns (code uint8, value float64)."""
    z = np.asarray(z, dtype=np.float32)
    zc = np.clip(z, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
    neg = np.signbit(zc)
    idx = _nearest_index(np.abs(zc.astype(np.float64)), E4M3_POS)
    val = np.where(neg, -E4M3_POS[idx], E4M3_POS[idx])
    code = (idx | np.where(neg, 0x80, 0)).astype(np.uint8)
    return code, val


def e2m1_round(z) -> tuple:
    """Saturating RNE onto the E2M1 grid. Returns (4-bit code uint8, value float64)."""
    z = np.asarray(z, dtype=np.float32)
    zc = np.clip(z, np.float32(-E2M1_MAX), np.float32(E2M1_MAX))
    neg = np.signbit(zc)
    idx = _nearest_index(np.abs(zc.astype(np.float64)), E2M1_POS)
    val = np.where(neg, -E2M1_POS[idx], E2M1_POS[idx])
    code = (idx | np.where(neg, 0x8, 0)).astype(np.uint8)
    return code, val


def e4m3_value_of_code(code) -> np.ndarray:
    code = np.asarray(code, dtype=np.int64)
    mag = E4M3_POS[code & 0x7F]
    return np.where(code & 0x80, -mag, mag)


def e2m1_value_of_code(code) -> np.ndarray:
    code = np.asarray(code, dtype=np.int64)
    mag = E2M1_POS[code & 0x7]
    return np.where(code & 0x8, -mag, mag)


@dataclasses.dataclass
class FQ:
    """Everything one fake-quant application defines, elementwise."""
    code: np.ndarray            # integer code (int8 two's complement, uint4, E4M3 byte, E2M1 nibble)
    q: np.ndarray               # grid value in z units: int8 c, int4 (c - zp), fp value(c)  (float64)
    v: np.ndarray               # dequantised fp32 value
    bits: np.ndarray            # bf16 output bits
    z: np.ndarray               # fp32 x * r
    mask: np.ndarray            # STE mask m (bool)
    dv_ds: np.ndarray           # STE factor for the learnable scale (theta for NVFP4), float64
    dv_dzp: Optional[np.ndarray] = None   # int4 only
    s: Optional[np.ndarray] = None        # effective fp32 scale per element


def _f32(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float32)


def _recip(s) -> np.ndarray:
    """r = 1/s in fp32, correctly rounded once per scale (R-1)."""
    with np.errstate(divide="ignore"):
        return (np.float32(1.0) / _f32(s)).astype(np.float32)


def fq_int8(x, s) -> FQ:
    """INT8 symmetric: c = rne(clamp(z, -128, 127)), v = c*s (R-3)."""
    x, s = _f32(x), _f32(s)
    z = (x * _recip(s)).astype(np.float32)
    zc = np.clip(z, np.float32(INT8_LO), np.float32(INT8_HI))
    c = np.rint(zc.astype(np.float64))
    c = c + 0.0  # integer formats: a zero code is +0.0 (R-2)
    m = (z >= INT8_LO) & (z <= INT8_HI)
    v = (c.astype(np.float32) * s).astype(np.float32)
    dv = c - np.where(m, z.astype(np.float64), 0.0)
    return FQ(code=c.astype(np.int64), q=c, v=v, bits=f32_to_bf16(v), z=z, mask=m, dv_ds=dv,
              s=np.broadcast_to(s, x.shape))


def fq_int4(x, s, zp) -> FQ:
    """INT4 asymmetric: zp' = clamp(rne(zp), 0, 15); c' = rne(clamp(z, -zp', 15-zp'));
    code = c' + zp'; v = c'*s (R-5)."""
    x, s = _f32(x), _f32(s)
    zpi = np.clip(np.rint(np.asarray(zp, dtype=np.float64)), INT4_LO, INT4_HI)
    zpi = np.broadcast_to(zpi, x.shape)
    z = (x * _recip(s)).astype(np.float32)
    lo, hi = -zpi, INT4_HI - zpi
    z64 = z.astype(np.float64)
    qv = np.rint(np.clip(z64, lo, hi)) + 0.0
    m = (z64 >= lo) & (z64 <= hi)
    v = (qv.astype(np.float32) * s).astype(np.float32)
    dv = qv - np.where(m, z64, 0.0)
    dzp = -np.broadcast_to(s, x.shape).astype(np.float64) * (~m)
    return FQ(code=(qv + zpi).astype(np.int64), q=qv, v=v, bits=f32_to_bf16(v), z=z, mask=m,
              dv_ds=dv, dv_dzp=dzp, s=np.broadcast_to(s, x.shape))


def fq_fp8(x, s) -> FQ:
    """FP8 E4M3: c = e4m3_rne(clamp(z, -448, 448)), v = value(c)*s (R-6)."""
    x, s = _f32(x), _f32(s)
    z = (x * _recip(s)).astype(np.float32)
    code, val = e4m3_round(z)
    m = (z >= -E4M3_MAX) & (z <= E4M3_MAX)
    v = (val.astype(np.float32) * s).astype(np.float32)
    dv = val - np.where(m, z.astype(np.float64), 0.0)
    return FQ(code=code.astype(np.int64), q=val, v=v, bits=f32_to_bf16(v), z=z, mask=m,
              dv_ds=dv, s=np.broadcast_to(s, x.shape))


def nvfp4_block_scale(theta, g) -> np.ndarray:
    """Effective NVFP4 block scale s_b = fp32(e4m3(clamp(theta, 0, 448)) * g) (R-8)."""
    th = np.clip(_f32(theta), np.float32(0.0), np.float32(E4M3_MAX))
    _, tq = e4m3_round(th)
    return (tq.astype(np.float32) * _f32(g)).astype(np.float32)


def fq_nvfp4(x, theta, g) -> FQ:
    """NVFP4 with per-element (already broadcast) block parameter theta and tensor scale g.

    x, theta, g broadcast together. dv_ds holds dv/dtheta.
    """
    x = _f32(x)
    theta = _f32(theta)
    g = _f32(g)
    s = np.broadcast_to(nvfp4_block_scale(theta, g), x.shape)
    zero = s == 0
    s_safe = np.where(zero, np.float32(1.0), s)
    z = (x * _recip(s_safe)).astype(np.float32)
    z = np.where(zero, np.float32(0.0), z)
    code, val = e2m1_round(z)
    code = np.where(zero, 0, code)
    val = np.where(zero, 0.0, val)
    m = (z >= -E2M1_MAX) & (z <= E2M1_MAX) & ~zero
    v = np.where(zero, np.float32(0.0), (val.astype(np.float32) * s).astype(np.float32))
    th_in = (theta >= 0) & (theta <= E4M3_MAX)
    dv = np.where(zero, 0.0, g.astype(np.float64) * th_in *
                  (val - np.where(m, z.astype(np.float64), 0.0)))
    return FQ(code=code.astype(np.int64), q=val, v=v.astype(np.float32), bits=f32_to_bf16(v),
              z=z, mask=m, dv_ds=dv, s=s)


def nvfp4_dynamic_theta(x, g_a) -> np.ndarray:
    """Dynamic activation block parameter from each 16-element block's amax.

    theta = e4m3(clamp(amax_b * (1/(6*g_a)), 0, 448)), computed in fp32 (the
    'dynamic' scale source of the mcore_qad article, section 六; same rule as
    the weight observer). Returns theta per block: [..., K/16].
    """
    x = _f32(x)
    K = x.shape[-1]
    blocks = np.abs(x).reshape(*x.shape[:-1], K // NVFP4_BLOCK, NVFP4_BLOCK)
    amax = blocks.max(axis=-1)
    d = (np.float32(6.0) * _f32(g_a)).astype(np.float32)
    rd = _recip(d)
    t = (amax * rd).astype(np.float32)
    _, tq = e4m3_round(np.clip(t, np.float32(0.0), np.float32(E4M3_MAX)))
    return tq.astype(np.float32)


def fq_nvfp4_act_dynamic(x, g_a) -> FQ:
    """NVFP4 activation fake-quant with dynamic block scales and a frozen g_a."""
    x = _f32(x)
    th = nvfp4_dynamic_theta(x, g_a)
    th_e = np.repeat(th, NVFP4_BLOCK, axis=-1)
    return fq_nvfp4(x, th_e, g_a)


def _expand_groups(a, group: int, K: int):
    """[..., K/group] -> [..., K] by repeating each group's value."""
    a = np.asarray(a)
    assert a.shape[-1] * group == K
    return np.repeat(a, group, axis=-1)


def fq_weight_stack(w_bits, fmt: int, group: int, scale, zero_point=None,
                    global_scale=None) -> FQ:
    """Fake-quantise a stacked weight [E, N, K] (mcore_qad article, section 二.4).

    fmt FMT_NONE: quantization off (the self-teacher), scale unused.
    scale: [E, N, K/group] (NVFP4: theta), or [E] for group GROUP_TENSOR (one
    scale per expert matrix, INT8 / FP8); zero_point: [E, N, K/group] (int4);
    global_scale: [E] (NVFP4 tensor scale g, one per expert, R-8).
    """
    w = bf16_to_f32(w_bits)
    E, N, K = w.shape
    if fmt == FMT_NONE:             # quantization off: the weights as they are
        return fq_act(w_bits, FMT_NONE, None)
    if group == GROUP_TENSOR:
        if fmt not in (FMT_INT8, FMT_FP8):
            raise ValueError("a per-tensor weight scale exists for int8 / fp8 only")
        s = np.broadcast_to(np.asarray(scale, dtype=np.float32).reshape(E, 1, 1), (E, N, K))
        return fq_int8(w, s) if fmt == FMT_INT8 else fq_fp8(w, s)
    assert K % group == 0
    s = _expand_groups(np.asarray(scale, dtype=np.float32).reshape(E, N, K // group), group, K)
    if fmt == FMT_INT8:
        return fq_int8(w, s)
    if fmt == FMT_FP8:
        return fq_fp8(w, s)
    if fmt == FMT_INT4:
        zp = _expand_groups(np.asarray(zero_point, dtype=np.float32).reshape(E, N, K // group),
                            group, K)
        return fq_int4(w, s, zp)
    if fmt == FMT_NVFP4:
        g = np.asarray(global_scale, dtype=np.float32).reshape(E, 1, 1)
        return fq_nvfp4(w, s, g)
    raise ValueError(f"unsupported weight format {fmt}")


def fq_act(x_bits, fmt: int, scale) -> FQ:
    """Activation fake-quant before the matmul (forward pre-hook, mcore_qad article
    section 二.3). FP8: frozen per-tensor scale; NVFP4: dynamic 16-blocks with a
    frozen tensor scale g_a; NONE: identity with mask 1."""
    x = bf16_to_f32(x_bits)
    if fmt == FMT_NONE:
        return FQ(code=np.zeros(x.shape, np.int64), q=x.astype(np.float64), v=x,
                  bits=np.asarray(x_bits, dtype=np.uint16).copy(), z=x,
                  mask=np.ones(x.shape, bool), dv_ds=np.zeros(x.shape))
    s = np.float32(np.asarray(scale, dtype=np.float32).reshape(-1)[0])
    if fmt == FMT_FP8:
        return fq_fp8(x, s)
    if fmt == FMT_NVFP4:
        return fq_nvfp4_act_dynamic(x, s)
    if fmt == FMT_INT8:
        return fq_int8(x, s)
    raise ValueError(f"unsupported activation format {fmt}")
