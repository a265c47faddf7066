"""Real-quantized export of a fake-quantized weight stack, and its decode
(test infrastructure only).

What it is (QAT + ZeRO-3 page, sections on convert / save: ``convert()``
turns each quantized linear into a quantize-dequantize module that keeps the
quantized weight with its weight scale and input scale, and
``save_format=real`` writes those compressed tensors; mcore_qad article,
section 三: each format's stored layout is the deployment side's). For a
stack [E, N, K] the stored tensors are
  int8  : codes int8 [E, N, K] (one byte, two's complement), scale fp32
  fp8   : codes E4M3 [E, N, K] (one byte), scale fp32
  int4  : codes uint4 [E, N, K/2] (two per byte, even k in the low nibble),
          scale fp32 [E, N, K/group], zero point uint8 [E, N, K/group]
  nvfp4 : codes E2M1 [E, N, K/2] (two per byte, even k low, sign in bit 3),
          block scale E4M3 bytes [E, N, K/16], tensor scale fp32 [E]
and decoding them gives back exactly the fake-quant values: v = fp32(value(c)
* s) with s the group scale (int4: value = code - zero point; nvfp4: s =
fp32(e4m3 value(block byte) * g)), then bf16.
"""
from __future__ import annotations

import numpy as np

from .codecs import (E4M3_MAX, FMT_FP8, FMT_INT4, FMT_INT8, FMT_NVFP4, GROUP_TENSOR,
                     INT4_HI, INT4_LO, e4m3_round, e4m3_value_of_code, e2m1_value_of_code)
from .numerics import f32_to_bf16


def pack_codes(code, fmt: int) -> np.ndarray:
    """Codes as stored, flattened: one byte per element (int8 two's complement,
    E4M3 byte) or two 4-bit codes per byte with the even element in the low
    nibble (int4, E2M1)."""
    c = np.asarray(code, dtype=np.int64).reshape(-1)
    if fmt in (FMT_INT8, FMT_FP8):
        return (c & 0xFF).astype(np.uint8)
    if fmt in (FMT_INT4, FMT_NVFP4):
        assert c.size % 2 == 0
        c = (c & 0xF).astype(np.uint8)
        return (c[0::2] | (c[1::2] << 4)).astype(np.uint8)
    raise ValueError(f"no codes for format {fmt}")


def unpack_codes(packed, fmt: int, n: int) -> np.ndarray:
    """The n codes of a packed byte array (inverse of pack_codes): int8 codes
    as signed integers, E4M3 bytes and 4-bit codes as unsigned."""
    b = np.asarray(packed, dtype=np.uint8).reshape(-1)
    if fmt == FMT_INT8:
        return b[:n].view(np.int8).astype(np.int64)
    if fmt == FMT_FP8:
        return b[:n].astype(np.int64)
    if fmt in (FMT_INT4, FMT_NVFP4):
        out = np.empty(2 * b.size, dtype=np.int64)
        out[0::2] = b & 0xF
        out[1::2] = b >> 4
        return out[:n]
    raise ValueError(f"no codes for format {fmt}")


def export_scales(fmt: int, scale, zero_point=None):
    """The quantizer parameters in their stored form.

    nvfp4: the block scale byte, E4M3 code of clamp(theta, 0, 448) (the same
           rounding the forward applies to theta, R-8);
    int4 : the zero point byte clamp(rne(zp), 0, 15) (R-5);
    int8 / fp8: the fp32 scale is stored as is (returned unchanged).
    Returns (scale_fp32 or None, scale_bytes or None, zero_point_bytes or None).
    """
    if fmt == FMT_NVFP4:
        th = np.clip(np.asarray(scale, dtype=np.float32), np.float32(0.0), np.float32(E4M3_MAX))
        code, _ = e4m3_round(th)
        return None, code.astype(np.uint8), None
    if fmt == FMT_INT4:
        zp = np.clip(np.rint(np.asarray(zero_point, dtype=np.float64)), INT4_LO, INT4_HI)
        return np.asarray(scale, dtype=np.float32), None, zp.astype(np.uint8)
    if fmt in (FMT_INT8, FMT_FP8):
        return np.asarray(scale, dtype=np.float32), None, None
    raise ValueError(f"no export for format {fmt}")


def _value_of_code(code, fmt: int) -> np.ndarray:
    if fmt == FMT_INT8:
        return code.astype(np.float64)
    if fmt == FMT_FP8:
        return e4m3_value_of_code(code)
    if fmt == FMT_NVFP4:
        return e2m1_value_of_code(code)
    raise ValueError(fmt)


def dequantize(packed, fmt: int, group: int, shape, scale=None, scale_bytes=None,
               zero_point_bytes=None, global_scale=None) -> np.ndarray:
    """bf16 bits [E, N, K] decoded from the stored tensors.

    group: elements per scale along K (int4 / int8 / fp8), 16 for nvfp4, or
    GROUP_TENSOR (int8 / fp8: one fp32 scale per expert matrix)."""
    E, N, K = shape
    code = unpack_codes(packed, fmt, E * N * K).reshape(E, N, K)
    if fmt == FMT_NVFP4:
        th = e4m3_value_of_code(np.asarray(scale_bytes, dtype=np.int64)).astype(np.float32)
        g = np.asarray(global_scale, dtype=np.float32).reshape(E, 1, 1)
        s_b = (th.reshape(E, N, K // 16) * g).astype(np.float32)          # one fp32 rounding (R-8)
        s = np.repeat(s_b, 16, axis=-1)
        q = _value_of_code(code, fmt)
    elif fmt == FMT_INT4:
        G = K // group
        s = np.repeat(np.asarray(scale, dtype=np.float32).reshape(E, N, G), group, axis=-1)
        zp = np.repeat(np.asarray(zero_point_bytes, dtype=np.int64).reshape(E, N, G), group, axis=-1)
        q = (code - zp).astype(np.float64) + 0.0
    else:
        if group == GROUP_TENSOR:
            s = np.broadcast_to(np.asarray(scale, dtype=np.float32).reshape(E, 1, 1), (E, N, K))
        else:
            G = K // group
            s = np.repeat(np.asarray(scale, dtype=np.float32).reshape(E, N, G), group, axis=-1)
        q = _value_of_code(code, fmt)
    v = (q.astype(np.float32) * s).astype(np.float32)
    return f32_to_bf16(v)

