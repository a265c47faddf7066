"""Pins of the oracle's real-quantized export and decode.

(i) decode(pack(codes), stored scales) reproduces the fake-quant values bit
for bit, for every format and scale granularity, with saturated elements,
zero NVFP4 blocks, block parameters above the E4M3 maximum and signed zeros.
(ii) Byte layout: int8 two's complement, even element in the low nibble.
(iii) E4M3 block-scale bytes of values whose encoding the OCP MX v1.0
definition fixes (bias 7, 3 mantissa bits, subnormals m * 2^-9).
(iv) Exhaustive NVFP4 decode: every E2M1 nibble under every finite positive
E4M3 scale byte at a power-of-two tensor scale equals the product of the
two table values.
CPU only."""
import numpy as np
import pytest

import oracle as O


def _w(rng, E, N, K, std=0.02):
    w = rng.standard_normal((E, N, K)).astype(np.float32) * std
    flat = w.reshape(-1)
    idx = rng.choice(flat.size, flat.size // 100, replace=False)
    flat[idx] *= 30.0                                     # saturating outliers
    flat[idx[: len(idx) // 4]] = -1e-9                    # tiny negatives -> signed zeros
    return O.f32_to_bf16(w)


CASES = [(O.FMT_INT8, 64), (O.FMT_INT8, O.GROUP_TENSOR), (O.FMT_FP8, 128), (O.FMT_FP8, 256),
         (O.FMT_FP8, O.GROUP_TENSOR), (O.FMT_INT4, 128), (O.FMT_INT4, 32), (O.FMT_NVFP4, 16)]


@pytest.mark.parametrize("fmt,group", CASES)
def test_decode_of_export_is_the_fake_quant_value(fmt, group):
    rng = np.random.default_rng(40 + fmt)
    E, N, K = 3, 8, 256
    w = _w(rng, E, N, K)
    s, zp, g = O.observer_weight(w, fmt, group)
    s = (s * rng.uniform(0.4, 1.1, s.shape)).astype(np.float32)
    if fmt == O.FMT_NVFP4:
        s[0, 0, :3] = 0.0                                 # zero blocks
        s[1, 2, 1] = 700.0                                # theta above the E4M3 max
    if fmt == O.FMT_INT4:
        zp = zp.copy()
        zp[0, 0, 0] = 20.0                                # clamped to 15 on export
    fq = O.fq_weight_stack(w, fmt, group, s, zp, g)
    packed = O.pack_codes(fq.code, fmt)
    s32, sbytes, zbytes = O.export_scales(fmt, s, zp)
    out = O.dequantize(packed, fmt, group, (E, N, K), s32, sbytes, zbytes, g)
    assert np.array_equal(out, fq.bits)
    if fmt in (O.FMT_FP8, O.FMT_NVFP4):
        assert np.any(out == 0x8000)                      # minifloats keep -0
    assert np.array_equal(O.unpack_codes(packed, fmt, fq.code.size).reshape(fq.code.shape),
                          fq.code)


def test_byte_layout():
    # 4-bit codes: element 2i in the low nibble of byte i
    assert list(O.pack_codes([1, 2, 3, 4, 0xF, 0x8], O.FMT_NVFP4)) == [0x21, 0x43, 0x8F]
    assert list(O.unpack_codes(np.array([0x21, 0x43, 0x8F], np.uint8), O.FMT_INT4, 6)) == \
        [1, 2, 3, 4, 0xF, 0x8]
    # int8: two's complement bytes
    assert list(O.pack_codes([-128, -1, 0, 1, 127], O.FMT_INT8)) == [0x80, 0xFF, 0x00, 0x01, 0x7F]
    assert list(O.unpack_codes(np.array([0x80, 0xFF, 0x7F], np.uint8), O.FMT_INT8, 3)) == \
        [-128, -1, 127]


def test_e4m3_block_scale_bytes():
    theta = np.array([448.0, 1.0, 0.75, 2.0 ** -9, 0.0, 500.0, -3.0, 3.0 * 2.0 ** -9, 240.0],
                     np.float32)
    _, b, _ = O.export_scales(O.FMT_NVFP4, theta)
    # 448 = 1.75*2^8 -> 0 1111 110; 1 -> 0 0111 000; 0.75 = 1.5*2^-1 -> 0 0110 100;
    # 2^-9 -> smallest subnormal; clamp(500) = 448; clamp(-3) = 0; 3*2^-9 -> subnormal 3;
    # 240 = 1.875*2^7 -> 0 1110 111
    assert list(b) == [0x7E, 0x38, 0x34, 0x01, 0x00, 0x7E, 0x00, 0x03, 0x77]


def test_nvfp4_decode_all_nibbles_all_scale_bytes():
    E, N = 1, 126
    K = 16 * 16
    g = np.float32(2.0 ** -6)
    sbytes = np.repeat(np.arange(126, dtype=np.uint8)[:, None], K // 16, axis=1)[None]  # [1,126,16]
    codes = np.tile(np.arange(16), K // 16 * N).reshape(E, N, K)                  # every nibble
    packed = O.pack_codes(codes, O.FMT_NVFP4)
    out = O.dequantize(packed, O.FMT_NVFP4, 16, (E, N, K), None, sbytes, None, [g])
    mag = O.E2M1_POS[codes & 7] * np.where(codes & 8, -1.0, 1.0)
    ref = mag * O.E4M3_POS[np.arange(126)][None, :, None] * np.float64(g)       # exact in fp32
    assert np.array_equal(O.bf16_to_f32(out).astype(np.float64),
                          O.bf16_to_f32(O.f32_to_bf16(ref.astype(np.float32))).astype(np.float64))
