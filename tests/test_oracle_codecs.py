"""Pins of the oracle's numerics and codecs against what fixes them independently:
library casts (special cases), format definitions (tie tables, code grids),
closed forms and invariants. CPU only."""
import math
import os

import numpy as np
import pytest
import torch

import oracle as O
from oracle import codecs as C

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- bf16 -----
def test_bf16_rne_matches_torch_cast():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(200_000).astype(np.float32) * 10.0 ** rng.integers(-8, 8, 200_000),
        # exact ties: bf16 value + half an ulp
        (O.bf16_to_f32(rng.integers(0, 0x7F00, 50_000, dtype=np.uint16)).view(np.uint32)
         | np.uint32(0x8000)).view(np.float32),
    ]).astype(np.float32)
    ours = O.f32_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_to_f32_exact_roundtrip():
    bits = np.arange(0, 0x7F80, dtype=np.uint16)
    assert np.array_equal(O.f32_to_bf16(O.bf16_to_f32(bits)), bits)
    neg = bits | np.uint16(0x8000)
    assert np.array_equal(O.f32_to_bf16(O.bf16_to_f32(neg)), neg)


# ---------------------------------------------------------------- E4M3 -----
def test_e4m3_grid_matches_torch_float8_definition():
    allc = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    for code in range(256):
        if code & 0x7F == 0x7F:
            assert math.isnan(allc[code])
            continue
        ours = O.e4m3_value_of_code(code)
        assert ours == allc[code] and np.signbit(ours) == np.signbit(allc[code]), code
    assert C.E4M3_POS[126] == 448.0 and C.E4M3_POS[1] == 2.0 ** -9 and C.E4M3_POS[8] == 2.0 ** -6
    assert np.all(np.diff(C.E4M3_POS) > 0)


def _e4m3_sweep():
    rng = np.random.default_rng(2)
    pos = C.E4M3_POS
    mids = (pos[:-1] + pos[1:]) / 2.0                       # exact ties
    near = np.concatenate([mids * (1 + 2.0 ** -20), mids * (1 - 2.0 ** -20)])
    rand = rng.uniform(0, 448, 300_000)
    small = rng.uniform(0, 2.0 ** -5, 100_000)
    a = np.concatenate([pos, mids, near, rand, small]).astype(np.float32)
    return np.concatenate([a, -a])


def test_e4m3_round_matches_torch_cast_dense_sweep():
    z = _e4m3_sweep()
    code, val = O.e4m3_round(z)
    ref = torch.from_numpy(z).to(torch.float8_e4m3fn)
    ref_code = ref.view(torch.uint8).numpy()
    assert np.array_equal(code, ref_code)
    assert np.array_equal(val, ref.double().numpy())


def test_e4m3_saturates():
    code, val = O.e4m3_round(np.array([448.0, 464.0, 1e4, -1e30, -448.0], np.float32))
    assert list(val) == [448.0, 448.0, 448.0, -448.0, -448.0]
    assert list(code) == [0x7E, 0x7E, 0x7E, 0xFE, 0xFE]


def test_e4m3_signed_zero():
    code, val = O.e4m3_round(np.array([-0.0, -2.0 ** -11, 0.0, 2.0 ** -11], np.float32))
    assert list(code) == [0x80, 0x80, 0x00, 0x00]
    assert np.signbit(val[0]) and np.signbit(val[1]) and not np.signbit(val[2])


# ---------------------------------------------------------------- E2M1 -----
def _load_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def test_e2m1_tie_table_golden():
    rows = _load_golden("e2m1_ties.txt")
    z = np.array([float(r[0]) for r in rows], np.float32)
    code, val = O.e2m1_round(z)
    for i, r in enumerate(rows):
        assert val[i] == float(r[1]) and np.signbit(val[i]) == r[1].startswith("-"), r
        assert code[i] == int(r[2]), r


def _e2m1_by_exponent(a: float) -> float:
    """Independent E2M1 rounding: quantum 2^(e-1) with e = clamp(floor(log2 a), 0, 2),
    round half to even on a / quantum, saturate at 6."""
    a = min(abs(a), 6.0)
    if a == 0.0:
        return 0.0
    e = min(max(math.floor(math.log2(a)), 0), 2)
    q = 2.0 ** (e - 1)
    return min(round(a / q) * q, 6.0)      # Python round() is half-to-even


def test_e2m1_round_matches_exponent_form():
    rng = np.random.default_rng(3)
    grid = C.E2M1_POS
    mids = (grid[:-1] + grid[1:]) / 2
    a = np.concatenate([grid, mids, rng.uniform(0, 8, 20_000)]).astype(np.float32)
    _, val = O.e2m1_round(a)
    ref = np.array([_e2m1_by_exponent(float(v)) for v in a])
    assert np.array_equal(val, ref)
    _, valn = O.e2m1_round(-a)
    assert np.array_equal(valn, -ref)


# ---------------------------------------------- exhaustive grid round trip -----
POW2_SCALES = [2.0 ** e for e in range(-12, 5)]


@pytest.mark.parametrize("s", POW2_SCALES)
def test_int8_grid_roundtrip(s):
    c = np.arange(-128, 128, dtype=np.float64)
    x = (c * s).astype(np.float32)
    fq = O.fq_int8(x, np.float32(s))
    assert np.array_equal(fq.code, c.astype(np.int64))
    assert np.array_equal(fq.v, x)
    assert np.all(fq.mask)
    assert np.all(fq.dv_ds == 0)                  # on-grid: rne(z) - z == 0


@pytest.mark.parametrize("s", POW2_SCALES)
def test_int4_grid_roundtrip_every_zero_point(s):
    for zp in range(16):
        c = np.arange(16, dtype=np.float64)
        x = ((c - zp) * s).astype(np.float32)
        fq = O.fq_int4(x, np.float32(s), np.float32(zp))
        assert np.array_equal(fq.code, c.astype(np.int64)), zp
        assert np.array_equal(fq.v, x)
        assert np.all(fq.mask) and np.all(fq.dv_ds == 0) and np.all(fq.dv_dzp == 0)


@pytest.mark.parametrize("s", POW2_SCALES)
def test_e4m3_grid_roundtrip(s):
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F])
    val = O.e4m3_value_of_code(codes)
    x = (val * s).astype(np.float32)
    fq = O.fq_fp8(x, np.float32(s))
    # x * (1/s) is exact for power-of-two s (no underflow in this range)
    assert np.array_equal(fq.code, codes)
    assert np.array_equal(fq.v, x) and np.array_equal(np.signbit(fq.v), np.signbit(val))
    assert np.array_equal(fq.bits, O.f32_to_bf16(x))


@pytest.mark.parametrize("theta,g", [(2.0 ** e, 1.0) for e in range(-9, 9)] +
                         [(1.0, 2.0 ** e) for e in range(-14, 0)])
def test_e2m1_grid_roundtrip(theta, g):
    # theta a power of two on the E4M3 grid (2^-9 .. 2^8) and g a power of two
    # make s_b = theta * g a power of two, so x * (1/s_b) is exact
    s = theta * g
    codes = np.arange(16)
    val = O.e2m1_value_of_code(codes)
    fq = O.fq_nvfp4((val * s).astype(np.float32), np.float32(theta), np.float32(g))
    assert np.array_equal(fq.code, codes)
    assert np.array_equal(fq.v, (val * s).astype(np.float32))
    assert np.array_equal(np.signbit(fq.v), np.signbit(val))
    assert np.all(fq.dv_ds == 0)


# ------------------------------------------------------------ idempotence -----
@pytest.mark.parametrize("fmt", ["int8", "int4", "fp8", "nvfp4"])
def test_fake_quant_idempotent(fmt):
    rng = np.random.default_rng(4)
    E, N, K = 2, 8, 256
    w = O.f32_to_bf16(rng.standard_normal((E, N, K)).astype(np.float32) * 0.02)
    group = {"int8": K, "int4": 128, "fp8": K, "nvfp4": 16}[fmt]
    f = O.FMT_NAMES[fmt]
    s, zp, g = O.observer_weight(w, f, group)
    once = O.fq_weight_stack(w, f, group, s, zp, g)
    twice = O.fq_weight_stack(once.bits, f, group, s, zp, g)
    assert np.array_equal(once.bits, twice.bits)
    assert np.array_equal(once.code, twice.code)


def test_fp8_activation_fq_idempotent_fixed_scale():
    rng = np.random.default_rng(5)
    x = O.f32_to_bf16(rng.standard_normal((16, 64)).astype(np.float32))
    s = O.observer_act(x, O.FMT_FP8)
    once = O.fq_act(x, O.FMT_FP8, s)
    assert np.array_equal(O.fq_act(once.bits, O.FMT_FP8, s).bits, once.bits)


# ------------------------------------------------------------- saturation -----
def test_saturation_masks_and_scale_grads():
    s = np.float32(0.5)
    for big, sign in ((1e4, 1.0), (-1e4, -1.0)):
        x = np.float32(big * s)
        f8 = O.fq_int8(x, s)
        assert not f8.mask and f8.dv_ds == (127.0 if sign > 0 else -128.0)
        ff = O.fq_fp8(x, s)
        assert not ff.mask and ff.dv_ds == 448.0 * sign
        f4 = O.fq_int4(x, s, np.float32(3.0))
        assert not f4.mask and f4.dv_ds == (12.0 if sign > 0 else -3.0) and f4.dv_dzp == -0.5
        fn = O.fq_nvfp4(x, np.float32(0.5), np.float32(1.0))
        assert not fn.mask and fn.dv_ds == 6.0 * sign


def test_mask_bounds_inclusive_on_unrounded_z():
    s = np.float32(1.0)
    f = O.fq_int8(np.array([127.0, 127.25, -128.0, -128.25], np.float32), s)
    assert list(f.mask) == [True, False, True, False]
    f = O.fq_fp8(np.array([448.0, 448.5], np.float32), s)
    assert list(f.mask) == [True, False]


# ------------------------------------------------------------ signed zero -----
def test_signed_zero_rule():
    s = np.float32(1.0)
    assert not np.signbit(O.fq_int8(np.float32(-0.3), s).v)       # int: +0.0
    assert not np.signbit(O.fq_int4(np.float32(-0.3), s, np.float32(0)).v)
    assert np.signbit(O.fq_fp8(np.float32(-2.0 ** -12), s).v)      # fp: keeps sign
    assert np.signbit(O.fq_nvfp4(np.float32(-0.1), np.float32(1.0), np.float32(1.0)).v)


# ----------------------------------------------------- NVFP4 block scale -----
def test_nvfp4_zero_block_scale_outputs_positive_zero():
    x = np.array([1.0, -2.0, 3.0], np.float32)
    for th in (0.0, 2.0 ** -11, -1.0):
        f = O.fq_nvfp4(x, np.float32(th), np.float32(1.0))
        assert np.all(f.v == 0) and not np.any(np.signbit(f.v))
        assert not np.any(f.mask) and np.all(f.dv_ds == 0)


def test_nvfp4_theta_rerounded_to_e4m3():
    # theta = 0.3 is off the E4M3 grid: s_b = e4m3(0.3) * g
    _, tq = O.e4m3_round(np.float32(0.3))
    f = O.fq_nvfp4(np.float32(1.0), np.float32(0.3), np.float32(2.0))
    assert f.s == np.float32(tq * 2.0)
    # theta above 448 saturates and stops the gradient
    f = O.fq_nvfp4(np.float32(100.0), np.float32(500.0), np.float32(1.0))
    assert f.s == 448.0 and f.dv_ds == 0.0


# ---------------------------------------------- library special cases -----
def test_int8_int4_forward_match_torch_fake_quantize():
    """torch.fake_quantize_per_channel_affine computes nearbyint(x * (1/s)) + zp,
    clamps, and dequantises: the same rule (R-1) on the integer grids."""
    rng = np.random.default_rng(6)
    N, K = 64, 256
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    w[0, :7] = [0.0, -0.0, 1e-8, -1e-8, 0.3, -0.3, 5.0]
    s8 = (np.abs(w).max(axis=1) / 127).astype(np.float32) * np.float32(0.7)   # some saturation
    ref = torch.fake_quantize_per_channel_affine(
        torch.from_numpy(w), torch.from_numpy(s8), torch.zeros(N, dtype=torch.int32), 0, -128, 127)
    ours = O.fq_int8(w, s8[:, None])
    assert np.array_equal(ours.v, ref.numpy())
    s4 = (np.float32(0.01) + rng.random(N).astype(np.float32) * np.float32(0.004)).astype(np.float32)
    zp = rng.integers(0, 16, N)
    ref4 = torch.fake_quantize_per_channel_affine(
        torch.from_numpy(w), torch.from_numpy(s4), torch.from_numpy(zp.astype(np.int32)), 0, 0, 15)
    ours4 = O.fq_int4(w, s4[:, None], zp[:, None].astype(np.float32))
    assert np.array_equal(ours4.v, ref4.numpy())
