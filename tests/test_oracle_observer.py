"""Pins of the oracle's scale initialisation (observer) by closed forms. CPU only."""
import numpy as np
import pytest

import oracle as O


def _w(E, N, K, seed=0, std=0.02):
    rng = np.random.default_rng(seed)
    return O.f32_to_bf16((rng.standard_normal((E, N, K)) * std).astype(np.float32))


def test_int8_absmax_element_maps_to_127():
    w = _w(3, 16, 64)
    s, zp, g = O.observer_weight(w, O.FMT_INT8, 64)
    assert zp is None and g is None and s.shape == (3, 16, 1)
    x = O.bf16_to_f32(w)
    amax = np.abs(x).max(axis=-1)
    # s*127 == amax within one ulp of s
    assert np.all(np.abs(s[..., 0].astype(np.float64) * 127 - amax) <= 127 * np.spacing(s[..., 0]))
    fq = O.fq_weight_stack(w, O.FMT_INT8, 64, s)
    am = np.abs(x) == amax[..., None]
    assert np.all(np.abs(fq.code[am]) == 127)
    # z of the amax element is 127 up to the rounding of s and 1/s
    assert np.all(np.abs(np.abs(fq.z[am]) - 127.0) <= 127.0 * 2.0 ** -22)
    assert np.all(fq.mask[~am])


def test_fp8_absmax_is_448_and_matches_ptq_closed_form():
    # PTQ weight scale = max|W| / 448 (QAT + ZeRO-3 page, "Quantizer 初始值")
    w = _w(2, 8, 128, seed=1)
    s, _, _ = O.observer_weight(w, O.FMT_FP8, 128)
    x = O.bf16_to_f32(w)
    amax = np.abs(x).max(axis=-1).astype(np.float32)
    assert np.array_equal(s[..., 0], (amax / np.float32(448)).astype(np.float32))
    fq = O.fq_weight_stack(w, O.FMT_FP8, 128, s)
    am = np.abs(x) == amax[..., None]
    assert np.all(np.abs(O.e4m3_value_of_code(fq.code[am])) == 448)


def test_per_group_fp8_int8():
    w = _w(1, 4, 256, seed=2)
    s, _, _ = O.observer_weight(w, O.FMT_INT8, 64)
    x = O.bf16_to_f32(w).reshape(1, 4, 4, 64)
    assert np.array_equal(s, (np.abs(x).max(-1) / np.float32(127)).astype(np.float32))


def test_int4_minmax_range_contains_zero():
    w = _w(2, 8, 256, seed=3)
    # a group with only positive values and one with only negatives
    x = O.bf16_to_f32(w).copy()
    x[0, 0, :128] = np.abs(x[0, 0, :128]) + 0.01
    x[0, 1, 128:] = -np.abs(x[0, 1, 128:]) - 0.01
    w = O.f32_to_bf16(x)
    s, zp, _ = O.observer_weight(w, O.FMT_INT4, 128)
    blk = O.bf16_to_f32(w).reshape(2, 8, 2, 128)
    lo = np.minimum(blk.min(-1), 0)
    hi = np.maximum(blk.max(-1), 0)
    assert np.all(lo <= 0) and np.all(hi >= 0)
    assert np.all(np.abs(s.astype(np.float64) * 15 - (hi - lo)) <= 15 * np.spacing(s))
    assert np.all((zp >= 0) & (zp <= 15) & (zp == np.rint(zp)))
    assert zp[0, 0, 0] == 0            # all positive: lo = 0
    assert zp[0, 1, 1] == 15           # all negative: hi = 0
    # zero is exactly representable: x = 0 dequantises to 0
    fq = O.fq_int4(np.zeros((2, 8, 2), np.float32), s, zp)
    assert np.all(fq.v == 0)
    # rounding zp shifts the window [-zp, 15-zp] by at most half a step from
    # [lo/s, hi/s], so no element lies more than half a step outside it
    full = O.fq_weight_stack(w, O.FMT_INT4, 128, s, zp)
    zpe = np.repeat(zp, 128, -1)
    out = np.maximum(-zpe - full.z, full.z - (15 - zpe))
    assert np.all(out <= 0.5 + 1e-5)


def test_nvfp4_theta_on_grid_and_bounded():
    w = _w(3, 8, 64, seed=4)
    th, _, g = O.observer_weight(w, O.FMT_NVFP4, 16)
    assert th.shape == (3, 8, 4) and g.shape == (3,)
    x = O.bf16_to_f32(w)
    assert np.array_equal(g, (np.abs(x).reshape(3, -1).max(-1) / np.float32(2688)).astype(np.float32))
    _, tq = O.e4m3_round(th)
    assert np.array_equal(tq.astype(np.float32), th)       # on the E4M3 grid
    assert np.all((th >= 0) & (th <= 448))
    # the expert's largest block gets theta = e4m3(448 * (1 +- 1ulp)) = 448
    amax_b = np.abs(x).reshape(3, 8, 4, 16).max(-1)
    for e in range(3):
        i = np.unravel_index(np.argmax(amax_b[e]), amax_b[e].shape)
        assert th[e][i] == 448.0


def test_all_zero_gets_unit_scale():
    w = np.zeros((1, 2, 32), np.uint16)
    for fmt, grp in ((O.FMT_INT8, 32), (O.FMT_FP8, 32), (O.FMT_INT4, 32)):
        s, zp, _ = O.observer_weight(w, fmt, grp)
        assert np.all(s == 1.0)
    th, _, g = O.observer_weight(w, O.FMT_NVFP4, 16)
    assert np.all(g == 1.0) and np.all(th == 0.0)


@pytest.mark.parametrize("fmt,div", [(O.FMT_FP8, 448.0), (O.FMT_NVFP4, 2688.0), (O.FMT_INT8, 127.0)])
def test_activation_per_tensor(fmt, div):
    rng = np.random.default_rng(5)
    x = O.f32_to_bf16(rng.standard_normal((32, 64)).astype(np.float32))
    s = O.observer_act(x, fmt)
    assert s == np.float32(np.abs(O.bf16_to_f32(x)).max() / np.float32(div))


@pytest.mark.parametrize("fmt,top", [(O.FMT_FP8, 448.0), (O.FMT_INT8, 127.0)])
def test_per_tensor_weight_scale_is_matrix_amax(fmt, top):
    """Per-tensor weights: one scale per expert matrix, the matrix's amax over
    the grid maximum; exactly the amax elements reach the top code."""
    w = _w(3, 8, 64, seed=5)
    s, zp, g = O.observer_weight(w, fmt, O.GROUP_TENSOR)
    x = O.bf16_to_f32(w)
    amax = np.abs(x).reshape(3, -1).max(axis=1).astype(np.float32)
    assert zp is None and g is None
    assert np.array_equal(s, (amax / np.float32(top)).astype(np.float32))
    fq = O.fq_weight_stack(w, fmt, O.GROUP_TENSOR, s)
    am = np.abs(x) == amax[:, None, None]
    assert np.all(np.abs(fq.q[am]) == top)
    assert np.all(np.abs(fq.q[~am]) <= top)
