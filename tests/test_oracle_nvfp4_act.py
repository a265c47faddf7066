"""Pins of the oracle's NVFP4 activation quantizer with dynamic block scales.

The activation side of the nvfp4 preset (AngelSlim mcore_qad article, section
三) takes each 16-element block's scale from the data of the step, the
"dynamic" scale source of section 六, under a frozen per-tensor scale g_a set
by calibration (the QAT + ZeRO-3 page's lazy activation-scale init). Reading
R-8: theta_b = e4m3(clamp(amax_b * (1/(6 g_a)), 0, 448)), s_b = theta_b * g_a,
then the E2M1 codec on z = x * (1/s_b).

Each test checks the oracle against something it does not share code with:
torch's float8_e4m3fn cast, the already pinned weight observer, closed forms
on constructed inputs, or a brute-force nearest-grid-point search. CPU only.
"""
import numpy as np
import pytest
import torch

import oracle as O

E2M1_GRID = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def _bf16(a):
    return O.f32_to_bf16(np.asarray(a, dtype=np.float32))


def _torch_theta(x_bits, g_a):
    """theta per 16-block written with torch fp32 ops and torch's E4M3 cast."""
    x = torch.from_numpy(O.bf16_to_f32(x_bits).copy())
    T, K = x.shape
    amax = x.abs().reshape(T, K // 16, 16).amax(dim=-1)
    g = torch.tensor(g_a, dtype=torch.float32)
    rd = torch.tensor(1.0, dtype=torch.float32) / (torch.tensor(6.0, dtype=torch.float32) * g)
    t = (amax * rd).clamp(0.0, 448.0)
    return t.to(torch.float8_e4m3fn).to(torch.float32).numpy(), (amax * rd).numpy()


def _heavy_tailed(T, K, seed):
    """Blocks of very different magnitude, so thetas cover much of the E4M3 range."""
    rng = np.random.default_rng(seed)
    mag = np.exp(rng.uniform(-10.0, 3.0, size=(T, K // 16, 1))).astype(np.float32)
    x = rng.standard_normal((T, K // 16, 16)).astype(np.float32) * mag
    return _bf16(x.reshape(T, K))


def test_dynamic_theta_equals_weight_observer():
    """With g_a from the activation observer, the dynamic thetas of a [T, K]
    tensor are the weight observer's thetas of the same data as one [1, T, K]
    expert (same rule, pinned there by closed forms)."""
    x = _heavy_tailed(24, 128, seed=1)
    g_a = O.observer_act(x, O.FMT_NVFP4)
    th = O.nvfp4_dynamic_theta(O.bf16_to_f32(x), g_a)
    th_w, _, g_w = O.observer_weight(x.reshape(1, 24, 128), O.FMT_NVFP4, 16)
    assert g_w[0] == g_a
    assert th.shape == (24, 8)
    assert np.array_equal(th, th_w[0])


@pytest.mark.parametrize("g_scale", [1.0, 1e-2, 3e-4])
def test_dynamic_theta_matches_torch_e4m3_cast(g_scale):
    """Dense sweep against torch: amax over 16 contiguous elements along K,
    times the fp32 reciprocal of 6 g_a, clamped to [0, 448], cast by torch to
    float8_e4m3fn. Small g_a forces the 448 clamp on many blocks."""
    x = _heavy_tailed(64, 256, seed=2)
    g_a = np.float32(O.observer_act(x, O.FMT_NVFP4) * np.float32(g_scale))
    th = O.nvfp4_dynamic_theta(O.bf16_to_f32(x), g_a)
    ref, t_raw = _torch_theta(x, g_a)
    assert np.array_equal(th, ref)
    if g_scale < 1.0:
        sat = t_raw > 448.0
        assert sat.any() and np.all(th[sat] == 448.0)
    # the unclamped sweep exercises many grid values, subnormals included
    if g_scale == 1.0:
        assert len(np.unique(th)) > 40 and np.any((th > 0) & (th < 2.0 ** -6))


def _div_vs_mul_cases(n_want=8):
    """(amax bf16 bits, g_a) pairs where amax * (1/(6 g)) and amax / (6 g)
    round to different E4M3 values: g is tuned so that the product lands
    within one ulp of an E4M3 rounding midpoint."""
    pos = torch.arange(0, 127, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    mids = ((pos[1:].astype(np.float64) + pos[:-1]) / 2).astype(np.float32)
    mids = mids[(mids > 8) & (mids < 400)][::3]
    rng = np.random.default_rng(0)
    bits = np.arange(0x3D80, 0x4080, dtype=np.uint32)
    A = (bits << 16).view(np.float32)
    out = []
    for M in mids:
        a_i = rng.choice(len(A), 64, replace=False)
        a = A[a_i]
        g0 = (a / np.float32(6.0) / M).astype(np.float32)
        gs = [g0]
        up, dn = g0, g0
        for _ in range(6):
            up = np.nextafter(up, np.float32(np.inf), dtype=np.float32)
            dn = np.nextafter(dn, np.float32(-np.inf), dtype=np.float32)
            gs += [up, dn]
        for g in gs:
            d = (np.float32(6.0) * g).astype(np.float32)
            tm = (a * (np.float32(1.0) / d).astype(np.float32)).astype(np.float32)
            td = (a / d).astype(np.float32)
            em = torch.from_numpy(tm).to(torch.float8_e4m3fn).float().numpy()
            ed = torch.from_numpy(td).to(torch.float8_e4m3fn).float().numpy()
            for i in np.nonzero(em != ed)[0]:
                out.append((int(bits[a_i[i]]), np.float32(g[i])))
        if len(out) >= n_want:
            return out[:n_want]
    return out


def test_dynamic_theta_uses_reciprocal_product():
    """R-1: the block amax is multiplied by the once-rounded reciprocal of
    6 g_a. On inputs where dividing instead moves an E4M3 rounding decision,
    the oracle follows the product form."""
    cases = _div_vs_mul_cases()
    assert len(cases) >= 4
    for abits, g in cases:
        row = np.zeros(32, np.float32)
        a = O.bf16_to_f32(np.array([abits], np.uint16))[0]
        row[5] = -a                       # the amax, negative, mid-block
        row[:16] += np.linspace(-0.5, 0.5, 16, dtype=np.float32) * a
        row[5] = -a
        row[16:] = a / 4
        x = _bf16(row[None, :])
        th = O.nvfp4_dynamic_theta(O.bf16_to_f32(x), g)
        ref, _ = _torch_theta(x, g)
        assert np.array_equal(th, ref)
        d = np.float32(np.float32(6.0) * g)
        alt = torch.from_numpy(np.array([a / d], np.float32)).to(torch.float8_e4m3fn).float().item()
        assert th[0, 0] != alt


def test_tensor_amax_block_gets_448_and_code_six():
    """With g_a = amax/2688 from calibration on the same tensor, the block that
    holds the tensor's amax gets theta = 448 and that element quantizes to the
    E2M1 end point +-6 (code 7 or 15)."""
    x = _heavy_tailed(32, 128, seed=3)
    xf = O.bf16_to_f32(x)
    g_a = O.observer_act(x, O.FMT_NVFP4)
    th = O.nvfp4_dynamic_theta(xf, g_a)
    t, k = np.unravel_index(np.argmax(np.abs(xf)), xf.shape)
    assert th[t, k // 16] == 448.0
    fq = O.fq_act(x, O.FMT_NVFP4, g_a)
    assert abs(fq.q[t, k]) == 6.0
    assert fq.code[t, k] in (7, 15)
    assert (fq.code[t, k] == 15) == (xf[t, k] < 0)


def test_zero_blocks_give_positive_zero_and_mask_zero():
    x = _heavy_tailed(4, 64, seed=4)
    xf = O.bf16_to_f32(x).copy()
    xf[1, 16:32] = 0.0
    xf[2, 48:64] = -0.0
    x = _bf16(xf)
    g_a = O.observer_act(x, O.FMT_NVFP4)
    th = O.nvfp4_dynamic_theta(O.bf16_to_f32(x), g_a)
    assert th[1, 1] == 0.0 and th[2, 3] == 0.0
    fq = O.fq_act(x, O.FMT_NVFP4, g_a)
    for t, sl in ((1, slice(16, 32)), (2, slice(48, 64))):
        assert np.all(fq.bits[t, sl] == 0)          # +0.0, also for -0.0 inputs
        assert not fq.mask[t, sl].any()
        assert np.all(fq.code[t, sl] == 0)
    # a zero block leaves the other blocks of its row as they are
    assert np.array_equal(fq.bits[0], O.fq_act(x[0:1], O.FMT_NVFP4, g_a).bits[0])


def test_blocks_run_along_the_contraction_axis():
    """x[t, k] = (t+1) * (k%16 + 1) / 64: every 16-block of row t along K has
    amax (t+1)/4. With g_a = 1/24, 1/(6 g_a) = 4 exactly and theta = t+1,
    on the E4M3 grid for t < 16. Blocks taken across rows would not give this."""
    T, K = 16, 64
    t = np.arange(T, dtype=np.float32)[:, None]
    k = np.arange(K, dtype=np.float32)[None, :]
    x = _bf16((t + 1) * (k % 16 + 1) / 64)
    g_a = np.float32(1.0) / np.float32(24.0)
    assert np.float32(np.float32(1.0) / np.float32(np.float32(6.0) * g_a)) == np.float32(4.0)
    th = O.nvfp4_dynamic_theta(O.bf16_to_f32(x), g_a)
    assert np.array_equal(th, np.repeat(np.arange(1, T + 1, dtype=np.float32)[:, None], K // 16, 1))


def test_activation_values_brute_force():
    """Every output element against a nearest-grid-point search in float64
    (ties to the even code), with the block scale from torch's E4M3 cast."""
    x = _heavy_tailed(4, 64, seed=5)
    xf = O.bf16_to_f32(x)
    g_a = O.observer_act(x, O.FMT_NVFP4)
    th_ref, _ = _torch_theta(x, g_a)
    fq = O.fq_act(x, O.FMT_NVFP4, g_a)
    for ti in range(4):
        for ki in range(64):
            s = np.float32(np.float32(th_ref[ti, ki // 16]) * g_a)
            if s == 0:
                assert fq.bits[ti, ki] == 0
                continue
            z = float(np.float32(xf[ti, ki] * np.float32(np.float32(1.0) / s)))
            a = min(abs(z), 6.0)
            best_i = 0
            for i, val in enumerate(E2M1_GRID):
                d, d_best = abs(a - val), abs(a - E2M1_GRID[best_i])
                if d < d_best or (d == d_best and i % 2 == 0):
                    best_i = i
            val = np.copysign(E2M1_GRID[best_i], z)      # minifloat codes keep the sign (R-2)
            assert fq.code[ti, ki] == best_i | (8 if np.signbit(z) else 0)
            assert fq.q[ti, ki] == val and np.signbit(fq.q[ti, ki]) == np.signbit(val)
            v = np.float32(np.float32(val) * s)
            assert fq.bits[ti, ki] == O.f32_to_bf16(np.array([v]))[0]
            assert fq.mask[ti, ki] == (-6.0 <= z <= 6.0)
