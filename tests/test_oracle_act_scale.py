"""Pins of the oracle's learnable activation-scale gradient (act_scale_grad).

(i) Torch CPU autograd of the written-out per-tensor fake quant with a
straight-through round (torch.round, the float8 cast) and the scale as a leaf.
(ii) Library special case: torch's learnable per-tensor fake quant (INT8, zero
point 0) away from the clamp bounds.
(iii) Activations on the grid at a power-of-two scale give exactly 0.
(iv) All-saturated activations give sum(g) * bound per sign.
CPU only."""
import numpy as np
import pytest
import torch

import oracle as O


def _ste(u, rounded):
    return u + (rounded - u).detach()


def _torch_fq_act(x, fmt, s):
    """Differentiable per-tensor FQ in fp32; s a one-element leaf."""
    z = x * (1.0 / s)
    if fmt == O.FMT_INT8:
        zc = z.clamp(-128.0, 127.0)
        return _ste(zc, torch.round(zc.detach())) * s
    zc = z.clamp(-448.0, 448.0)
    return _ste(zc, zc.detach().to(torch.float8_e4m3fn).to(torch.float32)) * s


def _act(rng, shape, std=1.0):
    return O.f32_to_bf16((rng.standard_normal(shape) * std).astype(np.float32))


@pytest.mark.parametrize("fmt,bound", [(O.FMT_FP8, 448.0), (O.FMT_INT8, 127.0)])
def test_act_scale_grad_matches_torch_autograd(fmt, bound):
    rng = np.random.default_rng(21)
    x = _act(rng, (37, 96))
    xv = O.bf16_to_f32(x)
    # about 3 % of the elements past the range, so both STE branches contribute
    s = np.float32(np.quantile(np.abs(xv), 0.97) / bound)
    g = rng.standard_normal(x.shape)
    ours = O.act_scale_grad(x, g, fmt, s)
    st = torch.tensor([s], dtype=torch.float32, requires_grad=True)
    v = _torch_fq_act(torch.from_numpy(xv.copy()), fmt, st)
    assert np.array_equal(O.f32_to_bf16(v.detach().numpy()), O.fq_act(x, fmt, s).bits)
    (v.double() * torch.from_numpy(g)).sum().backward()
    ref = float(st.grad[0])
    # torch sums the per-element terms into the fp32 leaf: normwise 1e-5
    terms = np.abs(g * O.fq_act(x, fmt, s).dv_ds).sum()
    assert abs(ours - ref) <= 1e-5 * terms
    assert ours != 0.0


def test_int8_act_scale_grad_matches_torch_learnable_per_tensor_fake_quant():
    """Away from the clamp bounds torch's learnable per-tensor affine fake quant
    (zero point 0) uses the same straight-through scale gradient."""
    rng = np.random.default_rng(22)
    x = _act(rng, (64, 48))
    xv = O.bf16_to_f32(x)
    s = np.float32(np.abs(xv).max() / 100.0)          # |z| <= 100: no bound effects
    g = rng.standard_normal(x.shape).astype(np.float32)
    st = torch.tensor([s], requires_grad=True)
    zp = torch.zeros(1, requires_grad=True)
    out = torch._fake_quantize_learnable_per_tensor_affine(torch.from_numpy(xv.copy()), st, zp,
                                                           -128, 127, 1.0)
    (out * torch.from_numpy(g)).sum().backward()
    assert np.array_equal(O.fq_act(x, O.FMT_INT8, s).v, out.detach().numpy())
    ours = O.act_scale_grad(x, g, O.FMT_INT8, s)
    ref = float(st.grad[0])
    assert abs(ours - ref) <= 1e-4 * np.abs(g * O.fq_act(x, O.FMT_INT8, s).dv_ds).sum()


@pytest.mark.parametrize("fmt", [O.FMT_FP8, O.FMT_INT8])
def test_act_scale_grad_zero_on_grid(fmt):
    """x = q * s with q on the format's grid and s a power of two: z = q exactly,
    so every STE factor q - z is 0."""
    rng = np.random.default_rng(23)
    s = np.float32(2.0 ** -5)
    if fmt == O.FMT_INT8:
        q = rng.integers(-128, 128, (20, 64)).astype(np.float32)
    else:
        codes = rng.integers(0, 256, (20, 64))
        codes = np.where((codes & 0x7F) == 0x7F, 0x00, codes)        # drop NaN codes
        q = O.e4m3_value_of_code(codes).astype(np.float32)
    x = O.f32_to_bf16(q * s)
    assert np.array_equal(O.bf16_to_f32(x), q * s)                   # exact in bf16
    g = rng.standard_normal(x.shape)
    assert O.act_scale_grad(x, g, fmt, s) == 0.0


@pytest.mark.parametrize("fmt,hi,lo", [(O.FMT_FP8, 448.0, -448.0), (O.FMT_INT8, 127.0, -128.0)])
def test_act_scale_grad_all_saturated(fmt, hi, lo):
    rng = np.random.default_rng(24)
    sign = rng.choice([-1.0, 1.0], (16, 32))
    x = O.f32_to_bf16(sign.astype(np.float32))
    s = np.float32(1e-4)                                              # |z| = 1e4
    g = rng.standard_normal(x.shape)
    ref = float(np.sum(g * np.where(sign > 0, hi, lo)))
    assert O.act_scale_grad(x, g, fmt, s) == pytest.approx(ref, rel=1e-12)


def test_act_scale_grad_rejects_dynamic_and_none():
    x = O.f32_to_bf16(np.ones((2, 16), np.float32))
    for fmt in (O.FMT_NONE, O.FMT_NVFP4):
        with pytest.raises(ValueError):
            O.act_scale_grad(x, np.ones(x.shape), fmt, np.float32(1.0))
