"""Pins of the oracle's scale-only backward (dX and dScale).

(i) An independent derivation: torch CPU autograd of the written-out
fake-quant formula with a straight-through round, using different rounding
code (torch.round, the float8 cast, an exponent-based E2M1 rounding) and
autograd instead of the hand-derived STE factors.
(ii) On-grid weights at power-of-two scales give dScale = 0 exactly.
(iii) All-saturated weights give dScale = sum(dWq) * bound.
(iv) A16 configurations: dX equals the plain matmul dY . FQ(W).
(v) Library special case: torch's learnable per-channel fake quant gives the
same scale gradient away from the clamp bounds.
CPU only."""
import numpy as np
import pytest
import torch

import oracle as O


def _ste(u, rounded):
    return u + (rounded - u).detach()


def _round_e2m1_torch(u):
    a = u.abs().clamp(max=6.0)
    e = torch.floor(torch.log2(a.clamp(min=1e-30))).clamp(0, 2)
    q = torch.pow(2.0, e - 1)
    r = torch.round(a / q) * q
    return torch.where(a == 0, torch.zeros_like(a), r).copysign(u)


def _torch_fq_weight(w, fmt, group, scale, zp=None, g=None):
    """Differentiable FQ(W) in fp32, scale (and zp) as leaves; returns v [E,N,K]."""
    E, N, K = w.shape
    rep = lambda p: p.repeat_interleave(group, dim=-1)  # noqa: E731
    if fmt == O.FMT_NVFP4:
        th = scale.clamp(0.0, 448.0)
        thq = _ste(th, th.detach().to(torch.float8_e4m3fn).to(torch.float32))
        s = thq * g.view(E, 1, 1)
        s_e = rep(s)
        zero = s_e == 0
        r = 1.0 / torch.where(zero, torch.ones_like(s_e), s_e)
        z = torch.where(zero, torch.zeros_like(w), w * r)
        zc = z.clamp(-6.0, 6.0)
        q = _ste(zc, _round_e2m1_torch(zc.detach()))
        return torch.where(zero, torch.zeros_like(w), q * s_e)
    s_e = rep(scale)
    r = 1.0 / s_e
    z = w * r
    if fmt == O.FMT_INT8:
        q = _ste(z.clamp(-128.0, 127.0), torch.round(z.clamp(-128.0, 127.0).detach()))
        return q * s_e
    if fmt == O.FMT_FP8:
        zc = z.clamp(-448.0, 448.0)
        q = _ste(zc, zc.detach().to(torch.float8_e4m3fn).to(torch.float32))
        return q * s_e
    if fmt == O.FMT_INT4:
        zpi = _ste(zp, torch.round(zp.detach()).clamp(0, 15))
        zp_e = rep(zpi)
        zc = torch.maximum(torch.minimum(z, 15.0 - zp_e), -zp_e)
        q = _ste(zc, torch.round(zc.detach()))
        return q * s_e
    raise ValueError(fmt)


def _case(fmt, seed=0):
    rng = np.random.default_rng(seed)
    E, N = 3, 16
    K = 256 if fmt == O.FMT_INT4 else 64
    group = {O.FMT_INT8: K, O.FMT_FP8: K, O.FMT_INT4: 128, O.FMT_NVFP4: 16}[fmt]
    w = O.f32_to_bf16((rng.standard_normal((E, N, K)) * 0.02).astype(np.float32))
    s, zp, g = O.observer_weight(w, fmt, group)
    # perturb scales so some elements saturate and rounding residues are generic
    if fmt == O.FMT_NVFP4:
        s = s.copy()
        s[0, 0, :] = 0.0                    # zero block scale
        s[1, 1, 0] = 500.0                  # above 448
        s[2, 2, 1] = O.e4m3_round(np.float32(s[2, 2, 1] * 0.6))[1].astype(np.float32)
    else:
        s = (s * rng.uniform(0.6, 1.1, s.shape)).astype(np.float32)
    R = 20
    seg = np.array([0, 9, 9, R], np.int32)      # expert 1 empty
    x = O.f32_to_bf16(rng.standard_normal((R, K)).astype(np.float32))
    dy = O.f32_to_bf16(rng.standard_normal((R, N)).astype(np.float32))
    return w, x, dy, seg, group, s, zp, g


@pytest.mark.parametrize("fmt", [O.FMT_INT8, O.FMT_INT4, O.FMT_FP8, O.FMT_NVFP4])
def test_dscale_and_dx_match_torch_autograd(fmt):
    w, x, dy, seg, group, s, zp, g = _case(fmt)
    dx_o, ds_o, dzp_o = O.grouped_gemm_bwd(dy, x, seg, w, fmt, group, s, zp, g)
    y_o = O.grouped_gemm_fwd(x, seg, w, fmt, group, s, zp, g)

    wt = torch.from_numpy(O.bf16_to_f32(w).copy())
    st = torch.from_numpy(s.copy()).requires_grad_(True)
    zpt = torch.from_numpy(zp.copy()).requires_grad_(True) if zp is not None else None
    gt = torch.from_numpy(g.copy()) if g is not None else None
    v = _torch_fq_weight(wt, fmt, group, st, zpt, gt)
    vq = v.to(torch.bfloat16).to(torch.float64)       # forward stores bf16; STE treats it as identity
    vq = v.to(torch.float64) + (vq - v.to(torch.float64)).detach()
    xt = torch.from_numpy(O.bf16_to_f32(x).astype(np.float64)).requires_grad_(True)
    dyt = torch.from_numpy(O.bf16_to_f32(dy).astype(np.float64))
    ys = []
    for e in range(3):
        ys.append(xt[seg[e]:seg[e + 1]] @ vq[e].T)
    y = torch.cat(ys)
    (y * dyt).sum().backward()

    assert np.array_equal(O.f64_to_bf16(y.detach().numpy()), y_o)
    ds_t = st.grad.double().numpy()
    scale = np.abs(ds_t).max()
    assert np.abs(ds_o - ds_t).max() <= 1e-6 * scale
    assert np.all(ds_o[1] == 0)                       # empty expert
    dx_t = xt.grad.numpy()
    assert np.array_equal(dx_o, O.f64_to_bf16(dx_t))
    if fmt == O.FMT_INT4:
        dzp_t = zpt.grad.double().numpy()
        assert np.abs(dzp_o - dzp_t).max() <= 1e-6 * max(np.abs(dzp_t).max(), 1e-30)


@pytest.mark.parametrize("fmt", [O.FMT_INT8, O.FMT_INT4, O.FMT_FP8, O.FMT_NVFP4])
def test_dscale_zero_for_on_grid_weights(fmt):
    rng = np.random.default_rng(7)
    E, N, K = 2, 8, 128
    group = {O.FMT_INT8: K, O.FMT_FP8: K, O.FMT_INT4: 128, O.FMT_NVFP4: 16}[fmt]
    G = K // group
    s = np.full((E, N, G), 2.0 ** -6, np.float32)
    zp = g = None
    if fmt == O.FMT_INT8:
        q = rng.integers(-128, 128, (E, N, K))
    elif fmt == O.FMT_INT4:
        zp = rng.integers(0, 16, (E, N, G)).astype(np.float32)
        q = rng.integers(0, 16, (E, N, K)) - np.repeat(zp, group, -1)
    elif fmt == O.FMT_FP8:
        codes = rng.integers(0, 0x7F, (E, N, K)) | (rng.integers(0, 2, (E, N, K)) << 7)
        q = O.e4m3_value_of_code(codes)
    else:
        q = O.e2m1_value_of_code(rng.integers(0, 16, (E, N, K)))
        s = np.full((E, N, G), 1.0, np.float32)
        g = np.full(E, 2.0 ** -6, np.float32)
    eff = 2.0 ** -6
    w = O.f32_to_bf16((q * eff).astype(np.float32))
    assert np.array_equal(O.bf16_to_f32(w), (q * eff).astype(np.float32))
    R = 12
    seg = np.array([0, 5, R], np.int32)
    x = O.f32_to_bf16(rng.standard_normal((R, K)).astype(np.float32))
    dy = O.f32_to_bf16(rng.standard_normal((R, N)).astype(np.float32))
    _, ds, _ = O.grouped_gemm_bwd(dy, x, seg, w, fmt, group, s, zp, g)
    assert np.all(ds == 0)


def test_dscale_all_saturated_closed_form():
    rng = np.random.default_rng(8)
    E, N, K = 1, 4, 32
    s = np.full((E, N, 1), 1e-4, np.float32)
    sign = rng.choice([-1.0, 1.0], (E, N, K))
    w = O.f32_to_bf16((sign * 1.0).astype(np.float32))        # |z| = 1e4 >> 448
    R = 7
    seg = np.array([0, R], np.int32)
    x = O.f32_to_bf16(rng.standard_normal((R, K)).astype(np.float32))
    dy = O.f32_to_bf16(rng.standard_normal((R, N)).astype(np.float32))
    dwq = O.bf16_to_f32(dy).astype(np.float64).T @ O.bf16_to_f32(x).astype(np.float64)
    for fmt, hi, lo in ((O.FMT_INT8, 127.0, -128.0), (O.FMT_FP8, 448.0, -448.0)):
        _, ds, _ = O.grouped_gemm_bwd(dy, x, seg, w, fmt, K, s)
        bound = np.where(sign[0] > 0, hi, lo)
        ref = (dwq * bound).sum(-1)
        assert np.allclose(ds[0, :, 0], ref, rtol=1e-12, atol=0)


def test_a16_dx_is_plain_matmul():
    w, x, dy, seg, group, s, zp, g = _case(O.FMT_INT8, seed=3)
    dx, _, _ = O.grouped_gemm_bwd(dy, x, seg, w, O.FMT_INT8, group, s)
    wq = O.bf16_to_f32(O.fq_weight_stack(w, O.FMT_INT8, group, s).bits).astype(np.float64)
    d = O.bf16_to_f32(dy).astype(np.float64)
    ref = np.concatenate([d[seg[e]:seg[e + 1]] @ wq[e] for e in range(3)])
    assert np.array_equal(dx, O.f64_to_bf16(ref))


def test_int8_scale_grad_matches_torch_learnable_fake_quant_away_from_bounds():
    """torch._fake_quantize_learnable_per_channel_affine masks on the rounded code;
    away from the clamp bounds it is the same STE, so the scale gradients agree."""
    rng = np.random.default_rng(9)
    N, K = 8, 64
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    s = (np.abs(w).max(1) / 100).astype(np.float32)    # |z| <= 100 < 127.5: no bound effects
    gy = rng.standard_normal((N, K)).astype(np.float32)
    wt = torch.from_numpy(w)
    st = torch.from_numpy(s.copy()).requires_grad_(True)
    zpt = torch.zeros(N, dtype=torch.float32, requires_grad=True)
    out = torch._fake_quantize_learnable_per_channel_affine(wt, st, zpt, 0, -128, 127, 1.0)
    (out * torch.from_numpy(gy)).sum().backward()
    fq = O.fq_int8(w, s[:, None])
    assert np.array_equal(fq.v, out.detach().numpy())
    ours = (fq.dv_ds * gy).sum(1)
    # torch reduces its per-element terms in fp32: compare normwise at 1e-4
    ref = st.grad.numpy().astype(np.float64)
    assert np.abs(ours - ref).max() <= 1e-4 * np.abs(ref).max()


@pytest.mark.parametrize("fmt", [O.FMT_INT8, O.FMT_FP8])
def test_per_tensor_dscale_matches_torch_autograd(fmt):
    """One scale per expert matrix (a [E] leaf broadcast over [N, K]): autograd
    sums the straight-through factors over the whole matrix."""
    rng = np.random.default_rng(31)
    E, N, K, R = 3, 8, 64, 21
    w = O.f32_to_bf16((rng.standard_normal((E, N, K)) * 0.02).astype(np.float32))
    s, _, _ = O.observer_weight(w, fmt, O.GROUP_TENSOR)
    assert s.shape == (E,)
    s = (s * rng.uniform(0.5, 1.0, E)).astype(np.float32)    # some elements saturate
    seg = np.array([0, 8, 8, R], np.int32)                     # expert 1 empty
    x = O.f32_to_bf16(rng.standard_normal((R, K)).astype(np.float32))
    dy = O.f32_to_bf16(rng.standard_normal((R, N)).astype(np.float32))
    dx_o, ds_o, _ = O.grouped_gemm_bwd(dy, x, seg, w, fmt, O.GROUP_TENSOR, s)
    assert ds_o.shape == (E,) and ds_o[1] == 0.0

    wt = torch.from_numpy(O.bf16_to_f32(w).copy())
    st = torch.from_numpy(s.copy()).requires_grad_(True)
    s_e = st.view(E, 1, 1)
    z = wt * (1.0 / s_e)
    bound = 127.0 if fmt == O.FMT_INT8 else 448.0
    zc = z.clamp(-128.0 if fmt == O.FMT_INT8 else -448.0, bound)
    rq = torch.round(zc.detach()) if fmt == O.FMT_INT8 else \
        zc.detach().to(torch.float8_e4m3fn).to(torch.float32)
    v = _ste(zc, rq) * s_e
    vq = v.to(torch.float64) + (v.to(torch.bfloat16).to(torch.float64) - v.to(torch.float64)).detach()
    assert np.array_equal(O.f32_to_bf16(v.detach().numpy()),
                          O.fq_weight_stack(w, fmt, O.GROUP_TENSOR, s).bits)
    xt = torch.from_numpy(O.bf16_to_f32(x).astype(np.float64))
    dyt = torch.from_numpy(O.bf16_to_f32(dy).astype(np.float64))
    y = torch.cat([xt[seg[e]:seg[e + 1]] @ vq[e].T for e in range(E)])
    (y * dyt).sum().backward()
    ds_t = st.grad.double().numpy()
    assert np.abs(ds_o - ds_t).max() <= 1e-6 * np.abs(ds_t).max()


@pytest.mark.parametrize("fmt", [O.FMT_INT8, O.FMT_FP8])
def test_per_tensor_is_per_channel_with_one_shared_scale(fmt):
    """The same values as per-channel quantization whose N scales all equal the
    expert's one scale; the per-tensor gradient is the sum of the N channel
    gradients."""
    rng = np.random.default_rng(32)
    E, N, K, R = 2, 16, 32, 30
    w = O.f32_to_bf16((rng.standard_normal((E, N, K)) * 0.05).astype(np.float32))
    s = np.array([0.02 / 127, 0.05 / 448], np.float32)
    rep = np.repeat(s[:, None, None], N, axis=1)              # [E, N, 1]
    a = O.fq_weight_stack(w, fmt, O.GROUP_TENSOR, s)
    b = O.fq_weight_stack(w, fmt, K, rep)
    assert np.array_equal(a.bits, b.bits) and np.array_equal(a.dv_ds, b.dv_ds)
    seg = np.array([0, 13, R], np.int32)
    x = O.f32_to_bf16(rng.standard_normal((R, K)).astype(np.float32))
    dy = O.f32_to_bf16(rng.standard_normal((R, N)).astype(np.float32))
    dx_t, ds_t, _ = O.grouped_gemm_bwd(dy, x, seg, w, fmt, O.GROUP_TENSOR, s)
    dx_c, ds_c, _ = O.grouped_gemm_bwd(dy, x, seg, w, fmt, K, rep)
    assert np.array_equal(dx_t, dx_c)
    assert np.allclose(ds_t, ds_c.sum(axis=(1, 2)), rtol=1e-12, atol=0)
