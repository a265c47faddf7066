"""GPU edge cases through the C ABI: the largest expert count a grouped GEMM
takes, calls whose segments are all empty, and a MoE layer step with zero
tokens."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from helpers import (bf16_vals, check_dscale_tol, check_gemm_tol, dev_bf16, dev_f32, dev_i32,
                     host_bits)

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import moe_fake_quant_amd as F
else:  # collected on CPU only to be deselected by -m "not gpu"
    F = None


def _wq(fmt, group, s, zp, g):
    return F.WeightQ(fmt=fmt, group=group, scale=dev_f32(s),
                     zero_point=None if zp is None else dev_f32(zp),
                     global_scale=None if g is None else dev_f32(g))


def test_gemm_1024_experts_mostly_empty():
    """E = 1024 (the per-stack maximum): most experts empty, a few with rows,
    the last one spanning two row tiles with a ragged tail; per-channel FP8
    (group 256, dScale through per-128 partials)."""
    print("[edge] 1024 experts", flush=True)
    rng = np.random.default_rng(1024)
    E, N, K = 1024, 256, 256
    sizes = np.where(rng.random(E) < 0.9, 0, rng.integers(1, 40, E))
    sizes[E - 1] = 300
    sizes[0] = 1
    seg = np.zeros(E + 1, np.int32)
    seg[1:] = np.cumsum(sizes)
    R = int(seg[-1])
    w = O.f32_to_bf16((rng.standard_normal((E, N, K)) * 0.02).astype(np.float32))
    s, zp, g = O.observer_weight(w, O.FMT_FP8, K)
    x = O.f32_to_bf16(rng.standard_normal((R, K)).astype(np.float32))
    dy = O.f32_to_bf16(rng.standard_normal((R, N)).astype(np.float32))
    wq = _wq(O.FMT_FP8, K, s, None, None)
    ws = torch.empty(max(F.fq_workspace_bytes(F.FQ_OP_GEMM_FWD, (E, N, K), R, O.FMT_FP8),
                         F.fq_workspace_bytes(F.FQ_OP_GEMM_BWD, (E, N, K), R, O.FMT_FP8)),
                     dtype=torch.uint8, device="cuda")
    y = torch.empty(R, N, dtype=torch.bfloat16, device="cuda")
    dx = torch.empty(R, K, dtype=torch.bfloat16, device="cuda")
    ds = torch.full((E, N, 1), 7.0, device="cuda")
    wd, segd = dev_bf16(w), dev_i32(seg)
    F.fq_grouped_gemm_fwd(dev_bf16(x), R, segd, (E, N, K), wd, None, wq, None, y, ws)
    F.fq_grouped_gemm_bwd_scale(dev_bf16(dy), dev_bf16(x), R, segd, (E, N, K), wd, None, wq, None,
                                dx, ds, None, ws)
    torch.cuda.synchronize()
    # the oracle on the non-empty experts only (same rows, same order)
    live = np.flatnonzero(sizes > 0)
    sub_seg = np.zeros(len(live) + 1, np.int64)
    sub_seg[1:] = np.cumsum(sizes[live])
    y_ref = O.grouped_gemm_fwd(x, sub_seg, w[live], O.FMT_FP8, K, s[live])
    dx_ref, ds_ref, _ = O.grouped_gemm_bwd(dy, x, sub_seg, w[live], O.FMT_FP8, K, s[live])
    check_gemm_tol(host_bits(y), y_ref, "y")
    check_gemm_tol(host_bits(dx), dx_ref, "dx")
    dsh = ds.cpu().numpy()
    check_dscale_tol(dsh[live], ds_ref, "dscale")
    assert np.all(dsh[sizes == 0] == 0)


@pytest.mark.parametrize("fmt,group", [(O.FMT_INT4, 128), (O.FMT_INT8, 512), (O.FMT_NVFP4, 16)])
def test_gemm_all_segments_empty(fmt, group):
    """seg_offsets all zero: outputs untouched, dScale (and dZP) zero."""
    print(f"[edge] all-empty fmt={fmt}", flush=True)
    rng = np.random.default_rng(7)
    E, N, K, R_max = 4, 256, 512, 64
    seg = np.zeros(E + 1, np.int32)
    w = O.f32_to_bf16((rng.standard_normal((E, N, K)) * 0.02).astype(np.float32))
    s, zp, g = O.observer_weight(w, fmt, group)
    wq = _wq(fmt, group, s, zp, g)
    x = dev_bf16(O.f32_to_bf16(rng.standard_normal((R_max, K)).astype(np.float32)))
    dy = dev_bf16(O.f32_to_bf16(rng.standard_normal((R_max, N)).astype(np.float32)))
    ws = torch.empty(max(F.fq_workspace_bytes(F.FQ_OP_GEMM_FWD, (E, N, K), R_max, fmt),
                         F.fq_workspace_bytes(F.FQ_OP_GEMM_BWD, (E, N, K), R_max, fmt)),
                     dtype=torch.uint8, device="cuda")
    y = torch.full((R_max, N), 7.0, dtype=torch.bfloat16, device="cuda")
    dx = torch.full((R_max, K), 7.0, dtype=torch.bfloat16, device="cuda")
    G = K // group
    ds = torch.full((E, N, G), 7.0, device="cuda")
    dzp = torch.full((E, N, G), 7.0, device="cuda") if fmt == O.FMT_INT4 else None
    segd = dev_i32(seg)
    F.fq_grouped_gemm_fwd(x, R_max, segd, (E, N, K), dev_bf16(w), None, wq, None, y, ws)
    F.fq_grouped_gemm_bwd_scale(dy, x, R_max, segd, (E, N, K), dev_bf16(w), None, wq, None, dx, ds,
                                dzp, ws)
    torch.cuda.synchronize()
    assert np.all(bf16_vals(host_bits(y)) == 7.0)
    assert np.all(bf16_vals(host_bits(dx)) == 7.0)
    assert np.all(ds.cpu().numpy() == 0)
    if dzp is not None:
        assert np.all(dzp.cpu().numpy() == 0)


def test_layer_step_with_zero_tokens():
    """A step over an empty batch routes nothing and yields dScale = 0."""
    print("[edge] zero tokens", flush=True)
    case = W.moe_case(T=64, fmt="nvfp4", E_global=8, H=256, F=256, topk=4, seed=3)
    L = F.MoEFakeQuantLayer(dev_bf16(case.w_gu), dev_bf16(case.w_d), F.FMT_NVFP4, F.FMT_NVFP4,
                            case.T, case.topk, 0, 16)
    x, ids = dev_bf16(case.x), dev_i32(case.expert_ids)
    L.init_weight_scales()
    L.calibrate(x, ids)
    x0 = x[:0]
    ids0 = ids[:0]
    p0 = dev_f32(case.probs)[:0]
    d0 = dev_bf16(case.dout)[:0]
    dx, ds_gu, ds_d = L.step(x0, ids0, p0, d0)
    torch.cuda.synchronize()
    assert dx.shape[0] == 0
    assert np.all(L.seg.cpu().numpy() == 0)
    assert np.all(ds_gu.cpu().numpy() == 0) and np.all(ds_d.cpu().numpy() == 0)


def test_learnable_act_scales_with_zero_tokens():
    """An empty batch gives activation-scale gradients of exactly 0 (the
    outputs are overwritten, not accumulated)."""
    print("[edge] zero tokens, learnable fp8 act scales", flush=True)
    case = W.moe_case(T=64, fmt="fp8", E_global=8, H=256, F=256, topk=4, seed=4)
    L = F.MoEFakeQuantLayer(dev_bf16(case.w_gu), dev_bf16(case.w_d), F.FMT_FP8_E4M3,
                            F.FMT_FP8_E4M3, case.T, case.topk, 0, None, learn_act_scales=True)
    x, ids = dev_bf16(case.x), dev_i32(case.expert_ids)
    L.init_weight_scales()
    L.calibrate(x, ids)
    L.step(x, ids, dev_f32(case.probs), dev_bf16(case.dout))
    torch.cuda.synchronize()
    assert float(L.ds_a1.cpu()[0]) != 0.0 and float(L.ds_a2.cpu()[0]) != 0.0
    L.step(x[:0], ids[:0], dev_f32(case.probs)[:0], dev_bf16(case.dout)[:0])
    torch.cuda.synchronize()
    assert float(L.ds_a1.cpu()[0]) == 0.0 and float(L.ds_a2.cpu()[0]) == 0.0


def _block_pattern_rows(rng, rows, cols):
    """bf16 rows whose 16-blocks take one of: all zero, one nonzero element in
    the first half, one in the second half, random normal, all equal, tiny
    (subnormal-range) values, or a wide spread of magnitudes."""
    x = np.zeros((rows, cols), np.float32)
    for r in range(rows):
        for b in range(cols // 16):
            kind = rng.integers(0, 7)
            blk = np.zeros(16, np.float32)
            if kind == 1:
                blk[rng.integers(0, 8)] = rng.standard_normal() * 3
            elif kind == 2:
                blk[8 + rng.integers(0, 8)] = rng.standard_normal() * 3
            elif kind == 3:
                blk = rng.standard_normal(16).astype(np.float32)
            elif kind == 4:
                blk[:] = rng.choice([-1.5, 0.75, 2.0])
            elif kind == 5:
                blk = (rng.standard_normal(16) * 1e-38).astype(np.float32)
            elif kind == 6:
                blk = (rng.standard_normal(16) * 10.0 ** rng.integers(-3, 4, 16)).astype(np.float32)
            x[r, 16 * b:16 * b + 16] = blk
    return O.f32_to_bf16(x)


@pytest.mark.parametrize("afmt", [O.FMT_NVFP4, O.FMT_FP8, O.FMT_INT8, O.FMT_NONE])
@pytest.mark.parametrize("scale_mul", [1.0, 0.25])
def test_gather_and_swiglu_act_fq_block_halves(afmt, scale_mul):
    """The gather and SwiGLU-forward kernels hold one 16-byte vector per lane,
    so an NVFP4 16-block spans two lanes: blocks that are zero, whose amax sits
    in either half, ties, tiny and wide-range values, an odd token count, and
    slots not routed here; a quarter of the calibrated scale drives blocks into
    the E4M3 clamp. Bit-exact against the oracle."""
    print(f"[edge] block halves afmt={afmt} scale_mul={scale_mul}", flush=True)
    rng = np.random.default_rng(77)
    T, H, k, F2 = 37, 64, 3, 64
    x = _block_pattern_rows(rng, T, H)
    routed = rng.random((T, k)) < 0.8
    R = int(routed.sum())
    row_of = np.full((T, k), -1, np.int32)
    row_of[routed] = rng.permutation(R).astype(np.int32)
    perm = np.zeros(R, np.int64)
    for t in range(T):
        for j in range(k):
            if row_of[t, j] >= 0:
                perm[row_of[t, j]] = t * k + j
    s1 = np.float32(O.observer_act(x, afmt) * np.float32(scale_mul)) if afmt else np.float32(1.0)
    aq1 = F.ActQ(afmt, dev_f32([s1])) if afmt else None
    xq = torch.zeros((R, H), dtype=torch.bfloat16, device="cuda")
    F.fq_moe_gather_actfq(dev_bf16(x), T, H, dev_i32(row_of), k, aq1, xq)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(xq), O.gather_actfq(x, perm, k, afmt, s1).bits)

    h = _block_pattern_rows(rng, R, F2)
    Fh = F2 // 2
    a_ref = O.swiglu_fwd(h)
    s2 = np.float32(O.observer_act(a_ref, afmt) * np.float32(scale_mul)) if afmt else np.float32(1.0)
    aq2 = F.ActQ(afmt, dev_f32([s2])) if afmt else None
    a = torch.zeros((R + 5, Fh), dtype=torch.bfloat16, device="cuda")
    aq = torch.zeros((R + 5, Fh), dtype=torch.bfloat16, device="cuda")
    hd = torch.zeros((R + 5, F2), dtype=torch.bfloat16, device="cuda")
    hd[:R] = dev_bf16(h)
    F.fq_swiglu_actfq(hd, R + 5, dev_i32([R]), Fh, aq2, a, aq)
    torch.cuda.synchronize()
    a_gpu = host_bits(a)
    check_gemm_tol(a_gpu[:R], a_ref, "a")
    assert np.array_equal(host_bits(aq)[:R], O.fq_act(a_gpu[:R], afmt, s2).bits)
    # rows past the device row count are never written
    assert not host_bits(aq)[R:].any() and not a_gpu[R:].any()
