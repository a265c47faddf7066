"""GPU parity at the five full-size workloads, in the launch configuration the
benchmark times (MoE: ``MoEFakeQuantLayer.step`` after observer init and one
calibration forward; dense: the C-ABI calls with E = 1).

The oracle cannot redo a full-size layer in seconds, so each stage is checked
on samples it can compute one by one, each fed the GPU's own inputs of that
stage:
  * routing: the whole permutation, row map and segment offsets (bit-exact);
  * observer and FQ pass: every scale and fake-quantized weight of sampled
    experts (bit-exact), the activation scales over the whole tensors;
  * act FQ, combine bwd: sampled routed rows (bit-exact);
  * GEMM outputs (h, o, daq, dxq) and SwiGLU: sampled rows of sampled experts
    (first rows, the ragged last rows and random middle rows);
  * dScale: sampled output channels of sampled experts, reduced over all of
    that expert's rows (a channel's dScale depends on no other channel);
  * combine and unpermute-reduce: sampled tokens;
  * empty experts: dScale exactly 0;
  * learnable FP8 activation scales: each gradient is one sum over a whole
    tensor, so the full-size result is checked by additivity (the kernel run
    on eight disjoint slices sums to the full-size value) and one slice
    against the oracle.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from helpers import (ACT_DSCALE_TOL, bf16_vals, check_act_dscale_tol, check_dscale_tol, dscale_p99,
                     check_gemm_tol, dev_bf16, dev_f32, dev_i32, host_bits)

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import moe_fake_quant_amd as F
else:  # collected on CPU only to be deselected by -m "not gpu"
    F = None


def _say(msg):
    print(msg, flush=True)


def _sample_rows(rng, lo, hi, n_edge=40, n_mid=40):
    """First rows, last (ragged-tail) rows and random middle rows of [lo, hi)."""
    if hi - lo <= 2 * n_edge + n_mid:
        return np.arange(lo, hi)
    mid = rng.choice(np.arange(lo + n_edge, hi - n_edge), n_mid, replace=False)
    return np.unique(np.concatenate([np.arange(lo, lo + n_edge), mid, np.arange(hi - n_edge, hi)]))


def _sample_channels(rng, N, n=48):
    return np.unique(np.concatenate([[0, N - 1], rng.choice(N, n, replace=False)]))


def _sub_q(wq, experts, channels=None):
    """Oracle quantizer parameters (scale, zp, g) restricted to experts / channels."""
    s, zp, g = wq
    sel = (lambda a: a[experts] if channels is None else a[experts][:, channels])
    return (sel(s), None if zp is None else sel(zp), None if g is None else g[experts])


MOE = [
    # cfg, weight/act format, group (None = per channel)
    (3, O.FMT_FP8, None),
    (4, O.FMT_NVFP4, 16),
    (5, O.FMT_NVFP4, 16),
]


@pytest.mark.parametrize("cfg,fmt,group", MOE)
def test_moe_full_size_sampled(cfg, fmt, group):
    case = W.config(cfg, seed=0)
    _say(f"[fullsize] {W.CONFIG_NAMES[cfg]}: T={case.T} E={case.E}")
    rng = np.random.default_rng(cfg)
    E, T, k = case.E, case.T, case.topk
    H, Fh = case.w_gu.shape[2], case.w_d.shape[2]
    g_gu, g_d = group or H, group or Fh
    ffmt = {O.FMT_FP8: F.FMT_FP8_E4M3, O.FMT_NVFP4: F.FMT_NVFP4}[fmt]
    L = F.MoEFakeQuantLayer(dev_bf16(case.w_gu), dev_bf16(case.w_d), ffmt, ffmt, T, k,
                            case.expert_begin, group)
    x, ids = dev_bf16(case.x), dev_i32(case.expert_ids)
    p, dout = dev_f32(case.probs), dev_bf16(case.dout)
    L.init_weight_scales()
    L.calibrate(x, ids)
    L.step(x, ids, p, dout)
    # SwiGLU output a (the step keeps only aq): the same kernel, writing both
    a_dev = torch.empty_like(L.a)
    aq_again = torch.empty_like(L.aq)
    F.fq_swiglu_actfq(L.h, L.R_max, L.n_rows, Fh, L.aq2, a_dev, aq_again)
    torch.cuda.synchronize()

    # routing, whole
    perm, row_of, seg = O.moe_permute(case.expert_ids, case.expert_begin, E)
    R = int(seg[-1])
    assert np.array_equal(L.seg.cpu().numpy(), seg)
    assert np.array_equal(L.perm.cpu().numpy()[:R], perm)
    assert np.array_equal(L.row_of.cpu().numpy()[:T], row_of)
    counts = np.diff(seg)
    empty = np.flatnonzero(counts == 0)
    if cfg == 5:
        assert set(empty.tolist()) == set(W.ZIPF_EMPTY_EXPERTS)

    # activation scales over the whole tensors
    s1 = L.aq1.scale.cpu().numpy()[0]
    s2 = L.aq2.scale.cpu().numpy()[0]
    assert s1 == O.observer_act(case.x, fmt)
    a_all = host_bits(a_dev)[:R]
    assert s2 == O.observer_act(a_all, fmt)
    assert torch.equal(aq_again[:R].view(torch.int16), L.aq[:R].view(torch.int16))

    # sampled experts: hottest, coldest non-empty, first, and one at random
    nonempty = np.flatnonzero(counts > 0)
    S = np.unique([int(np.argmax(counts)), int(nonempty[np.argmin(counts[nonempty])]), 0,
                   int(rng.choice(nonempty))])
    S = np.array([e for e in S if counts[e] > 0])

    # observer + FQ pass of the sampled experts, bit-exact
    wq_gu = O.observer_weight(case.w_gu[S], fmt, g_gu)
    wq_d = O.observer_weight(case.w_d[S], fmt, g_d)
    assert np.array_equal(L.q_gu.scale.cpu().numpy()[S], wq_gu[0])
    assert np.array_equal(L.q_d.scale.cpu().numpy()[S], wq_d[0])
    if fmt == O.FMT_NVFP4:
        assert np.array_equal(L.q_gu.global_scale.cpu().numpy()[S], wq_gu[2])
        assert np.array_equal(L.q_d.global_scale.cpu().numpy()[S], wq_d[2])
    wfq_gu = host_bits(L.wfq_gu[torch.from_numpy(S).cuda()])
    wfq_d = host_bits(L.wfq_d[torch.from_numpy(S).cuda()])
    assert np.array_equal(wfq_gu, O.fq_weight_stack(case.w_gu[S], fmt, g_gu, *wq_gu).bits)
    assert np.array_equal(wfq_d, O.fq_weight_stack(case.w_d[S], fmt, g_d, *wq_d).bits)

    # the expert input as token rows, read by the gate_up GEMMs through the
    # routing: token rows bit-exact, then the routed rows they stand for
    xq_tok = host_bits(L.xq_tok)[:T]
    toks = rng.choice(T, 64, replace=False)
    assert np.array_equal(xq_tok[toks], O.fq_act(case.x[toks], fmt, s1).bits)
    xq_all = xq_tok[perm // k]
    h_all, aq_all = host_bits(L.h), host_bits(L.aq)
    o_all, do_all, daq_all = host_bits(L.o), host_bits(L.do), host_bits(L.daq)
    dh_all, dxq_all = host_bits(L.dh), host_bits(L.dxq)
    ds_gu, ds_d = L.ds_gu.cpu().numpy(), L.ds_d.cpu().numpy()

    # empty experts: dScale exactly zero
    for e in empty:
        assert np.all(ds_gu[e] == 0) and np.all(ds_d[e] == 0)

    for i, e in enumerate(S):
        lo, hi = int(seg[e]), int(seg[e + 1])
        rows = _sample_rows(rng, lo, hi)
        sseg = np.array([0, len(rows)])
        qg, qd = _sub_q(wq_gu, [i]), _sub_q(wq_d, [i])
        wg, wd = case.w_gu[[e]], case.w_d[[e]]
        _say(f"[fullsize] expert {e}: {hi - lo} rows, {len(rows)} sampled")
        # gather + act FQ (bit-exact), combine bwd (bit-exact)
        assert np.array_equal(xq_all[rows], O.gather_actfq(case.x, perm[rows], k, fmt, s1).bits)
        assert np.array_equal(do_all[rows], O.combine_bwd(case.dout, case.probs, perm[rows], k))
        # forward GEMMs and SwiGLU on the GPU's inputs
        check_gemm_tol(h_all[rows], O.grouped_gemm_fwd(xq_all[rows], sseg, wg, fmt, g_gu, *qg),
                       f"h e{e}")
        check_gemm_tol(a_all[rows], O.swiglu_fwd(h_all[rows]), f"a e{e}")
        assert np.array_equal(aq_all[rows], O.fq_act(a_all[rows], fmt, s2).bits)
        check_gemm_tol(o_all[rows], O.grouped_gemm_fwd(aq_all[rows], sseg, wd, fmt, g_d, *qd),
                       f"o e{e}")
        # dgrads and SwiGLU bwd
        daq_ref, _, _ = O.grouped_gemm_bwd(do_all[rows], aq_all[rows], sseg, wd, fmt, g_d, *qd)
        check_gemm_tol(daq_all[rows], daq_ref, f"daq e{e}")
        check_gemm_tol(dh_all[rows], O.swiglu_bwd(daq_all[rows], h_all[rows], fmt, s2,
                                                  a_bits=a_all[rows]), f"dh e{e}")
        dxq_ref, _, _ = O.grouped_gemm_bwd(dh_all[rows], xq_all[rows], sseg, wg, fmt, g_gu, *qg)
        check_gemm_tol(dxq_all[rows], dxq_ref, f"dxq e{e}")
        # dScale: sampled channels over all rows of the expert
        full = np.array([0, hi - lo])
        for name, dy_all, x_all, w, q, grp, ds in (
                ("ds_d", do_all, aq_all, wd, wq_d, g_d, ds_d),
                ("ds_gu", dh_all, xq_all, wg, wq_gu, g_gu, ds_gu)):
            ch = _sample_channels(rng, w.shape[1])
            _, ref, _ = O.grouped_gemm_bwd(dy_all[lo:hi][:, ch], x_all[lo:hi], full,
                                           w[:, ch], fmt, grp, *_sub_q(q, [i], ch))
            rel = check_dscale_tol(ds[e][ch], ref[0], f"{name} e{e}")
            print(f"[dscale] {name} e{e}: max|err|/max|ref| {rel:.3g}, p99 element-wise "
                  f"{dscale_p99(ds[e][ch], ref[0]):.3g}", flush=True)

    # combine and unpermute-reduce on sampled tokens (GPU's O and dXq rows)
    tok = np.unique(np.concatenate([[0, T - 1], rng.choice(T, 256, replace=False)]))
    ro = row_of[tok]
    used = np.maximum(ro, 0).reshape(-1)          # the rows these tokens read
    ro_sub = np.where(ro >= 0, np.arange(ro.size).reshape(ro.shape), -1)
    check_gemm_tol(host_bits(L.out)[tok], O.combine(o_all[used], case.probs[tok], ro_sub), "out")
    check_gemm_tol(host_bits(L.dx)[tok],
                   O.unpermute_reduce(dxq_all[used], ro_sub, case.x[tok], fmt, s1), "dx")


def test_fp8_learnable_act_scales_full_size():
    """The FP8 MoE workload with learnable activation scales, in the layer's
    launch configuration."""
    case = W.config(3, seed=0)
    _say(f"[fullsize] {W.CONFIG_NAMES[3]} learnable act scales")
    E, T, k = case.E, case.T, case.topk
    H, Fh = case.w_gu.shape[2], case.w_d.shape[2]
    ffmt = F.FMT_FP8_E4M3
    L = F.MoEFakeQuantLayer(dev_bf16(case.w_gu), dev_bf16(case.w_d), ffmt, ffmt, T, k,
                            case.expert_begin, None, learn_act_scales=True)
    x, ids = dev_bf16(case.x), dev_i32(case.expert_ids)
    L.init_weight_scales()
    L.calibrate(x, ids)
    L.step(x, ids, dev_f32(case.probs), dev_bf16(case.dout))
    a_dev = torch.empty_like(L.a)
    F.fq_swiglu_actfq(L.h, L.R_max, L.n_rows, Fh, L.aq2, a_dev, torch.empty_like(L.aq))
    torch.cuda.synchronize()
    R = int(L.seg[E].item())
    s1 = L.aq1.scale.cpu().numpy()[0]
    s2 = L.aq2.scale.cpu().numpy()[0]
    full1, full2 = float(L.ds_a1.cpu()[0]), float(L.ds_a2.cpu()[0])
    ds = torch.empty(1, device="cuda")
    ws = L.ws
    # eight disjoint token slices of the unpermute-reduce
    tb = np.linspace(0, T, 9).astype(int)
    parts1 = []
    dx_tmp = torch.empty_like(L.dx)
    for t0, t1 in zip(tb[:-1], tb[1:]):
        F.fq_moe_unpermute_reduce(L.dxq, L.row_of[t0:t1], x[t0:t1], t1 - t0, k, H, L.aq1,
                                  dx_tmp[t0:t1], ds, ws)
        parts1.append(float(ds.cpu()[0]))
    # eight disjoint row slices of the SwiGLU backward (n_rows = the slice length)
    rb = np.linspace(0, R, 9).astype(int)
    parts2 = []
    dh_tmp = torch.empty_like(L.dh)
    for r0, r1 in zip(rb[:-1], rb[1:]):
        n = dev_i32([r1 - r0])
        F.fq_swiglu_bwd(L.daq[r0:r1], L.h[r0:r1], r1 - r0, n, Fh, L.aq2, dh_tmp[r0:r1], ds, ws)
        parts2.append(float(ds.cpu()[0]))
    torch.cuda.synchronize()
    # the oracle on the first slice of each, from the GPU's own dXq / dAq / A
    row_of = L.row_of.cpu().numpy()[:T]
    t1 = int(tb[1])
    ro = row_of[:t1]
    used = np.maximum(ro, 0).reshape(-1)
    ro_sub = np.where(ro >= 0, np.arange(ro.size).reshape(ro.shape), -1)
    dxq_used = host_bits(L.dxq)[used]
    fx = O.fq_act(case.x[:t1], O.FMT_FP8, s1)
    g1 = O.unpermute_sum(dxq_used, ro_sub)
    sc1 = float(np.sum(O.unpermute_sum(dxq_used & np.uint16(0x7FFF), ro_sub) * np.abs(fx.dv_ds)))
    check_act_dscale_tol(parts1[0], float(np.sum(g1 * fx.dv_ds)), sc1, "ds_a1 slice 0")
    r1 = int(rb[1])
    a_sl = host_bits(a_dev)[:r1]
    g2 = bf16_vals(host_bits(L.daq)[:r1])
    fa = O.fq_act(a_sl, O.FMT_FP8, s2)
    sc2 = float(np.sum(np.abs(g2 * fa.dv_ds)))
    check_act_dscale_tol(parts2[0], O.act_scale_grad(a_sl, g2, O.FMT_FP8, s2), sc2,
                         "ds_a2 slice 0")
    # additivity at full size; sum|terms| extrapolated from the first slice
    # (the slices are equal in size and identically distributed)
    check_act_dscale_tol(sum(parts1), full1, 8 * sc1, "ds_a1 additivity",
                         tol=2 * ACT_DSCALE_TOL)
    check_act_dscale_tol(sum(parts2), full2, 8 * sc2, "ds_a2 additivity",
                         tol=2 * ACT_DSCALE_TOL)
    assert full1 != 0.0 and full2 != 0.0


def _dense_run(case, fmt, group):
    w, x, dy = case.w, case.x, case.dy
    N, K = w.shape
    M = x.shape[0]
    shape = (1, N, K)
    ffmt = {O.FMT_INT8: F.FMT_INT8, O.FMT_INT4: F.FMT_INT4}[fmt]
    G = K // group
    s = torch.empty(1, N, G, device="cuda")
    zp = torch.empty(1, N, G, device="cuda") if fmt == O.FMT_INT4 else None
    wd = dev_bf16(w[None])
    F.observer_absmax_init(wd, shape, ffmt, group, 0, s, zp, None)
    q = F.WeightQ(ffmt, group, s, zp, None)
    seg = dev_i32([0, M])
    wfq = torch.empty_like(wd)
    F.fq_quantize_stacked(wd, shape, q, wfq)
    ws = torch.empty(max(F.fq_workspace_bytes(F.FQ_OP_GEMM_FWD, shape, M, ffmt),
                         F.fq_workspace_bytes(F.FQ_OP_GEMM_BWD, shape, M, ffmt)),
                     dtype=torch.uint8, device="cuda")
    y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    dx = torch.empty(M, K, dtype=torch.bfloat16, device="cuda")
    ds = torch.empty(1, N, G, device="cuda")
    dzp = torch.empty(1, N, G, device="cuda") if fmt == O.FMT_INT4 else None
    xd, dyd = dev_bf16(x), dev_bf16(dy)
    # weights fake-quantized inside the calls (raw W + scales), as a dense
    # linear would use them
    F.fq_grouped_gemm_fwd(xd, M, seg, shape, wd, None, q, None, y, ws)
    F.fq_grouped_gemm_bwd_scale(dyd, xd, M, seg, shape, wd, None, q, None, dx, ds, dzp, ws)
    torch.cuda.synchronize()
    return dict(s=s.cpu().numpy(), zp=None if zp is None else zp.cpu().numpy(),
                wfq=host_bits(wfq)[0], y=host_bits(y), dx=host_bits(dx), ds=ds.cpu().numpy()[0],
                dzp=None if dzp is None else dzp.cpu().numpy()[0])


def test_dense_int8_per_channel_full():
    case = W.config(1, seed=0)
    _say(f"[fullsize] {case.name}")
    K = case.w.shape[1]
    got = _dense_run(case, O.FMT_INT8, K)
    wq = O.observer_weight(case.w[None], O.FMT_INT8, K)
    assert np.array_equal(got["s"], wq[0])
    assert np.array_equal(got["wfq"], O.fq_weight_stack(case.w[None], O.FMT_INT8, K, *wq).bits[0])
    seg = np.array([0, case.x.shape[0]])
    check_gemm_tol(got["y"], O.grouped_gemm_fwd(case.x, seg, case.w[None], O.FMT_INT8, K, *wq), "y")
    dx_ref, ds_ref, _ = O.grouped_gemm_bwd(case.dy, case.x, seg, case.w[None], O.FMT_INT8, K, *wq)
    check_gemm_tol(got["dx"], dx_ref, "dx")
    check_dscale_tol(got["ds"], ds_ref[0], "dscale")


def test_dense_int4_group128_sampled():
    case = W.config(2, seed=0)
    _say(f"[fullsize] {case.name}")
    rng = np.random.default_rng(2)
    N, K = case.w.shape
    M = case.x.shape[0]
    got = _dense_run(case, O.FMT_INT4, 128)
    wq = O.observer_weight(case.w[None], O.FMT_INT4, 128)
    assert np.array_equal(got["s"], wq[0])
    assert np.array_equal(got["zp"], wq[1])
    assert np.array_equal(got["wfq"], O.fq_weight_stack(case.w[None], O.FMT_INT4, 128, *wq).bits[0])
    rows = _sample_rows(rng, 0, M)
    sseg = np.array([0, len(rows)])
    check_gemm_tol(got["y"][rows],
                   O.grouped_gemm_fwd(case.x[rows], sseg, case.w[None], O.FMT_INT4, 128, *wq), "y")
    dx_ref, _, _ = O.grouped_gemm_bwd(case.dy[rows], case.x[rows], sseg, case.w[None], O.FMT_INT4,
                                      128, *wq)
    check_gemm_tol(got["dx"][rows], dx_ref, "dx")
    ch = _sample_channels(rng, N)
    _, ds_ref, dzp_ref = O.grouped_gemm_bwd(case.dy[:, ch], case.x, np.array([0, M]),
                                            case.w[None][:, ch], O.FMT_INT4, 128,
                                            *_sub_q(wq, [0], ch))
    check_dscale_tol(got["ds"][ch], ds_ref[0], "dscale")
    check_dscale_tol(got["dzp"][ch], dzp_ref[0], "dzero_point")
