"""Pins of the oracle's grouped GEMM, permutation and MoE chain by brute force
(per-row / per-element Python loops on tiny inputs), reductions to library
routines (E = 1 is np.matmul; the permutation is Python's sorted) and
invariants (row independence, power-of-two scaling). CPU only."""
import numpy as np
import pytest

import oracle as O
import workloads as W


def _rand_bf16(rng, shape, std=1.0):
    return O.f32_to_bf16((rng.standard_normal(shape) * std).astype(np.float32))


def _expert_of_row(seg, r):
    for e in range(len(seg) - 1):
        if seg[e] <= r < seg[e + 1]:
            return e
    raise AssertionError


@pytest.mark.parametrize("fmt,group,K", [(O.FMT_INT8, 32, 32), (O.FMT_NVFP4, 16, 32),
                                         (O.FMT_INT4, 128, 128), (O.FMT_FP8, 64, 64)])
def test_grouped_gemm_matches_per_element_loops(fmt, group, K):
    rng = np.random.default_rng(11)
    E, N = 4, 5
    w = _rand_bf16(rng, (E, N, K), 0.02)
    s, zp, g = O.observer_weight(w, fmt, group)
    seg = np.array([0, 3, 3, 7, 9], np.int32)     # expert 1 empty, ragged sizes
    R = int(seg[-1])
    x = _rand_bf16(rng, (R + 2, K))               # R_max > R: extra rows ignored
    dy = _rand_bf16(rng, (R + 2, N))
    afmt = O.FMT_FP8 if fmt == O.FMT_FP8 else O.FMT_NONE
    sa = O.observer_act(x[:R], O.FMT_FP8) if afmt else None
    y = O.grouped_gemm_fwd(x, seg, w, fmt, group, s, zp, g, afmt, sa)
    dx, ds, dzp = O.grouped_gemm_bwd(dy, x, seg, w, fmt, group, s, zp, g, afmt, sa)
    wq = O.fq_weight_stack(w, fmt, group, s, zp, g)
    wv = O.bf16_to_f32(wq.bits)
    xa = O.fq_act(x[:R], afmt, sa)
    xv = O.bf16_to_f32(xa.bits)
    dyv = O.bf16_to_f32(dy)
    y_ref = np.zeros((R, N))
    dx_ref = np.zeros((R, K))
    ds_ref = np.zeros_like(ds)
    for r in range(R):
        e = _expert_of_row(seg, r)
        for n in range(N):
            acc = 0.0
            for k in range(K):
                acc += float(xv[r, k]) * float(wv[e, n, k])
                ds_ref[e, n, k // group] += float(dyv[r, n]) * float(xv[r, k]) * wq.dv_ds[e, n, k]
            y_ref[r, n] = acc
        for k in range(K):
            acc = 0.0
            for n in range(N):
                acc += float(dyv[r, n]) * float(wv[e, n, k])
            dx_ref[r, k] = acc * xa.mask[r, k]
    assert np.array_equal(y, O.f64_to_bf16(y_ref))
    assert np.array_equal(dx, O.f64_to_bf16(dx_ref))
    assert np.allclose(ds, ds_ref, rtol=1e-12, atol=1e-12 * np.abs(ds_ref).max())
    assert np.all(ds[1] == 0)


def test_single_expert_is_matmul_and_rows_independent():
    rng = np.random.default_rng(12)
    N, K, M = 24, 64, 17
    w = _rand_bf16(rng, (1, N, K), 0.02)
    s, _, _ = O.observer_weight(w, O.FMT_INT8, K)
    x = _rand_bf16(rng, (M, K))
    y = O.grouped_gemm_fwd(x, np.array([0, M]), w, O.FMT_INT8, K, s)
    wq = O.bf16_to_f32(O.fq_weight_stack(w, O.FMT_INT8, K, s).bits)
    ref = O.f64_to_bf16(O.bf16_to_f32(x).astype(np.float64) @ wq[0].T.astype(np.float64))
    assert np.array_equal(y, ref)
    # row independence: permuting the rows permutes the output rows
    p = rng.permutation(M)
    y2 = O.grouped_gemm_fwd(x[p], np.array([0, M]), w, O.FMT_INT8, K, s)
    assert np.array_equal(y2, y[p])
    # power-of-two input scaling scales outputs exactly (A16: no act FQ)
    x4 = O.f32_to_bf16(O.bf16_to_f32(x) * np.float32(4.0))
    y4 = O.grouped_gemm_fwd(x4, np.array([0, M]), w, O.FMT_INT8, K, s)
    assert np.array_equal(O.bf16_to_f32(y4), O.bf16_to_f32(y) * np.float32(4.0))


@pytest.mark.parametrize("T,k,Eg,begin,El", [(37, 8, 16, 0, 16), (50, 4, 32, 8, 8),
                                               (1, 8, 8, 0, 8), (0, 8, 8, 0, 8), (64, 8, 128, 16, 16)])
def test_permute_matches_sorted_brute_force(T, k, Eg, begin, El):
    rng = np.random.default_rng(T + k)
    ids = np.stack([rng.permutation(Eg)[:k] for _ in range(T)]).astype(np.int32) if T else \
        np.zeros((0, k), np.int32)
    perm, row_of, seg = O.moe_permute(ids, begin, El)
    flat = ids.reshape(-1)
    local = [f for f in range(T * k) if begin <= flat[f] < begin + El]
    ref = sorted(local, key=lambda f: (flat[f], f))
    assert list(perm) == ref
    assert seg[0] == 0 and seg[-1] == len(ref) and np.all(np.diff(seg) >= 0)
    for e in range(El):
        assert seg[e + 1] - seg[e] == sum(1 for f in local if flat[f] == begin + e)
    for r, f in enumerate(perm):
        assert row_of.reshape(-1)[f] == r
    assert np.sum(row_of >= 0) == len(ref)


def _tiny_moe(fmt, seed=0):
    case = W.moe_case(T=9, fmt=fmt, E_global=6, H=32, F=16, topk=2, seed=seed)
    return case


@pytest.mark.parametrize("fmt,afmt,group", [("fp8", O.FMT_FP8, None), ("nvfp4", O.FMT_NVFP4, 16),
                                            ("int8", O.FMT_INT8, None), ("int4", O.FMT_FP8, 16),
                                            ("fp8", O.FMT_FP8, O.GROUP_TENSOR)])
def test_moe_chain_matches_per_token_brute_force(fmt, afmt, group):
    case = _tiny_moe(fmt)
    wfmt = O.FMT_NAMES[fmt]
    grp_gu = group or case.w_gu.shape[2]
    grp_d = group or case.w_d.shape[2]
    # one group size per call: per-channel uses K of each stack
    wq_gu = O.observer_weight(case.w_gu, wfmt, grp_gu)
    wq_d = O.observer_weight(case.w_d, wfmt, grp_d)
    out = O.moe_layer(case, wfmt, group, afmt, wq_gu, wq_d)
    # ---- brute force, one (token, slot) at a time
    F = case.w_d.shape[2]
    Wgu = O.bf16_to_f32(O.fq_weight_stack(case.w_gu, wfmt, grp_gu, *wq_gu).bits).astype(np.float64)
    Wd = O.bf16_to_f32(O.fq_weight_stack(case.w_d, wfmt, grp_d, *wq_d).bits).astype(np.float64)
    s1, s2 = out["s_a1"], out["s_a2"]
    T, k = case.expert_ids.shape
    H = case.x.shape[1]
    y = np.zeros((T, H))
    dx = np.zeros((T, H))
    wfq_gu = O.fq_weight_stack(case.w_gu, wfmt, grp_gu, *wq_gu)
    wfq_d = O.fq_weight_stack(case.w_d, wfmt, grp_d, *wq_d)
    ds_gu = np.zeros_like(out["ds_gu"])
    ds_d = np.zeros_like(out["ds_d"])
    ds_a1 = ds_a2 = 0.0
    for t in range(T):
        xq = O.fq_act(case.x[t:t + 1], afmt, s1)
        xv = O.bf16_to_f32(xq.bits)[0].astype(np.float64)
        dxt = np.zeros(H)
        for j in range(k):
            e = case.expert_ids[t, j]
            p = np.float64(case.probs[t, j])
            h = O.f64_to_bf16(Wgu[e] @ xv)
            hv = O.bf16_to_f32(h).astype(np.float64)
            g_, u_ = hv[:F], hv[F:]
            sig = 1 / (1 + np.exp(-g_))
            a = O.f64_to_bf16(g_ * sig * u_)
            aq = O.fq_act(a[None], afmt, s2)
            av = O.bf16_to_f32(aq.bits)[0].astype(np.float64)
            o = O.bf16_to_f32(O.f64_to_bf16(Wd[e] @ av)).astype(np.float64)
            y[t] += p * o
            do = O.bf16_to_f32(O.f64_to_bf16(p * O.bf16_to_f32(case.dout[t]).astype(np.float64)))
            do = do.astype(np.float64)
            da = O.bf16_to_f32(O.f64_to_bf16(do @ Wd[e])).astype(np.float64) * aq.mask[0]
            dgate = da * u_ * sig * (1 + g_ * (1 - sig))
            dup = da * g_ * sig
            dh = O.bf16_to_f32(O.f64_to_bf16(np.concatenate([dgate, dup]))).astype(np.float64)
            dxq_row = O.bf16_to_f32(O.f64_to_bf16(dh @ Wgu[e])).astype(np.float64)
            dxt += dxq_row
            # each routed row's own contribution to the activation-scale gradients
            ds_a1 += float(np.sum(dxq_row * xq.dv_ds[0]))
            ds_a2 += float(np.sum(O.bf16_to_f32(O.f64_to_bf16(do @ Wd[e])) * aq.dv_ds[0]))
            ds_d[e] += (np.outer(do, av) * wfq_d.dv_ds[e]).reshape(ds_d.shape[1:] + (-1,)).sum(-1)
            ds_gu[e] += (np.outer(dh, xv) * wfq_gu.dv_ds[e]).reshape(ds_gu.shape[1:] + (-1,)).sum(-1)
        dx[t] = dxt * xq.mask[0]
    ulp = lambda v: np.abs(O.bf16_to_f32(v)) * 2.0 ** -7 + 1e-30  # noqa: E731
    assert np.all(np.abs(O.bf16_to_f32(out["out"]) - O.bf16_to_f32(O.f64_to_bf16(y))) <= ulp(out["out"]))
    assert np.all(np.abs(O.bf16_to_f32(out["dx"]) - O.bf16_to_f32(O.f64_to_bf16(dx))) <= ulp(out["dx"]))
    for got, ref in ((out["ds_gu"], ds_gu), (out["ds_d"], ds_d)):
        assert np.abs(got - ref).max() <= 1e-9 * np.abs(ref).max()
    if afmt in (O.FMT_FP8, O.FMT_INT8):
        assert abs(out["ds_a1"] - ds_a1) <= 1e-9 * abs(ds_a1) and ds_a1 != 0.0
        assert abs(out["ds_a2"] - ds_a2) <= 1e-9 * abs(ds_a2) and ds_a2 != 0.0
    else:
        assert out["ds_a1"] is None and out["ds_a2"] is None


def test_combine_bwd_is_exact_product():
    # p (fp32) * dOut (bf16) is exact in float64, so the fp32 product then bf16
    # is one correctly rounded multiply followed by RNE
    rng = np.random.default_rng(13)
    T, k, H = 5, 3, 16
    dout = _rand_bf16(rng, (T, H))
    p = rng.random((T, k)).astype(np.float32)
    perm = np.array([4, 0, 7, 14, 2], np.int32)
    do = O.combine_bwd(dout, p, perm, k)
    for r, f in enumerate(perm):
        t, j = divmod(int(f), k)
        ref = O.f32_to_bf16((O.bf16_to_f32(dout[t]) * p[t, j]).astype(np.float32))
        assert np.array_equal(do[r], ref)


def test_silu_special_values():
    h = O.f32_to_bf16(np.array([[0.0, 20.0, -20.0, 1.0, 2.0, 2.0, 2.0, 3.0]], np.float32))
    a = O.bf16_to_f32(O.swiglu_fwd(h))[0]
    # silu(0) = 0; silu(20) ~ 20 (within bf16); silu(-20) ~ -4e-8; silu(1) = 1/(1+e^-1)
    assert a[0] == 0.0
    assert abs(a[1] - 2 * 20.0) <= 2 * 20.0 * 2 ** -8
    assert abs(a[2]) < 1e-6
    ref = 3.0 / (1 + np.exp(-1.0))
    assert abs(a[3] - ref) <= ref * 2 ** -8            # half a bf16 ulp


def test_workloads_are_deterministic_and_shaped():
    a = W.moe_case(T=64, fmt="nvfp4", E_global=16, H=64, F=32, seed=3)
    b = W.moe_case(T=64, fmt="nvfp4", E_global=16, H=64, F=32, seed=3)
    assert np.array_equal(a.w_gu, b.w_gu) and np.array_equal(a.expert_ids, b.expert_ids)
    assert a.w_gu.shape == (16, 64, 64) and a.w_d.shape == (16, 64, 32)
    assert np.allclose(a.probs.sum(1), 1.0, atol=1e-6)
    # each token picks k distinct experts
    assert all(len(set(r)) == a.topk for r in a.expert_ids)
    z = W.moe_case(T=256, fmt="nvfp4", E_global=32, H=32, F=16, seed=1, E_local=8,
                   zipf_s=1.2, zero_experts=(3, 7))
    assert not np.isin(z.expert_ids, [3, 7]).any()
    counts = np.bincount(z.expert_ids.reshape(-1), minlength=32)
    assert counts[0] > counts[20]          # skewed toward low ids
