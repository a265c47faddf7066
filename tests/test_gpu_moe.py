"""GPU parity of the whole routed-expert path of one MoE layer (forward and
scale-only backward through the C ABI), stage by stage against the oracle fed
the GPU's own inputs of that stage, and end to end against the oracle given
the GPU-calibrated activation scales."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from helpers import (bf16_vals, check_act_dscale_tol, check_dscale_per_expert, check_dscale_tol,
                     check_gemm_tol, dev_bf16, dev_f32, dev_i32, host_bits)

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import moe_fake_quant_amd as F
else:
    F = None

CASES = [
    # name, weight fmt, act fmt, group (None = per channel), T, E_global, E_local, begin, zipf,
    # learnable activation scales
    ("fp8", O.FMT_FP8, O.FMT_FP8, None, 300, 8, 8, 0, None, False),
    ("nvfp4", O.FMT_NVFP4, O.FMT_NVFP4, 16, 300, 8, 8, 0, None, False),
    ("nvfp4-local-zipf", O.FMT_NVFP4, O.FMT_NVFP4, 16, 700, 32, 8, 0, 1.2, False),
    ("int4-a16", O.FMT_INT4, O.FMT_NONE, 128, 200, 8, 8, 0, None, False),
    # the other format pairings the pages list, on the same kernels
    ("nvfp4a16", O.FMT_NVFP4, O.FMT_NONE, 16, 260, 8, 8, 0, None, False),
    ("w4afp8", O.FMT_INT4, O.FMT_FP8, 128, 260, 8, 8, 0, None, True),
    ("w8a8-int8", O.FMT_INT8, O.FMT_INT8, None, 260, 8, 8, 0, None, True),
    ("fp8-learn-act-local", O.FMT_FP8, O.FMT_FP8, None, 500, 16, 8, 4, None, True),
    # fp8_static: per-tensor weights and activations
    ("fp8-static", O.FMT_FP8, O.FMT_FP8, O.GROUP_TENSOR, 260, 8, 8, 0, None, True),
]


def _run_layer(case, wfmt, afmt, group, learn=False):
    layer = F.MoEFakeQuantLayer(dev_bf16(case.w_gu), dev_bf16(case.w_d), wfmt, afmt, case.T,
                                case.topk, case.expert_begin, group, learn_act_scales=learn)
    x, ids = dev_bf16(case.x), dev_i32(case.expert_ids)
    p, dout = dev_f32(case.probs), dev_bf16(case.dout)
    layer.init_weight_scales()
    layer.calibrate(x, ids)
    layer.quantize_weights()
    layer.forward(x, ids, p, keep_a=True)
    layer.backward(x, p, dout)
    torch.cuda.synchronize()
    return layer


def _abs_bits(bits):
    return np.asarray(bits, np.uint16) & np.uint16(0x7FFF)


@pytest.mark.parametrize("name,wfmt,afmt,group,T,Eg,El,begin,zipf,learn", CASES)
def test_moe_layer_stagewise_and_end_to_end(name, wfmt, afmt, group, T, Eg, El, begin, zipf,
                                            learn):
    _check_layer(name, wfmt, afmt, group, T, Eg, El, begin, zipf, learn, 256, 256)


@pytest.mark.parametrize("name,wfmt,afmt,group", [("nvfp4", O.FMT_NVFP4, O.FMT_NVFP4, 16),
                                                   ("fp8", O.FMT_FP8, O.FMT_FP8, None)])
def test_moe_layer_small_calls_split_the_contraction(name, wfmt, afmt, group):
    """A small layer (200 tokens x top-4 over 8 experts) with H = 1024 and
    F = 512: the gate_up forward (routed X) and both dgrads have too few
    tiles for the CUs and 16 stages each, so they run split along the
    contraction; every stage still matches the oracle."""
    _check_layer(name + "-split", wfmt, afmt, group, 200, 8, 8, 0, None, False, 1024, 512)


@pytest.mark.parametrize("name,wfmt,afmt,group", [("nvfp4", O.FMT_NVFP4, O.FMT_NVFP4, 16),
                                                  ("w8a8-int8", O.FMT_INT8, O.FMT_INT8, None)])
def test_moe_layer_ffn_not_multiple_of_256(name, wfmt, afmt, group):
    """The whole layer with hidden 272 and expert FFN 208 (2F = 416): every
    GEMM runs on zero-padded copies inside its call; every stage is checked
    against the oracle as in the layer test above."""
    _check_layer(name, wfmt, afmt, group, 300, 8, 8, 0, None, False, 272, 208)


def _check_layer(name, wfmt, afmt, group, T, Eg, El, begin, zipf, learn, H, Fh):
    print(f"[moe] {name} H={H} F={Fh}", flush=True)
    case = W.moe_case(T=T, fmt=name, E_global=Eg, H=H, F=Fh, topk=4, seed=11,
                      expert_begin=begin, E_local=El, zipf_s=zipf,
                      zero_experts=(3,) if zipf else ())
    L = _run_layer(case, wfmt, afmt, group, learn)
    E, k = El, case.topk
    g_gu = group or case.w_gu.shape[2]
    g_d = group or case.w_d.shape[2]
    # weight scales from the GPU observer == oracle observer
    wq_gu = O.observer_weight(case.w_gu, wfmt, g_gu)
    wq_d = O.observer_weight(case.w_d, wfmt, g_d)
    assert np.array_equal(L.q_gu.scale.cpu().numpy(), wq_gu[0])
    assert np.array_equal(L.q_d.scale.cpu().numpy(), wq_d[0])
    # routing
    perm, row_of, seg = O.moe_permute(case.expert_ids, begin, E)
    R = int(seg[-1])
    assert np.array_equal(L.seg.cpu().numpy(), seg)
    assert np.array_equal(L.perm.cpu().numpy()[:R], perm)
    assert np.array_equal(L.row_of.cpu().numpy()[:T], row_of)
    s1 = L.aq1.scale.cpu().numpy()[0]
    s2 = L.aq2.scale.cpu().numpy()[0]
    if afmt:
        assert s1 == O.observer_act(case.x, afmt)
    # stage by stage, each oracle step fed the GPU's inputs of that step.
    # The expert input as token rows: FQ_a of each token once (bit-exact); the
    # gate_up GEMMs read routed row r as token row perm[r] / topk, which is
    # the oracle's gather bit for bit.
    xq_tok = host_bits(L.xq_tok)[:T] if afmt else case.x
    assert np.array_equal(xq_tok, O.fq_act(case.x, afmt, s1).bits)
    xq = xq_tok[perm // k]
    assert np.array_equal(xq, O.gather_actfq(case.x, perm, k, afmt, s1).bits)
    h = host_bits(L.h)[:R]
    check_gemm_tol(h, O.grouped_gemm_fwd(xq, seg, case.w_gu, wfmt, g_gu, *wq_gu), "h")
    a = host_bits(L.a)[:R]
    check_gemm_tol(a, O.swiglu_fwd(h), "a")
    if afmt:
        assert s2 == O.observer_act(a, afmt)
    aq = host_bits(L.aq)[:R]
    assert np.array_equal(aq, O.fq_act(a, afmt, s2).bits)
    o = host_bits(L.o)[:R]
    check_gemm_tol(o, O.grouped_gemm_fwd(aq, seg, case.w_d, wfmt, g_d, *wq_d), "o")
    check_gemm_tol(host_bits(L.out)[:T], O.combine(o, case.probs, row_of), "out")
    do = host_bits(L.do)[:R]
    assert np.array_equal(do, O.combine_bwd(case.dout, case.probs, perm, k))
    daq_ref, ds_d_ref, dzp_d_ref = O.grouped_gemm_bwd(do, aq, seg, case.w_d, wfmt, g_d, *wq_d)
    daq = host_bits(L.daq)[:R]
    check_gemm_tol(daq, daq_ref, "daq")
    check_dscale_tol(L.ds_d.cpu().numpy(), ds_d_ref, "ds_d")
    check_dscale_per_expert(L.ds_d.cpu().numpy(), ds_d_ref, "ds_d")
    dh = host_bits(L.dh)[:R]
    check_gemm_tol(dh, O.swiglu_bwd(daq, h, afmt, s2, a_bits=a), "dh")
    dxq_ref, ds_gu_ref, dzp_gu_ref = O.grouped_gemm_bwd(dh, xq, seg, case.w_gu, wfmt, g_gu, *wq_gu)
    dxq = host_bits(L.dxq)[:R]
    check_gemm_tol(dxq, dxq_ref, "dxq")
    check_dscale_tol(L.ds_gu.cpu().numpy(), ds_gu_ref, "ds_gu")
    check_dscale_per_expert(L.ds_gu.cpu().numpy(), ds_gu_ref, "ds_gu")
    if wfmt == O.FMT_INT4:
        check_dscale_tol(L.dzp_gu.cpu().numpy(), dzp_gu_ref, "dzp_gu")
        check_dscale_tol(L.dzp_d.cpu().numpy(), dzp_d_ref, "dzp_d")
        check_dscale_per_expert(L.dzp_gu.cpu().numpy(), dzp_gu_ref, "dzp_gu")
        check_dscale_per_expert(L.dzp_d.cpu().numpy(), dzp_d_ref, "dzp_d")
    dx = host_bits(L.dx)[:T]
    check_gemm_tol(dx, O.unpermute_reduce(dxq, row_of, case.x, afmt, s1), "dx")
    if learn:
        # activation-scale gradients from the GPU's own dXq / dAq
        fx = O.fq_act(case.x, afmt, s1)
        g1 = O.unpermute_sum(dxq, row_of)
        sc1 = float(np.sum(O.unpermute_sum(_abs_bits(dxq), row_of) * np.abs(fx.dv_ds)))
        ds_a1 = float(L.ds_a1.cpu()[0])
        check_act_dscale_tol(ds_a1, O.act_scale_grad(case.x, g1, afmt, s1), sc1, "ds_a1")
        fa = O.fq_act(a, afmt, s2)
        g2 = bf16_vals(daq)
        sc2 = float(np.sum(np.abs(g2 * fa.dv_ds)))
        ds_a2 = float(L.ds_a2.cpu()[0])
        check_act_dscale_tol(ds_a2, O.act_scale_grad(a, g2, afmt, s2), sc2, "ds_a2")
        # bitwise reproducible: the same backward again
        L.backward(dev_bf16(case.x), dev_f32(case.probs), dev_bf16(case.dout))
        torch.cuda.synchronize()
        assert float(L.ds_a1.cpu()[0]) == ds_a1 and float(L.ds_a2.cpu()[0]) == ds_a2
    # end to end: the oracle's own chain with the GPU-calibrated activation scales
    ref = O.moe_layer(case, wfmt, g_gu if g_gu == g_d else None, afmt, wq_gu, wq_d, (s1, s2)) \
        if g_gu == g_d else None
    if ref is not None:
        check_gemm_tol(host_bits(L.out)[:T], ref["out"], "out e2e")
        check_gemm_tol(dx, ref["dx"], "dx e2e")
        check_dscale_tol(L.ds_gu.cpu().numpy(), ref["ds_gu"], "ds_gu e2e")
        check_dscale_tol(L.ds_d.cpu().numpy(), ref["ds_d"], "ds_d e2e")
        if learn:
            # the oracle's own dXq / dAq differ from the GPU's by GEMM rounding
            check_act_dscale_tol(ds_a1, ref["ds_a1"], sc1, "ds_a1 e2e", tol=1e-2)
            check_act_dscale_tol(ds_a2, ref["ds_a2"], sc2, "ds_a2 e2e", tol=1e-2)


@pytest.mark.parametrize("name,wfmt,afmt,group,learn", [("nvfp4", O.FMT_NVFP4, O.FMT_NVFP4, 16, False),
                                                       ("fp8", O.FMT_FP8, O.FMT_FP8, None, True)])
def test_overlapped_step_is_bitwise_the_serial_step(name, wfmt, afmt, group, learn):
    """layer.step() with the wgrad -> dScale calls on the side stream beside
    the dgrads gives the same bits as the serialized step, twice in a row
    (every kernel is deterministic)."""
    case = W.moe_case(T=700, fmt=name, E_global=16, H=256, F=256, topk=4, seed=13)
    x, ids = dev_bf16(case.x), dev_i32(case.expert_ids)
    p, dout = dev_f32(case.probs), dev_bf16(case.dout)
    outs = []
    for overlap in (False, True):
        L = F.MoEFakeQuantLayer(dev_bf16(case.w_gu), dev_bf16(case.w_d), wfmt, afmt, case.T,
                                case.topk, 0, group, learn_act_scales=learn)
        L.init_weight_scales()
        L.calibrate(x, ids)
        L.overlap_wgrad = overlap
        got = []
        for _ in range(2):
            L.step(x, ids, p, dout)
            torch.cuda.synchronize()
            t = [host_bits(L.out[:case.T]), host_bits(L.dx[:case.T]), L.ds_gu.cpu().numpy(),
                 L.ds_d.cpu().numpy()]
            if learn:
                t += [L.ds_a1.cpu().numpy(), L.ds_a2.cpu().numpy()]
            got.append(t)
        outs.append(got)
    for a, b in zip(outs[0], outs[1]):
        for u, v in zip(a, b):
            assert np.array_equal(np.asarray(u).view(np.uint8), np.asarray(v).view(np.uint8))
