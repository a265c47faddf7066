"""The hot path captured in a HIP graph (torch.cuda.CUDAGraph over the ABI
calls) and replayed: every replay, with eager work and synchronizations
between the replays, gives the same bits as the eager step. The library
enqueues no memset, copy, allocation or host synchronization inside a call,
so a whole step records as kernels alone."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from helpers import dev_bf16, dev_f32, dev_i32, host_bits

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import moe_fake_quant_amd as F
else:  # collected on CPU only to be deselected by -m "not gpu"
    F = None


def _capture(step):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    return g


def _snapshot(tensors):
    return [t.detach().clone() for t in tensors]


def _same_bits(a, b):
    return all(torch.equal(x.view(torch.uint8), y.view(torch.uint8)) for x, y in zip(a, b))


def test_dense_int8_step_replays_bitwise():
    """FQ pass, forward, dX and dScale of one INT8 per-channel linear
    (the latency-bound dense shape, W [256, 512], 64 rows)."""
    print("[graph] dense int8", flush=True)
    case = W.config(1, seed=0)
    N, K = case.w.shape
    M = case.x.shape[0]
    shape = (1, N, K)
    w, x, dy = dev_bf16(case.w[None]), dev_bf16(case.x), dev_bf16(case.dy)
    s = torch.empty(1, N, 1, device="cuda")
    F.observer_absmax_init(w, shape, F.FMT_INT8, K, 0, s, None, None)
    q = F.WeightQ(F.FMT_INT8, K, s, None, None)
    seg = dev_i32(np.array([0, M]))
    ws = torch.empty(max(F.fq_workspace_bytes(F.FQ_OP_GEMM_FWD, shape, M, 0),
                         F.fq_workspace_bytes(F.FQ_OP_GEMM_BWD, shape, M, 0), 256),
                     dtype=torch.uint8, device="cuda")
    wfq = torch.empty_like(w)
    y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    dx = torch.empty(M, K, dtype=torch.bfloat16, device="cuda")
    ds = torch.empty(1, N, 1, device="cuda")
    outs = (wfq, y, dx, ds)

    def step():
        F.fq_quantize_stacked(w, shape, q, wfq)
        F.fq_grouped_gemm_fwd(x, M, seg, shape, None, wfq, q, None, y, ws)
        F.fq_grouped_gemm_bwd_scale(dy, x, M, seg, shape, w, wfq, q, None, dx, None, None, ws)
        F.fq_grouped_gemm_bwd_scale(dy, x, M, seg, shape, w, wfq, q, None, None, ds, None, ws)

    step()
    torch.cuda.synchronize()
    eager = _snapshot(outs)
    # the eager step itself against the oracle
    wq = O.observer_weight(case.w[None], O.FMT_INT8, K)
    assert np.array_equal(host_bits(wfq)[0], O.fq_weight_stack(case.w[None], O.FMT_INT8, K, *wq).bits[0])
    g = _capture(step)
    for rep in range(4):
        for t in outs:
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert _same_bits(_snapshot(outs), eager), f"replay {rep}"
        step()  # eager work between the replays
        torch.cuda.synchronize()
        assert _same_bits(_snapshot(outs), eager)


@pytest.mark.parametrize("overlap", [False, True])
def test_moe_layer_step_replays_bitwise(overlap):
    """The NVFP4 MoE layer step (routing, FQ pass, forward, scale-only
    backward); with overlap the wgrad calls run on the side stream, whose
    fork and join the capture records as graph dependencies."""
    print(f"[graph] moe step overlap={overlap}", flush=True)
    case = W.moe_case(T=600, fmt="nvfp4", E_global=16, H=256, F=256, topk=4, seed=21,
                      zipf_s=1.2, zero_experts=(5,))
    x, ids = dev_bf16(case.x), dev_i32(case.expert_ids)
    p, dout = dev_f32(case.probs), dev_bf16(case.dout)
    L = F.MoEFakeQuantLayer(dev_bf16(case.w_gu), dev_bf16(case.w_d), F.FMT_NVFP4, F.FMT_NVFP4,
                            case.T, case.topk, 0, 16)
    L.init_weight_scales()
    L.calibrate(x, ids)
    L.overlap_wgrad = overlap
    outs = (L.out[:case.T], L.dx[:case.T], L.ds_gu, L.ds_d, L.wfq_gu, L.wfq_d, L.seg)

    def step():
        L.step(x, ids, p, dout)

    step()
    torch.cuda.synchronize()
    eager = _snapshot(outs)
    g = _capture(step)
    for rep in range(4):
        for t in outs:
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert _same_bits(_snapshot(outs), eager), f"replay {rep}"
        step()
        torch.cuda.synchronize()
        assert _same_bits(_snapshot(outs), eager)
