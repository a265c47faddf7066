"""The allocation-free permute entry point against the workspace one.

fq_moe_permute_noalloc keeps its scratch in a static device array inside the
library; its results must equal fq_moe_permute's bit for bit (integer work),
also on a second call right after a larger one, which leaves its counts in
that array. Both are called through the C ABI.
"""
import numpy as np
import pytest
import torch

import moe_fake_quant_amd as F

pytestmark = pytest.mark.gpu


def _run(fn_ws, ids, T, topk, ebegin, E):
    dev = ids.device
    perm = torch.full((max(T * topk, 1),), -7, dtype=torch.int32, device=dev)
    row_of = torch.full((max(T, 1), topk), -7, dtype=torch.int32, device=dev)
    seg = torch.full((E + 1,), -7, dtype=torch.int32, device=dev)
    fn_ws(perm, row_of, seg)
    torch.cuda.synchronize()
    return perm.cpu().numpy(), row_of.cpu().numpy(), seg.cpu().numpy()


def _ids(T, topk, E_global, seed, dev):
    g = torch.Generator().manual_seed(seed)
    # distinct experts per token: the top-k of random scores
    s = torch.rand(T, E_global, generator=g)
    return torch.topk(s, topk, dim=1).indices.to(torch.int32).contiguous().to(dev)


@pytest.mark.parametrize("order", ["large_then_small"])
def test_noalloc_permute_matches_workspace_permute(order):
    assert torch.cuda.is_available()
    dev = torch.device("cuda:0")
    cases = [(16384, 8, 128, 0, 128, 0),     # the bench routing size, all experts local
             (1000, 8, 128, 32, 16, 1)]      # smaller, a 16-expert local share
    ws = torch.empty(F.fq_workspace_bytes(F.FQ_OP_PERMUTE, (128, 0, 0), 16384 * 8, 0),
                     dtype=torch.uint8, device=dev)
    for T, topk, E_global, ebegin, E, seed in cases:
        ids = _ids(T, topk, E_global, seed, dev)
        ref = _run(lambda p, r, s: F.fq_moe_permute(ids, T, topk, ebegin, E, p, r, s, ws),
                   ids, T, topk, ebegin, E)
        got = _run(lambda p, r, s: F.fq_moe_permute_noalloc(ids, T, topk, ebegin, E, p, r, s),
                   ids, T, topk, ebegin, E)
        R = int(ref[2][-1])
        assert np.array_equal(got[2], ref[2])            # seg_offsets
        assert np.array_equal(got[0][:R], ref[0][:R])    # perm
        assert np.array_equal(got[1][:T], ref[1][:T])    # row_of
        assert R == int(((ids >= ebegin) & (ids < ebegin + E)).sum())


def test_noalloc_permute_rejects_requests_beyond_its_scratch():
    dev = torch.device("cuda:0")
    T, topk, E = 262144, 8, 1024     # 4 * 1024 * (8192 + 1) bytes > 4 MiB
    ids = torch.zeros(T, topk, dtype=torch.int32, device=dev)
    perm = torch.empty(T * topk, dtype=torch.int32, device=dev)
    row_of = torch.empty(T, topk, dtype=torch.int32, device=dev)
    seg = torch.empty(E + 1, dtype=torch.int32, device=dev)
    with pytest.raises(F.FQError) as ei:
        F.fq_moe_permute_noalloc(ids, T, topk, 0, E, perm, row_of, seg)
    assert ei.value.status == F.FQ_ERR_WORKSPACE_TOO_SMALL
    assert "scratch" in str(ei.value)
