"""The debug precondition check (fq_validate): valid inputs give status 0;
each planted violation sets exactly its bit and nothing faults. Every bad
value here is read, never used as an index or a divisor."""
import numpy as np
import pytest
import torch

import oracle as O
from helpers import dev_f32, dev_i32

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import moe_fake_quant_amd as F
else:
    F = None


def _status(**kw):
    st = torch.full((1,), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
    F.fq_validate(st, **kw)
    torch.cuda.synchronize()
    return int(st.cpu().numpy().view(np.uint32)[0])


def _good():
    rng = np.random.default_rng(3)
    T, k, Eg = 300, 8, 64
    ids = np.stack([rng.choice(Eg, k, replace=False) for _ in range(T)]).astype(np.int32)
    seg = np.array([0, 10, 10, 250, 300], np.int32)
    E, N, K = 4, 32, 64
    w = O.f32_to_bf16((rng.standard_normal((E, N, K)) * 0.02).astype(np.float32))
    th, _, g = O.observer_weight(w, O.FMT_NVFP4, 16)
    s4, zp4, _ = O.observer_weight(w, O.FMT_INT4, 32)
    return dict(ids=ids, T=T, k=k, Eg=Eg, seg=seg, shape=(E, N, K), th=th, g=g, s4=s4, zp4=zp4)


def _call(c, ids=None, seg=None, q=None, aq=None):
    kw = {}
    if ids is not None:
        kw.update(expert_ids=dev_i32(ids), T=c["T"], topk=c["k"], n_experts=c["Eg"])
    if seg is not None:
        kw.update(seg_offsets=dev_i32(seg), E=len(seg) - 1, R_max=300)
    if q is not None:
        kw.update(shape=c["shape"], wq=q)
    if aq is not None:
        kw.update(aq=aq)
    return _status(**kw)


def _nvfp4(c, th=None, g=None):
    return F.WeightQ(F.FMT_NVFP4, 16, dev_f32(c["th"] if th is None else th), None,
                     dev_f32(c["g"] if g is None else g))


def _int4(c, s=None, zp=None):
    return F.WeightQ(F.FMT_INT4, 32, dev_f32(c["s4"] if s is None else s),
                     dev_f32(c["zp4"] if zp is None else zp), None)


def test_valid_inputs_report_zero():
    c = _good()
    th = c["th"].copy()
    th[0, 0, 0] = 0.0                          # a zero NVFP4 block parameter is allowed
    assert _call(c, ids=c["ids"], seg=c["seg"], q=_nvfp4(c, th=th),
                 aq=F.ActQ(F.FMT_NVFP4, dev_f32([0.01]))) == 0
    assert _call(c, q=_int4(c)) == 0
    assert _call(c, seg=np.array([0, 0, 0, 0, 0], np.int32)) == 0   # all experts empty


def test_each_violation_sets_its_bit():
    c = _good()
    ids = c["ids"].copy()
    ids[7, 3] = c["Eg"]                        # one past the last expert
    assert _call(c, ids=ids) == F.FQ_BAD_EXPERT_ID
    ids = c["ids"].copy()
    ids[299, 0] = -1
    assert _call(c, ids=ids) == F.FQ_BAD_EXPERT_ID
    assert _call(c, seg=np.array([1, 10, 10, 250, 300], np.int32)) == F.FQ_BAD_SEG_START
    assert _call(c, seg=np.array([0, 10, 9, 250, 300], np.int32)) == F.FQ_BAD_SEG_ORDER
    assert _call(c, seg=np.array([0, 10, 10, 250, 301], np.int32)) == F.FQ_BAD_SEG_END
    th = c["th"].copy()
    th[3, 31, 3] = np.nan
    assert _call(c, q=_nvfp4(c, th=th)) == F.FQ_BAD_SCALE
    th = c["th"].copy()
    th[1, 2, 0] = -1.0
    assert _call(c, q=_nvfp4(c, th=th)) == F.FQ_BAD_SCALE
    g = c["g"].copy()
    g[2] = np.inf
    assert _call(c, q=_nvfp4(c, g=g)) == F.FQ_BAD_GLOBAL_SCALE
    s = c["s4"].copy()
    s[0, 5, 1] = 0.0                           # an integer-grid scale must be > 0
    assert _call(c, q=_int4(c, s=s)) == F.FQ_BAD_SCALE
    zp = c["zp4"].copy()
    zp[2, 0, 0] = np.nan
    assert _call(c, q=_int4(c, zp=zp)) == F.FQ_BAD_ZERO_POINT
    assert _call(c, aq=F.ActQ(F.FMT_FP8_E4M3, dev_f32([-1.0]))) == F.FQ_BAD_ACT_SCALE
    # several at once: the bits combine
    ids = c["ids"].copy()
    ids[0, 0] = 1 << 20
    got = _call(c, ids=ids, seg=np.array([0, 10, 9, 250, 300], np.int32),
                aq=F.ActQ(F.FMT_NVFP4, dev_f32([np.nan])))
    assert got == F.FQ_BAD_EXPERT_ID | F.FQ_BAD_SEG_ORDER | F.FQ_BAD_ACT_SCALE
