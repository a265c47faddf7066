"""GPU parity of the self-distillation pieces through the C ABI: the layer's
quantization-off teacher forward, and the top-K KL kernel (top-K set
bit-exact, loss and student-logit gradient to the stated tolerances) at test
sizes with equal logits, signed zeros, invalid tokens and K = 1 / K = V, and
at the full distillation workload on sampled tokens."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from helpers import check_gemm_tol, dev_bf16, dev_f32, dev_i32, host_bits

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import moe_fake_quant_amd as F
else:  # collected on CPU only to be deselected by -m "not gpu"
    F = None

# Loss and gradient tolerance. Each restricted log-softmax entry carries an
# absolute error of a few 2^-24 times (|l| + |lse| + 1) (fp32 sums and the
# hardware exp / log); an entry's probability inherits it as a relative error,
# and the loss / gradient sums weight it by the probabilities.
KL_TOL = 4e-6


def _run(s_bits, t_bits, K, reverse, valid=None):
    T, V = t_bits.shape
    s, t = dev_bf16(s_bits), dev_bf16(t_bits)
    idx = torch.full((T, K), -7, dtype=torch.int32, device="cuda")
    g = torch.full((T, K), 7.0, device="cuda")
    lt = torch.full((T,), 7.0, device="cuda")
    lm = torch.full((1,), 7.0, device="cuda")
    ws = torch.empty(F.fq_workspace_bytes(F.FQ_OP_TOPK_KL, (1, 1, 1), 0, 0), dtype=torch.uint8,
                     device="cuda")
    vd = None if valid is None else torch.from_numpy(valid.astype(np.uint8)).cuda()
    F.fq_topk_kl(s, t, T, V, K, reverse, vd, idx, g, lt, lm, ws)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), g.cpu().numpy(), lt.cpu().numpy(), float(lm.cpu()[0])


def _check(s_bits, t_bits, K, reverse, valid, got, n_scale=None):
    """got = (idx, grad, loss_tok, loss_mean) of the GPU on these rows; n_scale:
    the GPU's valid-token count when the rows are a sample of a larger batch."""
    idx, g, lt, lm = got
    ridx, rg, rl, rm = O.topk_kl(s_bits, t_bits, K, reverse=reverse, valid=valid)
    assert np.array_equal(idx, ridx)
    zs = np.take_along_axis(O.bf16_to_f32(s_bits).astype(np.float64), ridx, 1)
    zt = np.take_along_axis(O.bf16_to_f32(t_bits).astype(np.float64), ridx, 1)
    lse = lambda z: z.max(1, keepdims=True) + np.log(np.exp(z - z.max(1, keepdims=True)).sum(1, keepdims=True))  # noqa: E731
    ls, ltt = zs - lse(zs), zt - lse(zt)
    ps, pt = np.exp(ls), np.exp(ltt)
    mag = 1 + np.abs(ls) + np.abs(ltt) + np.abs(lse(zs)) + np.abs(lse(zt))
    row_b = ((ps + pt) * mag * (1 + np.abs(ls - ltt))).sum(1)
    assert np.all(np.abs(lt - rl) <= KL_TOL * row_b), np.abs(lt - rl).max()
    n_ref = max(int(np.sum(valid)) if valid is not None else len(rl), 1)
    n_gpu = n_scale or n_ref
    eb = KL_TOL * (ps + pt) * mag * (1 + np.abs(ls - ltt) + np.abs(rl)[:, None]) + 1e-12
    assert np.all(np.abs(g * n_gpu - rg * n_ref) <= eb), np.abs(g * n_gpu - rg * n_ref).max()
    if n_scale is None:
        assert abs(lm - rm) <= KL_TOL * row_b.sum() / n_ref


def _ties(rng, T, V, step):
    z = rng.standard_normal((T, V)) * 2.0
    if step:
        z = np.round(z / step) * step
    b = O.f32_to_bf16(z.astype(np.float32))
    b[b == 0] = np.where(rng.random(np.sum(b == 0)) < 0.5, 0x8000, 0)   # signed zeros
    return b


@pytest.mark.parametrize("reverse", [False, True])
@pytest.mark.parametrize("K,V,step", [(100, 8000, 0.25), (1, 4096, 0.5), (4096, 8 * 1031, 0.0),
                                      (512, 512, 0.125), (777, 20008, 1.0),
                                      (1024, 8 * 751, 0.25), (1025, 8 * 751, 0.25)])
def test_topk_kl_parity(K, V, step, reverse):
    """K = 1024 and 1025 sit either side of the smaller selection-storage
    instance of the kernel."""
    print(f"[kd] K={K} V={V} step={step} reverse={reverse}", flush=True)
    rng = np.random.default_rng(K + V)
    T = 37
    t = _ties(rng, T, V, step)
    s = O.f32_to_bf16((O.bf16_to_f32(t) + rng.standard_normal((T, V)) * 0.3).astype(np.float32))
    valid = rng.random(T) < 0.8
    valid[0] = True
    got = _run(s, t, K, reverse, valid)
    _check(s, t, K, reverse, valid, got)
    assert np.all(got[1][~valid] == 0) and np.all(got[2][~valid] == 0)
    again = _run(s, t, K, reverse, valid)                 # bitwise reproducible
    for a, b in zip(got[:3], again[:3]):
        assert np.array_equal(a, b)
    assert got[3] == again[3]


def test_topk_kl_identical_logits_and_all_equal_rows():
    rng = np.random.default_rng(9)
    T, V, K = 8, 4096, 300
    t = _ties(rng, T, V, 0.5)
    t[3] = O.f32_to_bf16(np.full(V, 1.25, np.float32))   # every logit equal: the first K
    idx, g, lt, lm = _run(t, t, K, False)
    assert np.all(lt == 0) and np.all(g == 0) and lm == 0
    assert np.array_equal(idx[3], np.arange(K))
    assert np.array_equal(idx, O.topk_set(t, K))


@pytest.mark.parametrize("reverse", [False, True])
def test_topk_kl_negative_and_positive_bounds(reverse):
    """Rows whose K-th largest logit is negative (log-probability-like rows:
    every logit < 0) take the general key compare in the stream; rows with a
    positive one take the raw-bits compare; both in one launch, with ties and
    signed zeros."""
    print(f"[kd] negative / positive bounds reverse={reverse}", flush=True)
    rng = np.random.default_rng(31)
    T, V, K = 12, 8 * 2503, 211
    t = _ties(rng, T, V, 0.25)
    z = O.bf16_to_f32(t).astype(np.float64)
    neg = np.arange(T) % 2 == 1
    z[neg] = -np.abs(z[neg]) - 3.0                        # every logit negative
    z[4] = -np.abs(z[4])                                  # 100 positives, then half zeros:
    z[4, :V // 2] = 0.0                                   # the K-th largest is +-0
    z[4, rng.choice(V, 100, replace=False)] = 1.5
    t = O.f32_to_bf16(z.astype(np.float32))
    t[4, :V // 2] = np.where(rng.random(V // 2) < 0.5, 0x8000, 0)
    s = O.f32_to_bf16((O.bf16_to_f32(t) + rng.standard_normal((T, V)) * 0.3).astype(np.float32))
    got = _run(s, t, K, reverse)
    _check(s, t, K, reverse, None, got)


def test_topk_kl_long_rows():
    """Rows longer than 8 x 65536 entries: the candidate list holds plain
    vocabulary indices (a wave's stretch of the row no longer fits the packed
    16-bit index) and the keys are read again from the teacher row."""
    print("[kd] long rows", flush=True)
    rng = np.random.default_rng(5)
    T, V, K = 3, 8 * 65600, 1000
    t = _ties(rng, T, V, 0.0)
    s = O.f32_to_bf16((O.bf16_to_f32(t) + rng.standard_normal((T, V)) * 0.3).astype(np.float32))
    got = _run(s, t, K, False)
    _check(s, t, K, False, None, got)


@pytest.mark.parametrize("reverse", [False, True])
def test_topk_kl_histogram_path(reverse):
    """Rows whose sampled bracket admits more candidates than LDS holds (long
    runs of equal logits) take the histogram selection; mixed with rows that
    take the sampled path in the same launch."""
    print(f"[kd] histogram path reverse={reverse}", flush=True)
    rng = np.random.default_rng(77)
    T, V, K = 6, 16384 + 8 * 37, 300
    t = _ties(rng, T, V, 0.25)
    t[1] = O.f32_to_bf16(np.full(V, -0.5, np.float32))                 # all equal
    z = np.where(rng.random(V) < 0.7, 2.0, rng.standard_normal(V))      # 70 % tied at the top
    t[3] = O.f32_to_bf16(z.astype(np.float32))
    s = O.f32_to_bf16((O.bf16_to_f32(t) + rng.standard_normal((T, V)) * 0.3).astype(np.float32))
    got = _run(s, t, K, reverse)
    _check(s, t, K, reverse, None, got)
    assert np.array_equal(got[0][1], np.arange(K))


def test_topk_kl_full_workload_sampled():
    """kd-topk1000-t4096-v151936: the whole batch on the GPU, sampled tokens
    against the oracle, the mean against the GPU's own per-token losses."""
    T, V, K = W.KD_TOKENS, W.KD_VOCAB, W.KD_TOPK
    print(f"[kd] {W.KD_NAME}", flush=True)
    s, t = W.kd_logits(T, V, seed=0, device="cuda")
    idx = torch.empty(T, K, dtype=torch.int32, device="cuda")
    g = torch.empty(T, K, device="cuda")
    lt = torch.empty(T, device="cuda")
    lm = torch.empty(1, device="cuda")
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    for reverse in (False, True):
        F.fq_topk_kl(s, t, T, V, K, reverse, None, idx, g, lt, lm, ws)
        torch.cuda.synchronize()
        rng = np.random.default_rng(reverse)
        rows = np.unique(np.concatenate([[0, T - 1], rng.choice(T, 22, replace=False)]))
        rt = torch.from_numpy(rows).cuda()
        sb, tb = host_bits(s[rt]), host_bits(t[rt])
        got = (idx[rt].cpu().numpy(), g[rt].cpu().numpy(), lt[rt].cpu().numpy(), None)
        _check(sb, tb, K, reverse, None, got, n_scale=T)
        ltf = lt.cpu().numpy().astype(np.float64)
        assert abs(float(lm.cpu()[0]) - ltf.mean()) <= 1e-5 * np.abs(ltf).mean()
        assert ltf.min() >= -1e-6 and ltf.mean() > 0


def test_teacher_forward_is_quantization_off():
    case = W.moe_case(T=300, fmt="nvfp4", E_global=8, H=256, F=256, topk=4, seed=13)
    L = F.MoEFakeQuantLayer(dev_bf16(case.w_gu), dev_bf16(case.w_d), F.FMT_NVFP4, F.FMT_NVFP4,
                            case.T, case.topk, 0, 16)
    x, ids, p = dev_bf16(case.x), dev_i32(case.expert_ids), dev_f32(case.probs)
    L.init_weight_scales()
    L.calibrate(x, ids)
    L.quantize_weights()
    out_s = L.forward(x, ids, p).clone()
    out_t = L.teacher_forward(x, ids, p)
    torch.cuda.synchronize()
    check_gemm_tol(host_bits(out_t), O.teacher_forward(case), "teacher out")
    # the student's forward buffers are untouched by the teacher
    assert torch.equal(L.out[:case.T].view(torch.int16), out_s.view(torch.int16))
    assert not torch.equal(out_t.view(torch.int16), out_s.view(torch.int16))
