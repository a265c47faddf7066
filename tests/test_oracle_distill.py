"""Pins of the oracle's self-distillation pieces.

(i) The top-K set against a pure-Python sort with many equal logits.
(ii) K = V: the restricted KL is the full-vocabulary KL, which torch's
kl_div of two log_softmax rows gives (library special case), forward and
reverse.
(iii) The student-logit gradient against torch autograd of the written-out
restricted loss (fp64).
(iv) Identical logits give loss 0 and gradient 0; K = 1 gives loss 0.
(v) The valid-token mask: mean over valid tokens only.
(vi) The self-teacher forward against a per-token brute force of the layer
with quantization off.
CPU only."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W


def _logits(rng, T, V, step=0.25):
    """Logits on a coarse grid (many equal values) as bf16 bits."""
    z = np.round(rng.standard_normal((T, V)) * 2.0 / step) * step
    return O.f32_to_bf16(z.astype(np.float32))


def test_topk_set_matches_python_sort_with_ties():
    rng = np.random.default_rng(1)
    t = _logits(rng, 12, 97, step=0.5)
    t[:, ::3] = np.where(rng.random((12, 33)) < 0.5, 0x8000, 0x0000)   # -0 and +0: equal logits
    tv = O.bf16_to_f32(t)
    for K in (1, 5, 30, 97):
        idx = O.topk_set(t, K)
        for r in range(12):
            ref = sorted(sorted(range(97), key=lambda i: (-tv[r, i], i))[:K])
            assert list(idx[r]) == ref


@pytest.mark.parametrize("reverse", [False, True])
def test_full_vocab_case_is_torch_kl_div(reverse):
    rng = np.random.default_rng(2)
    T, V = 7, 64
    s, t = _logits(rng, T, V), _logits(rng, T, V)
    _, _, loss, mean = O.topk_kl(s, t, V, reverse=reverse)
    ls = torch.log_softmax(torch.from_numpy(O.bf16_to_f32(s).astype(np.float64)), -1)
    lt = torch.log_softmax(torch.from_numpy(O.bf16_to_f32(t).astype(np.float64)), -1)
    # kl_div(input, target) = sum target_prob * (log target - input)
    ref = torch.nn.functional.kl_div(lt if reverse else ls, ls if reverse else lt,
                                     reduction="none", log_target=True).sum(-1).numpy()
    assert np.allclose(loss, ref, rtol=1e-12, atol=1e-14)
    assert mean == pytest.approx(ref.mean(), rel=1e-12)


@pytest.mark.parametrize("reverse", [False, True])
def test_gradient_matches_autograd(reverse):
    rng = np.random.default_rng(3)
    T, V, K = 6, 80, 17
    s, t = _logits(rng, T, V), _logits(rng, T, V)
    valid = np.array([1, 1, 0, 1, 1, 1], bool)
    idx, g, loss, mean = O.topk_kl(s, t, K, reverse=reverse, valid=valid)
    st = torch.from_numpy(O.bf16_to_f32(s).astype(np.float64)).requires_grad_(True)
    tt = torch.from_numpy(O.bf16_to_f32(t).astype(np.float64))
    it = torch.from_numpy(idx)
    ls = torch.log_softmax(st.gather(1, it), -1)
    lt = torch.log_softmax(tt.gather(1, it), -1)
    per = (ls.exp() * (ls - lt)).sum(-1) if reverse else (lt.exp() * (lt - ls)).sum(-1)
    vt = torch.from_numpy(valid)
    m = per[vt].sum() / vt.sum()
    m.backward()
    assert mean == pytest.approx(float(m.detach()), rel=1e-12)
    gref = st.grad.gather(1, it).numpy()
    assert np.allclose(g, gref, rtol=1e-10, atol=1e-15)
    # nothing outside the top-K set gets a gradient
    mask = np.ones((T, V), bool)
    np.put_along_axis(mask, idx, False, axis=1)
    assert np.all(st.grad.numpy()[mask] == 0)
    assert np.all(loss[~valid] == 0) and np.all(g[~valid] == 0)


def test_identical_logits_and_single_token():
    rng = np.random.default_rng(4)
    t = _logits(rng, 5, 50)
    for reverse in (False, True):
        _, g, loss, mean = O.topk_kl(t, t, 20, reverse=reverse)
        assert np.all(loss == 0) and np.all(g == 0) and mean == 0
        s = _logits(rng, 5, 50)
        _, g, loss, _ = O.topk_kl(s, t, 1, reverse=reverse)
        assert np.all(loss == 0) and np.all(g == 0)


def test_teacher_forward_matches_per_token_brute_force():
    case = W.moe_case(T=9, fmt="nvfp4", E_global=6, H=32, F=16, topk=2, seed=5)
    out = O.teacher_forward(case)
    wgu = O.bf16_to_f32(case.w_gu).astype(np.float64)
    wd = O.bf16_to_f32(case.w_d).astype(np.float64)
    F = wd.shape[2]
    ref = np.zeros((case.x.shape[0], wd.shape[1]))
    for t in range(case.x.shape[0]):
        x = O.bf16_to_f32(case.x[t]).astype(np.float64)
        for j in range(case.expert_ids.shape[1]):
            e = case.expert_ids[t, j]
            h = O.bf16_to_f32(O.f64_to_bf16(wgu[e] @ x)).astype(np.float64)
            g, u = h[:F], h[F:]
            a = O.bf16_to_f32(O.f64_to_bf16(g / (1 + np.exp(-g)) * u)).astype(np.float64)
            o = O.bf16_to_f32(O.f64_to_bf16(wd[e] @ a)).astype(np.float64)
            ref[t] += np.float64(case.probs[t, j]) * o
    got = O.bf16_to_f32(out)
    assert np.all(np.abs(got - O.bf16_to_f32(O.f64_to_bf16(ref))) <= np.abs(got) * 2.0 ** -7 + 1e-30)
