"""GPU parity of the real-quantized export through the C ABI: codes and stored
scale bytes bit-exact against the oracle, and the decode of an export equal
bit for bit to the fake-quant values (both the GPU's own FQ pass and the
oracle's), at test sizes with edge values and at the full bench stacks."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from helpers import dev_bf16, dev_f32, host_bits

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import moe_fake_quant_amd as F
else:  # collected on CPU only to be deselected by -m "not gpu"
    F = None

CASES = [(O.FMT_INT8, 64), (O.FMT_INT8, O.GROUP_TENSOR), (O.FMT_FP8, 256), (O.FMT_FP8, 128),
         (O.FMT_FP8, O.GROUP_TENSOR), (O.FMT_INT4, 128), (O.FMT_INT4, 32), (O.FMT_NVFP4, 16)]


def _w(rng, E, N, K, std=0.02):
    w = rng.standard_normal((E, N, K)).astype(np.float32) * std
    flat = w.reshape(-1)
    idx = rng.choice(flat.size, flat.size // 100, replace=False)
    flat[idx] *= 30.0
    flat[idx[: len(idx) // 4]] = -1e-9
    return O.f32_to_bf16(w)


def _export(wd, shape, fmt, group, s, zp, g):
    """GPU: FQ pass (values + codes), stored scale bytes, decode."""
    E, N, K = shape
    q = F.WeightQ(fmt=fmt, group=group, scale=dev_f32(s),
                  zero_point=None if zp is None else dev_f32(zp),
                  global_scale=None if g is None else dev_f32(g))
    wfq = torch.empty_like(wd)
    nbytes = E * N * K // 2 if fmt in (O.FMT_INT4, O.FMT_NVFP4) else E * N * K
    codes = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    F.fq_quantize_stacked(wd, shape, q, wfq, codes)
    sb = zb = None
    if fmt == O.FMT_NVFP4:
        sb = torch.empty(E * N * K // 16, dtype=torch.uint8, device="cuda")
        F.fq_export_scales(shape, q, sb, None)
    elif fmt == O.FMT_INT4:
        zb = torch.empty(E * N * (K // group), dtype=torch.uint8, device="cuda")
        F.fq_export_scales(shape, q, None, zb)
    out = torch.full_like(wd, 7.0)
    F.fq_dequantize_stacked(codes, shape, fmt, group, out,
                            None if fmt == O.FMT_NVFP4 else q.scale, sb, zb, q.global_scale)
    return wfq, codes, sb, zb, out


@pytest.mark.parametrize("fmt,group", CASES)
def test_export_and_decode_bitexact(fmt, group):
    print(f"[export] fmt={fmt} group={group}", flush=True)
    rng = np.random.default_rng(60 + fmt)
    E, N, K = 3, 40, 512
    w = _w(rng, E, N, K)
    s, zp, g = O.observer_weight(w, fmt, group)
    s = (s * rng.uniform(0.4, 1.1, s.shape)).astype(np.float32)
    if fmt == O.FMT_NVFP4:
        s[0, 0, :3] = 0.0
        s[1, 2, 1] = 700.0
    if fmt == O.FMT_INT4:
        zp = zp.copy()
        zp[0, 0, 0] = 20.0
        zp[2, 3, 1] = -2.0
    wfq, codes, sb, zb, out = _export(dev_bf16(w), (E, N, K), fmt, group, s, zp, g)
    torch.cuda.synchronize()
    fq = O.fq_weight_stack(w, fmt, group, s, zp, g)
    _, sb_ref, zb_ref = O.export_scales(fmt, s, zp)
    assert np.array_equal(codes.cpu().numpy(), O.pack_codes(fq.code, fmt))
    if sb is not None:
        assert np.array_equal(sb.cpu().numpy(), sb_ref.reshape(-1))
    if zb is not None:
        assert np.array_equal(zb.cpu().numpy(), zb_ref.reshape(-1))
    assert torch.equal(out.view(torch.int16), wfq.view(torch.int16))
    assert np.array_equal(host_bits(out), fq.bits)


@pytest.mark.parametrize("cfg", [3, 4])
def test_export_round_trip_full_stacks(cfg):
    """The bench workload's stacks with observer scales: decode(export) equals
    the FQ pass over both whole stacks; one expert's bytes against the oracle."""
    case = W.config(cfg, seed=0)
    fmt = O.FMT_FP8 if cfg == 3 else O.FMT_NVFP4
    print(f"[export] {W.CONFIG_NAMES[cfg]}", flush=True)
    for name, w in (("gate_up", case.w_gu), ("down", case.w_d)):
        E, N, K = w.shape
        group = K if fmt == O.FMT_FP8 else 16
        wd = dev_bf16(w)
        G = K // group
        s = torch.empty(E, N, G, device="cuda")
        g = torch.empty(E, device="cuda") if fmt == O.FMT_NVFP4 else None
        F.observer_absmax_init(wd, (E, N, K), fmt, group, 0, s, None, g)
        torch.cuda.synchronize()
        s_h = s.cpu().numpy()
        g_h = None if g is None else g.cpu().numpy()
        wfq, codes, sb, zb, out = _export(wd, (E, N, K), fmt, group, s_h, None, g_h)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), wfq.view(torch.int16)), name
        e = E - 1
        fq = O.fq_weight_stack(w[e:e + 1], fmt, group, s_h[e:e + 1], None,
                               None if g_h is None else g_h[e:e + 1])
        per_e = N * K // 2 if fmt == O.FMT_NVFP4 else N * K
        assert np.array_equal(codes[e * per_e:(e + 1) * per_e].cpu().numpy(),
                              O.pack_codes(fq.code, fmt)), name
        if sb is not None:
            _, sb_ref, _ = O.export_scales(fmt, s_h[e])
            nb = N * K // 16
            assert np.array_equal(sb[e * nb:(e + 1) * nb].cpu().numpy(), sb_ref.reshape(-1)), name
        assert np.array_equal(host_bits(out[e]), fq.bits[0]), name
