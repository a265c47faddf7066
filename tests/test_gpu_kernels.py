"""GPU parity of each libfq entry point against the CPU oracle on identical
inputs (bit-exact for codes, fake-quant values, observer outputs and the
permutation; the stated tolerances for GEMM outputs, dX and dScale).
Calls go through the C ABI (ctypes binding)."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from helpers import (bf16_vals, check_dscale_per_expert, check_dscale_tol, check_gemm_tol,
                     dev_bf16, dev_f32, dev_i32, host_bits)

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import moe_fake_quant_amd as F
else:  # collected on CPU only to be deselected by -m "not gpu"
    F = None

FMTS = [("int8", O.FMT_INT8), ("int4", O.FMT_INT4), ("fp8", O.FMT_FP8), ("nvfp4", O.FMT_NVFP4)]


def _group(fmt, K):
    return {O.FMT_INT8: K, O.FMT_FP8: K, O.FMT_INT4: 128, O.FMT_NVFP4: 16}[fmt]


def _rand_w(rng, E, N, K, std=0.02):
    w = rng.standard_normal((E, N, K)).astype(np.float32) * std
    # outliers, exact zeros, negative zeros, tiny values
    flat = w.reshape(-1)
    idx = rng.choice(flat.size, flat.size // 200, replace=False)
    flat[idx] *= 20.0
    flat[idx[: len(idx) // 4]] = 0.0
    flat[idx[len(idx) // 4: len(idx) // 2]] = -0.0
    flat[idx[len(idx) // 2: 3 * len(idx) // 4]] *= 1e-6
    return O.f32_to_bf16(w)


def _wq(fmt, group, s, zp, g):
    return F.WeightQ(fmt=fmt, group=group, scale=dev_f32(s),
                     zero_point=None if zp is None else dev_f32(zp),
                     global_scale=None if g is None else dev_f32(g))


# --------------------------------------------------------------- FQ pass --
@pytest.mark.parametrize("name,fmt", FMTS)
def test_quantize_stacked_bitexact_observer_scales(name, fmt):
    rng = np.random.default_rng(100 + fmt)
    E, N, K = 3, 48, 256
    group = _group(fmt, K)
    w = _rand_w(rng, E, N, K)
    s, zp, g = O.observer_weight(w, fmt, group)
    s = (s * rng.uniform(0.5, 1.2, s.shape)).astype(np.float32)    # saturate some elements
    if fmt == O.FMT_NVFP4:
        s[0, 0, :2] = 0.0          # zero blocks
        s[1, 1, 0] = 600.0         # above the E4M3 max
    ref = O.fq_weight_stack(w, fmt, group, s, zp, g)
    wd = dev_bf16(w)
    out = torch.empty_like(wd)
    ncode = E * N * K if fmt in (O.FMT_INT8, O.FMT_FP8) else E * N * K // 2
    codes = torch.zeros(ncode, dtype=torch.uint8, device="cuda")
    F.fq_quantize_stacked(wd, (E, N, K), _wq(fmt, group, s, zp, g), out, codes)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(out), ref.bits)
    assert np.array_equal(codes.cpu().numpy(), O.pack_codes(ref.code, fmt))


@pytest.mark.parametrize("name,fmt", FMTS)
def test_quantize_stacked_bitexact_grid_ties(name, fmt):
    """Power-of-two scales, weights at grid points and exact midpoints (ties)."""
    rng = np.random.default_rng(200 + fmt)
    E, N, K = 2, 32, 256
    group = _group(fmt, K)
    G = K // group
    zp = g = None
    if fmt == O.FMT_INT8:
        grid = np.arange(-128, 128, dtype=np.float64)
        mids = np.arange(-128, 127) + 0.5
    elif fmt == O.FMT_INT4:
        grid = np.arange(-8, 8, dtype=np.float64)
        mids = np.arange(-8, 7) + 0.5
        zp = np.full((E, N, G), 8.0, np.float32)
    elif fmt == O.FMT_FP8:
        grid = O.e4m3_value_of_code(np.array([c for c in range(256) if c & 0x7F != 0x7F]))
        pos = np.unique(np.abs(grid))
        mids = np.concatenate([(pos[:-1] + pos[1:]) / 2, -(pos[:-1] + pos[1:]) / 2])
    else:
        pos = O.E2M1_POS
        grid = np.concatenate([pos, -pos])
        mids = np.concatenate([(pos[:-1] + pos[1:]) / 2, -(pos[:-1] + pos[1:]) / 2])
    vals = np.concatenate([grid, mids, [8192.0, -8192.0]])   # saturating, bf16-exact
    z = rng.choice(vals, (E, N, K))
    if fmt == O.FMT_NVFP4:
        s = np.full((E, N, G), 2.0 ** -3, np.float32)
        g = np.full(E, 2.0 ** -4, np.float32)
        eff = 2.0 ** -7
    else:
        s = np.full((E, N, G), 2.0 ** -7, np.float32)
        eff = 2.0 ** -7
    w = O.f32_to_bf16((z * eff).astype(np.float32))
    assert np.array_equal(bf16_vals(w), z * eff)       # exactly representable
    ref = O.fq_weight_stack(w, fmt, group, s, zp, g)
    out = torch.empty(E, N, K, dtype=torch.bfloat16, device="cuda")
    F.fq_quantize_stacked(dev_bf16(w), (E, N, K), _wq(fmt, group, s, zp, g), out, None)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(out), ref.bits)


# -------------------------------------------------------------- observer --
@pytest.mark.parametrize("name,fmt", FMTS)
@pytest.mark.parametrize("per_channel", [True, False])
def test_observer_weight_bitexact(name, fmt, per_channel):
    if fmt == O.FMT_NVFP4 and per_channel:
        pytest.skip("nvfp4 scales are per 16-block")
    rng = np.random.default_rng(300 + fmt)
    E, N = 3, 40
    K = 1024 if per_channel else 512     # per-channel 1024: one block per row
    group = K if per_channel else (16 if fmt == O.FMT_NVFP4 else 128 if fmt == O.FMT_INT4 else 32)
    w = _rand_w(rng, E, N, K)
    w[1, 2] = 0                      # an all-zero row
    s_ref, zp_ref, g_ref = O.observer_weight(w, fmt, group)
    G = K // group
    s = torch.full((E, N, G), -1.0, device="cuda")
    zp = torch.full((E, N, G), -1.0, device="cuda") if fmt == O.FMT_INT4 else None
    g = torch.full((E,), -1.0, device="cuda") if fmt == O.FMT_NVFP4 else None
    F.observer_absmax_init(dev_bf16(w), (E, N, K), fmt, group, 0, s, zp, g)
    torch.cuda.synchronize()
    assert np.array_equal(s.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    if zp is not None:
        assert np.array_equal(zp.cpu().numpy(), zp_ref)
    if g is not None:
        assert np.array_equal(g.cpu().numpy().view(np.uint32), g_ref.view(np.uint32))


@pytest.mark.parametrize("name,fmt", [("fp8", O.FMT_FP8), ("nvfp4", O.FMT_NVFP4), ("int8", O.FMT_INT8)])
def test_observer_activation_bitexact(name, fmt):
    rng = np.random.default_rng(400 + fmt)
    x = O.f32_to_bf16(rng.standard_normal((333, 64)).astype(np.float32))
    s = torch.zeros(1, device="cuda")
    F.observer_absmax_init(dev_bf16(x), (1, 333, 64), fmt, 16, 1, s)
    torch.cuda.synchronize()
    assert s.cpu().numpy()[0] == O.observer_act(x, fmt)


# --------------------------------------------------------------- permute --
@pytest.mark.parametrize("T,k,Eg,begin,El,zipf", [
    (1000, 8, 128, 0, 128, None), (777, 8, 128, 16, 16, None), (5000, 8, 128, 0, 16, 1.2),
    (1, 8, 16, 0, 16, None), (0, 8, 16, 0, 16, None), (300, 2, 6, 0, 6, None)])
def test_permute_bitexact(T, k, Eg, begin, El, zipf):
    if T > 0:
        case = W.moe_case(T=T, fmt="nvfp4", E_global=Eg, H=16, F=16, topk=k, seed=T,
                          expert_begin=begin, E_local=El, zipf_s=zipf,
                          zero_experts=(3, 7) if zipf else ())
        ids = case.expert_ids
    else:
        ids = np.zeros((0, k), np.int32)
    perm_ref, row_ref, seg_ref = O.moe_permute(ids, begin, El)
    P = max(T * k, 1)
    perm = torch.full((P,), -7, dtype=torch.int32, device="cuda")
    row_of = torch.full((max(T, 1), k), -7, dtype=torch.int32, device="cuda")
    seg = torch.full((El + 1,), -7, dtype=torch.int32, device="cuda")
    wsb = F.fq_workspace_bytes(F.FQ_OP_PERMUTE, (El, 0, 0), T * k, 0)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    F.fq_moe_permute(dev_i32(ids) if T else None, T, k, begin, El, perm, row_of, seg, ws)
    torch.cuda.synchronize()
    R = int(seg_ref[-1])
    assert np.array_equal(seg.cpu().numpy(), seg_ref)
    assert np.array_equal(perm.cpu().numpy()[:R], perm_ref)
    if T:
        assert np.array_equal(row_of.cpu().numpy(), row_ref)


# ---------------------------------------------------- grouped GEMM forward --
def _segments(rng, E, sizes):
    seg = np.zeros(E + 1, np.int32)
    seg[1:] = np.cumsum(sizes)
    return seg


@pytest.mark.parametrize("name,fmt", FMTS)
@pytest.mark.parametrize("afmt", [O.FMT_NONE, O.FMT_FP8, O.FMT_NVFP4])
def test_gemm_fwd_parity(name, fmt, afmt):
    rng = np.random.default_rng(500 + 10 * fmt + afmt)
    E, N, K = 5, 512, 384 if fmt != O.FMT_INT4 else 512
    sizes = [70, 0, 300, 1, 257]                      # empty, single-row, multi-tile, ragged
    seg = _segments(rng, E, sizes)
    R = int(seg[-1])
    R_max = R + 40
    group = _group(fmt, K)
    w = _rand_w(rng, E, N, K)
    s, zp, g = O.observer_weight(w, fmt, group)
    x = O.f32_to_bf16(rng.standard_normal((R_max, K)).astype(np.float32))
    sa = O.observer_act(x[:R], afmt) if afmt else np.float32(1.0)
    y_ref = O.grouped_gemm_fwd(x, seg, w, fmt, group, s, zp, g, afmt, sa)
    y = torch.full((R_max, N), 7.0, dtype=torch.bfloat16, device="cuda")
    wq = _wq(fmt, group, s, zp, g)
    aq = F.ActQ(afmt, dev_f32([sa])) if afmt else None
    wsb = F.fq_workspace_bytes(F.FQ_OP_GEMM_FWD, (E, N, K), R_max, fmt | (afmt << 8))
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
    F.fq_grouped_gemm_fwd(dev_bf16(x), R_max, dev_i32(seg), (E, N, K), dev_bf16(w), None, wq, aq,
                          y, ws)
    torch.cuda.synchronize()
    yb = host_bits(y)
    check_gemm_tol(yb[:R], y_ref, "y")
    assert np.all(bf16_vals(yb[R:]) == 7.0)           # rows past R untouched


def test_gemm_fwd_prequantized_weights_match():
    """w_fq from fq_quantize_stacked gives the same bits as the in-call FQ."""
    rng = np.random.default_rng(600)
    E, N, K = 3, 256, 256
    seg = _segments(rng, E, [100, 200, 50])
    R = int(seg[-1])
    w = _rand_w(rng, E, N, K)
    s, _, g = O.observer_weight(w, O.FMT_NVFP4, 16)
    x = O.f32_to_bf16(rng.standard_normal((R, K)).astype(np.float32))
    wq = _wq(O.FMT_NVFP4, 16, s, None, g)
    wd = dev_bf16(w)
    wfq = torch.empty_like(wd)
    F.fq_quantize_stacked(wd, (E, N, K), wq, wfq)
    ws = torch.empty(F.fq_workspace_bytes(F.FQ_OP_GEMM_FWD, (E, N, K), R, O.FMT_NVFP4),
                     dtype=torch.uint8, device="cuda")
    y1 = torch.empty(R, N, dtype=torch.bfloat16, device="cuda")
    y2 = torch.empty_like(y1)
    F.fq_grouped_gemm_fwd(dev_bf16(x), R, dev_i32(seg), (E, N, K), wd, None, wq, None, y1, ws)
    # the same workspace: a call this small splits its contraction when the
    # workspace holds the parts' sums, and runs unsplit without them
    F.fq_grouped_gemm_fwd(dev_bf16(x), R, dev_i32(seg), (E, N, K), None, wfq, wq, None, y2, ws)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    # rows are independent: a row's output does not depend on its neighbours
    x2 = x.copy()
    x2[1::2] = 0
    y3 = torch.empty_like(y1)
    F.fq_grouped_gemm_fwd(dev_bf16(x2), R, dev_i32(seg), (E, N, K), None, wfq, wq, None, y3, ws)
    torch.cuda.synchronize()
    assert torch.equal(y3[0::2].view(torch.int16), y2[0::2].view(torch.int16))


# --------------------------------------------------- grouped GEMM backward --
@pytest.mark.parametrize("name,fmt", FMTS)
@pytest.mark.parametrize("afmt", [O.FMT_NONE, O.FMT_FP8, O.FMT_NVFP4])
@pytest.mark.parametrize("grouping", ["default", "per_channel", "g16", "g32"])
def test_gemm_bwd_parity(name, fmt, afmt, grouping):
    if grouping == "per_channel" and fmt in (O.FMT_NVFP4, O.FMT_INT4):
        pytest.skip("block / group formats")
    if grouping in ("g16", "g32") and fmt == O.FMT_NVFP4:
        pytest.skip("nvfp4 blocks are always 16")
    rng = np.random.default_rng(700 + 10 * fmt + afmt)
    E, N, K = 4, 256, 512
    sizes = [90, 0, 301, 33]
    seg = _segments(rng, E, sizes)
    R = int(seg[-1])
    R_max = R + 17
    group = K if grouping == "per_channel" else _group(fmt, K)
    if fmt in (O.FMT_INT8, O.FMT_FP8) and grouping == "default":
        group = 64
    if grouping in ("g16", "g32"):
        group = int(grouping[1:])
    w = _rand_w(rng, E, N, K)
    s, zp, g = O.observer_weight(w, fmt, group)
    s = (s * rng.uniform(0.7, 1.1, s.shape)).astype(np.float32)
    x = O.f32_to_bf16(rng.standard_normal((R_max, K)).astype(np.float32))
    dy = O.f32_to_bf16(rng.standard_normal((R_max, N)).astype(np.float32))
    sa = O.observer_act(x[:R], afmt) if afmt else np.float32(1.0)
    if afmt:
        sa = np.float32(sa * 0.8)          # some activations clamp: mask zeros in dX
    dx_ref, ds_ref, dzp_ref = O.grouped_gemm_bwd(dy, x, seg, w, fmt, group, s, zp, g, afmt, sa)
    wq = _wq(fmt, group, s, zp, g)
    aq = F.ActQ(afmt, dev_f32([sa])) if afmt else None
    G = K // group
    dx = torch.full((R_max, K), 7.0, dtype=torch.bfloat16, device="cuda")
    ds = torch.full((E, N, G), 7.0, device="cuda")
    dzp = torch.full((E, N, G), 7.0, device="cuda") if fmt == O.FMT_INT4 else None
    wsb = F.fq_workspace_bytes(F.FQ_OP_GEMM_BWD, (E, N, K), R_max, fmt | (afmt << 8))
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    F.fq_grouped_gemm_bwd_scale(dev_bf16(dy), dev_bf16(x), R_max, dev_i32(seg), (E, N, K),
                                dev_bf16(w), None, wq, aq, dx, ds, dzp, ws)
    torch.cuda.synchronize()
    dxb = host_bits(dx)
    check_gemm_tol(dxb[:R], dx_ref, "dx")
    assert np.all(bf16_vals(dxb[R:]) == 7.0)
    dsh = ds.cpu().numpy()
    check_dscale_tol(dsh, ds_ref, "dscale")
    check_dscale_per_expert(dsh, ds_ref, "dscale")
    assert np.all(dsh[1] == 0)                         # empty expert
    if dzp is not None:
        check_dscale_tol(dzp.cpu().numpy(), dzp_ref, "dzero_point")
        check_dscale_per_expert(dzp.cpu().numpy(), dzp_ref, "dzero_point")


@pytest.mark.parametrize("name,fmt,group", [("nvfp4", O.FMT_NVFP4, 16), ("int4", O.FMT_INT4, 128),
                                            ("int4_g16", O.FMT_INT4, 16),
                                            ("int8_g32", O.FMT_INT8, 32),
                                            ("fp8_pc", O.FMT_FP8, 256)])
def test_gemm_bwd_rows_beyond_one_chunk(name, fmt, group):
    """Experts above 2048 routed rows: the wgrad contraction runs in row chunks
    whose partial sums per block are added in chunk order afterwards. Both
    hot experts' dScale (and dZP) and dX against the oracle, per expert."""
    rng = np.random.default_rng(900 + fmt + group)
    E, N, K = 4, 256, 256
    sizes = [2600, 0, 4500, 37]                       # 2 and 3 chunks, empty, ragged
    seg = _segments(rng, E, sizes)
    R = int(seg[-1])
    w = _rand_w(rng, E, N, K)
    s, zp, g = O.observer_weight(w, fmt, group)
    s = (s * rng.uniform(0.7, 1.1, s.shape)).astype(np.float32)
    x = O.f32_to_bf16(rng.standard_normal((R, K)).astype(np.float32))
    dy = O.f32_to_bf16(rng.standard_normal((R, N)).astype(np.float32))
    dx_ref, ds_ref, dzp_ref = O.grouped_gemm_bwd(dy, x, seg, w, fmt, group, s, zp, g)
    wq = _wq(fmt, group, s, zp, g)
    G = K // group
    dx = torch.empty((R, K), dtype=torch.bfloat16, device="cuda")
    ds = torch.full((E, N, G), 7.0, device="cuda")
    dzp = torch.full((E, N, G), 7.0, device="cuda") if fmt == O.FMT_INT4 else None
    ws = torch.empty(F.fq_workspace_bytes(F.FQ_OP_GEMM_BWD, (E, N, K), R, fmt), dtype=torch.uint8,
                     device="cuda")
    F.fq_grouped_gemm_bwd_scale(dev_bf16(dy), dev_bf16(x), R, dev_i32(seg), (E, N, K),
                                dev_bf16(w), None, wq, None, dx, ds, dzp, ws)
    torch.cuda.synchronize()
    check_gemm_tol(host_bits(dx), dx_ref, "dx")
    dsh = ds.cpu().numpy()
    check_dscale_per_expert(dsh, ds_ref, "dscale")
    assert np.all(dsh[1] == 0)
    if dzp is not None:
        check_dscale_per_expert(dzp.cpu().numpy(), dzp_ref, "dzero_point")


@pytest.mark.parametrize("name,fmt,grp", [("int8_pc", O.FMT_INT8, "K"), ("int4_g16", O.FMT_INT4, 16),
                                          ("fp8_pc", O.FMT_FP8, "K"), ("nvfp4", O.FMT_NVFP4, 16),
                                          ("int8_pt", O.FMT_INT8, "T")])
@pytest.mark.parametrize("afmt", [O.FMT_NONE, O.FMT_NVFP4])
@pytest.mark.parametrize("N,K", [(80, 48), (272, 208)])
def test_gemm_shapes_not_multiple_of_tiles(name, fmt, grp, afmt, N, K):
    """N and K multiples of 16 but not of the tile sizes: the calls pad the
    operands with zeros (neutral scales) in the workspace and copy back only
    their own region. Forward and backward against the oracle; rows past the
    routed rows stay untouched."""
    rng = np.random.default_rng(1000 + 7 * fmt + afmt + N + K)
    E = 3
    seg = _segments(rng, E, [70, 0, 33])
    R = int(seg[-1])
    R_max = R + 5
    group = K if grp == "K" else (O.GROUP_TENSOR if grp == "T" else grp)
    w = _rand_w(rng, E, N, K)
    s, zp, g = O.observer_weight(w, fmt, group)
    x = O.f32_to_bf16(rng.standard_normal((R_max, K)).astype(np.float32))
    dy = O.f32_to_bf16(rng.standard_normal((R_max, N)).astype(np.float32))
    sa = O.observer_act(x[:R], afmt) if afmt else np.float32(1.0)
    y_ref = O.grouped_gemm_fwd(x, seg, w, fmt, group, s, zp, g, afmt, sa)
    dx_ref, ds_ref, dzp_ref = O.grouped_gemm_bwd(dy, x, seg, w, fmt, group, s, zp, g, afmt, sa)
    gq = F.FQ_GROUP_TENSOR if group == O.GROUP_TENSOR else group
    wq = _wq(fmt, gq, s, zp, g)
    aq = F.ActQ(afmt, dev_f32([sa])) if afmt else None
    fmts = fmt | (afmt << 8)
    ws = torch.empty(max(F.fq_workspace_bytes(F.FQ_OP_GEMM_FWD, (E, N, K), R_max, fmts),
                         F.fq_workspace_bytes(F.FQ_OP_GEMM_BWD, (E, N, K), R_max, fmts)),
                     dtype=torch.uint8, device="cuda")
    y = torch.full((R_max, N), 7.0, dtype=torch.bfloat16, device="cuda")
    wd = dev_bf16(w)
    F.fq_grouped_gemm_fwd(dev_bf16(x), R_max, dev_i32(seg), (E, N, K), wd, None, wq, aq, y, ws)
    dx = torch.full((R_max, K), 7.0, dtype=torch.bfloat16, device="cuda")
    ds = torch.full(s.shape, 7.0, device="cuda")
    dzp = torch.full(s.shape, 7.0, device="cuda") if fmt == O.FMT_INT4 else None
    F.fq_grouped_gemm_bwd_scale(dev_bf16(dy), dev_bf16(x), R_max, dev_i32(seg), (E, N, K), wd,
                                None, wq, aq, dx, ds, dzp, ws)
    torch.cuda.synchronize()
    yb, dxb = host_bits(y), host_bits(dx)
    check_gemm_tol(yb[:R], y_ref, "y")
    assert np.all(bf16_vals(yb[R:]) == 7.0)
    check_gemm_tol(dxb[:R], dx_ref, "dx")
    assert np.all(bf16_vals(dxb[R:]) == 7.0)
    dsh = ds.cpu().numpy()
    check_dscale_tol(dsh, ds_ref, "dscale")
    if group != O.GROUP_TENSOR:
        check_dscale_per_expert(dsh, ds_ref, "dscale")
    assert np.all(dsh[1] == 0)                         # the empty expert
    if dzp is not None:
        check_dscale_per_expert(dzp.cpu().numpy(), dzp_ref, "dzero_point")


@pytest.mark.parametrize("name,fmt", [("int8", O.FMT_INT8), ("fp8", O.FMT_FP8)])
def test_per_tensor_weight_scales(name, fmt):
    """One scale per expert matrix: observer and FQ pass bit-exact, forward
    and backward (dX, dScale [E]) to the GEMM / dScale tolerances."""
    rng = np.random.default_rng(750 + fmt)
    E, N, K = 4, 256, 512
    seg = _segments(rng, E, [90, 0, 301, 33])
    R = int(seg[-1])
    R_max = R + 17
    GT = F.FQ_GROUP_TENSOR
    w = _rand_w(rng, E, N, K)
    s_ref, _, _ = O.observer_weight(w, fmt, O.GROUP_TENSOR)
    s_dev = torch.full((E,), -1.0, device="cuda")
    wd = dev_bf16(w)
    F.observer_absmax_init(wd, (E, N, K), fmt, GT, 0, s_dev)
    torch.cuda.synchronize()
    assert np.array_equal(s_dev.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    s = (s_ref * rng.uniform(0.3, 0.9, E)).astype(np.float32)     # saturate the outliers
    wq = F.WeightQ(fmt=fmt, group=GT, scale=dev_f32(s))
    ref = O.fq_weight_stack(w, fmt, O.GROUP_TENSOR, s)
    assert not ref.mask.all()
    wfq = torch.empty_like(wd)
    codes = torch.zeros(E * N * K, dtype=torch.uint8, device="cuda")
    F.fq_quantize_stacked(wd, (E, N, K), wq, wfq, codes)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(wfq), ref.bits)
    assert np.array_equal(codes.cpu().numpy(), O.pack_codes(ref.code, fmt))
    afmt = O.FMT_FP8
    x = O.f32_to_bf16(rng.standard_normal((R_max, K)).astype(np.float32))
    dy = O.f32_to_bf16(rng.standard_normal((R_max, N)).astype(np.float32))
    sa = np.float32(O.observer_act(x[:R], afmt) * 0.8)
    aq = F.ActQ(afmt, dev_f32([sa]))
    ws = torch.empty(max(F.fq_workspace_bytes(F.FQ_OP_GEMM_FWD, (E, N, K), R_max, fmt | afmt << 8),
                         F.fq_workspace_bytes(F.FQ_OP_GEMM_BWD, (E, N, K), R_max, fmt | afmt << 8)),
                     dtype=torch.uint8, device="cuda")
    y = torch.empty(R_max, N, dtype=torch.bfloat16, device="cuda")
    F.fq_grouped_gemm_fwd(dev_bf16(x), R_max, dev_i32(seg), (E, N, K), wd, None, wq, aq, y, ws)
    dx = torch.empty(R_max, K, dtype=torch.bfloat16, device="cuda")
    ds = torch.full((E,), 7.0, device="cuda")
    F.fq_grouped_gemm_bwd_scale(dev_bf16(dy), dev_bf16(x), R_max, dev_i32(seg), (E, N, K), wd,
                                None, wq, aq, dx, ds, None, ws)
    torch.cuda.synchronize()
    check_gemm_tol(host_bits(y)[:R], O.grouped_gemm_fwd(x, seg, w, fmt, O.GROUP_TENSOR, s,
                                                        afmt=afmt, act_scale=sa), "y")
    dx_ref, ds_ref, _ = O.grouped_gemm_bwd(dy, x, seg, w, fmt, O.GROUP_TENSOR, s, afmt=afmt,
                                           act_scale=sa)
    check_gemm_tol(host_bits(dx)[:R], dx_ref, "dx")
    dsh = ds.cpu().numpy()
    assert dsh.shape == (E,) and dsh[1] == 0.0
    check_dscale_tol(dsh, ds_ref, "dscale per tensor")


def test_bwd_deterministic_run_to_run():
    rng = np.random.default_rng(800)
    E, N, K = 3, 256, 256
    seg = _segments(rng, E, [500, 20, 270])
    R = int(seg[-1])
    w = _rand_w(rng, E, N, K)
    s, _, _ = O.observer_weight(w, O.FMT_FP8, K)
    x = dev_bf16(O.f32_to_bf16(rng.standard_normal((R, K)).astype(np.float32)))
    dy = dev_bf16(O.f32_to_bf16(rng.standard_normal((R, N)).astype(np.float32)))
    wq = _wq(O.FMT_FP8, K, s, None, None)
    ws = torch.empty(F.fq_workspace_bytes(F.FQ_OP_GEMM_BWD, (E, N, K), R, O.FMT_FP8),
                     dtype=torch.uint8, device="cuda")
    outs = []
    for _ in range(2):
        dx = torch.empty(R, K, dtype=torch.bfloat16, device="cuda")
        ds = torch.empty(E, N, 1, device="cuda")
        F.fq_grouped_gemm_bwd_scale(dy, x, R, dev_i32(seg), (E, N, K), dev_bf16(w), None, wq, None,
                                    dx, ds, None, ws)
        outs.append((dx.clone(), ds.clone()))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0].view(torch.int16), outs[1][0].view(torch.int16))
    assert torch.equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("N,K", [(256, 256), (512, 512)])
def test_gemm_ragged_tiles_every_launch(N, K):
    """FWD and DGRAD on experts whose last 256-row tile leaves waves without
    rows in every pattern (1..64, 65..128, 129..191, 192..255 valid rows of
    the tile). A wave with no rows skips its LDS reads and reaches its next
    loads early; the loads of a stage may not land in a buffer that another
    wave still reads. Every launch is checked: bitwise equal to the first,
    the first against the oracle."""
    rng = np.random.default_rng(850 + N)
    sizes = [189, 0, 129, 191, 65, 257, 320, 1, 450, 146, 64, 192, 255, 128]
    E = len(sizes)
    seg = _segments(rng, E, sizes)
    R = int(seg[-1])
    w = _rand_w(rng, E, N, K)
    s, _, g = O.observer_weight(w, O.FMT_NVFP4, 16)
    wq = _wq(O.FMT_NVFP4, 16, s, None, g)
    wd = dev_bf16(w)
    wfq = torch.empty_like(wd)
    F.fq_quantize_stacked(wd, (E, N, K), wq, wfq)
    wsb = F.fq_workspace_bytes(F.FQ_OP_GEMM_BWD, (E, N, K), R, 0)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
    x = O.f32_to_bf16(rng.standard_normal((R, K)).astype(np.float32))
    dy = O.f32_to_bf16(rng.standard_normal((R, N)).astype(np.float32))
    xd, dyd, segd = dev_bf16(x), dev_bf16(dy), dev_i32(seg)
    y_ref = O.grouped_gemm_fwd(x, seg, w, O.FMT_NVFP4, 16, s, None, g)
    dx_ref, _, _ = O.grouped_gemm_bwd(dy, x, seg, w, O.FMT_NVFP4, 16, s, None, g)
    ys, dxs = [], []
    for _ in range(12):
        y = torch.full((R, N), 7.0, dtype=torch.bfloat16, device="cuda")
        dx = torch.full((R, K), 7.0, dtype=torch.bfloat16, device="cuda")
        F.fq_grouped_gemm_fwd(xd, R, segd, (E, N, K), None, wfq, wq, None, y, None)
        F.fq_grouped_gemm_bwd_scale(dyd, xd, R, segd, (E, N, K), wd, wfq, wq, None, dx, None,
                                    None, ws)
        ys.append(y)
        dxs.append(dx)
    torch.cuda.synchronize()
    check_gemm_tol(host_bits(ys[0]), y_ref, "y")
    check_gemm_tol(host_bits(dxs[0]), dx_ref, "dx")
    for i in range(1, len(ys)):
        assert torch.equal(ys[i].view(torch.int16), ys[0].view(torch.int16)), f"y launch {i}"
        assert torch.equal(dxs[i].view(torch.int16), dxs[0].view(torch.int16)), f"dx launch {i}"



@pytest.mark.parametrize("E,sizes,N,K", [
    (1, [300], 1024, 4096),          # FWD 8 tiles in 8 parts, DGRAD 32 tiles in 2 parts
    (3, [200, 0, 45], 1024, 1520),   # ragged experts, one empty; K zero-padded to 1536:
                                     # FWD 12 tiles in 3 parts, DGRAD 18 tiles in 2 parts
    (1, [64], 256, 8192),            # FWD one tile in 8 parts; DGRAD (4 stages) unsplit
    (2, [150, 90], 512, 1088),       # FWD 17 stages as parts of 9 and 8 (odd, uneven);
                                     # DGRAD zero-padded to K = 1280, unsplit
])
def test_gemm_small_calls_split_along_the_contraction(E, sizes, N, K):
    """Calls whose 256 x 256 tiles would leave most CUs idle run each tile's
    contraction (when it is 16 stages of 64 or more) as several parts, the
    parts' fp32 sums added in part order by a second kernel. Forward and dX
    against the oracle, bitwise equal from launch to launch, rows past the
    experts untouched; the forward given no workspace (then unsplit) within
    the same tolerance."""
    rng = np.random.default_rng(1200 + N + K + E)
    seg = _segments(rng, E, sizes)
    R = int(seg[-1])
    R_max = R + 16
    fmt, g = O.FMT_INT8, K
    w = _rand_w(rng, E, N, K)
    s, zp, gs = O.observer_weight(w, fmt, g)
    wq = _wq(fmt, g, s, zp, gs)
    x = O.f32_to_bf16(rng.standard_normal((R_max, K)).astype(np.float32))
    dy = O.f32_to_bf16(rng.standard_normal((R_max, N)).astype(np.float32))
    wd, xd, dyd, segd = dev_bf16(w), dev_bf16(x), dev_bf16(dy), dev_i32(seg)
    wfq = torch.empty_like(wd)
    F.fq_quantize_stacked(wd, (E, N, K), wq, wfq)
    nbf = F.fq_workspace_bytes(F.FQ_OP_GEMM_FWD, (E, N, K), R_max, 0)
    assert nbf > 0                 # the parts' sums (and the padded copies)
    ws_f = torch.empty(nbf, dtype=torch.uint8, device="cuda")
    ws_b = torch.empty(F.fq_workspace_bytes(F.FQ_OP_GEMM_BWD, (E, N, K), R_max, 0),
                       dtype=torch.uint8, device="cuda")
    ys, dxs = [], []
    for _ in range(3):
        y = torch.full((R_max, N), 7.0, dtype=torch.bfloat16, device="cuda")
        dx = torch.full((R_max, K), 7.0, dtype=torch.bfloat16, device="cuda")
        F.fq_grouped_gemm_fwd(xd, R_max, segd, (E, N, K), None, wfq, wq, None, y, ws_f)
        F.fq_grouped_gemm_bwd_scale(dyd, xd, R_max, segd, (E, N, K), wd, wfq, wq, None, dx, None,
                                    None, ws_b)
        ys.append(y)
        dxs.append(dx)
    y_one = torch.full((R_max, N), 7.0, dtype=torch.bfloat16, device="cuda")
    if K % 64 == 0 and N % 256 == 0:
        F.fq_grouped_gemm_fwd(xd, R_max, segd, (E, N, K), None, wfq, wq, None, y_one, None)
    else:
        F.fq_grouped_gemm_fwd(xd, R_max, segd, (E, N, K), None, wfq, wq, None, y_one, ws_f)
    torch.cuda.synchronize()
    y_ref = O.grouped_gemm_fwd(x, seg, w, fmt, g, s, zp, gs)
    dx_ref, _, _ = O.grouped_gemm_bwd(dy, x, seg, w, fmt, g, s, zp, gs)
    check_gemm_tol(host_bits(ys[0])[:R], y_ref, "y")
    check_gemm_tol(host_bits(dxs[0])[:R], dx_ref, "dx")
    check_gemm_tol(host_bits(y_one)[:R], y_ref, "y unsplit")
    for i in range(1, len(ys)):
        assert torch.equal(ys[i].view(torch.int16), ys[0].view(torch.int16)), f"y launch {i}"
        assert torch.equal(dxs[i].view(torch.int16), dxs[0].view(torch.int16)), f"dx launch {i}"
    assert np.all(bf16_vals(host_bits(ys[0])[R:]) == 7.0)
    assert np.all(bf16_vals(host_bits(dxs[0])[R:]) == 7.0)


@pytest.mark.parametrize("seed", range(8))
def test_gemm_split_random_shapes(seed):
    """Seeded random small calls with long contractions (mostly split along
    it: 1-5 experts, ragged and empty segments, N and K multiples of 16 that
    the calls zero-pad, 16-96 stages): forward and dX against the oracle,
    and the forward given no workspace (unsplit where the shape is
    tile-aligned) within the same tolerance."""
    rng = np.random.default_rng(1300 + seed)
    E = int(rng.integers(1, 6))
    sizes = [int(v) for v in rng.integers(0, 400, E)]
    sizes[int(rng.integers(0, E))] = int(rng.integers(1, 300))      # at least one non-empty expert
    if E > 2:
        sizes[int(rng.integers(0, E))] = 0                            # an empty one
    N = int(rng.choice([256, 512, 272, 768, 1040]))
    K = int(rng.choice([1024, 1536, 2048, 3072, 6144, 1488, 2064]))
    seg = _segments(rng, E, sizes)
    R = int(seg[-1])
    R_max = R + int(rng.integers(0, 40))
    fmt, g = O.FMT_INT8, K
    w = _rand_w(rng, E, N, K)
    s_, zp, gs = O.observer_weight(w, fmt, g)
    wq = _wq(fmt, g, s_, zp, gs)
    x = O.f32_to_bf16(rng.standard_normal((R_max, K)).astype(np.float32))
    dy = O.f32_to_bf16(rng.standard_normal((R_max, N)).astype(np.float32))
    wd, xd, dyd, segd = dev_bf16(w), dev_bf16(x), dev_bf16(dy), dev_i32(seg)
    wfq = torch.empty_like(wd)
    F.fq_quantize_stacked(wd, (E, N, K), wq, wfq)
    ws_f = torch.empty(max(F.fq_workspace_bytes(F.FQ_OP_GEMM_FWD, (E, N, K), R_max, 0), 1),
                       dtype=torch.uint8, device="cuda")
    ws_b = torch.empty(F.fq_workspace_bytes(F.FQ_OP_GEMM_BWD, (E, N, K), R_max, 0),
                       dtype=torch.uint8, device="cuda")
    y = torch.full((R_max, N), 7.0, dtype=torch.bfloat16, device="cuda")
    dx = torch.full((R_max, K), 7.0, dtype=torch.bfloat16, device="cuda")
    F.fq_grouped_gemm_fwd(xd, R_max, segd, (E, N, K), None, wfq, wq, None, y, ws_f)
    F.fq_grouped_gemm_bwd_scale(dyd, xd, R_max, segd, (E, N, K), wd, wfq, wq, None, dx, None,
                                None, ws_b)
    y_one = torch.full((R_max, N), 7.0, dtype=torch.bfloat16, device="cuda")
    aligned = K % 64 == 0 and N % 256 == 0
    F.fq_grouped_gemm_fwd(xd, R_max, segd, (E, N, K), None, wfq, wq, None, y_one,
                          None if aligned else ws_f)
    torch.cuda.synchronize()
    y_ref = O.grouped_gemm_fwd(x, seg, w, fmt, g, s_, zp, gs)
    dx_ref, _, _ = O.grouped_gemm_bwd(dy, x, seg, w, fmt, g, s_, zp, gs)
    case = f"E={E} sizes={sizes} N={N} K={K} R_max={R_max}"
    check_gemm_tol(host_bits(y)[:R], y_ref, f"y ({case})")
    check_gemm_tol(host_bits(dx)[:R], dx_ref, f"dx ({case})")
    check_gemm_tol(host_bits(y_one)[:R], y_ref, f"y unsplit ({case})")
    assert np.all(bf16_vals(host_bits(y)[R:]) == 7.0), case
    assert np.all(bf16_vals(host_bits(dx)[R:]) == 7.0), case

# ------------------------------------------- the expert input as token rows --
def _routing(rng, T, topk, E, hot=None):
    """Routing over E local experts (expert 1 empty; `hot` takes most rows)."""
    ids = np.empty((T, topk), np.int32)
    for t in range(T):
        pool = [e for e in range(E) if e != 1]
        if hot is not None and rng.random() < 0.8:
            first = [hot]
            pool = [e for e in pool if e != hot]
            ids[t] = first + list(rng.choice(pool, topk - 1, replace=False))
        else:
            ids[t] = rng.choice(pool, topk, replace=False)
    perm, _, seg = O.moe_permute(ids, 0, E)
    return perm, seg


@pytest.mark.parametrize("afmt", [O.FMT_NONE, O.FMT_FP8, O.FMT_INT8, O.FMT_NVFP4])
def test_actfq_bitexact(afmt):
    rng = np.random.default_rng(900 + afmt)
    T, K = 300, 272
    x = _rand_w(rng, 1, T, K, std=1.0)[0]
    s = O.observer_act(x, afmt) if afmt else np.float32(1.0)
    xq = torch.full((T, K), 7.0, dtype=torch.bfloat16, device="cuda")
    F.fq_actfq(dev_bf16(x), T, K, F.ActQ(afmt, dev_f32([s])) if afmt else None, xq)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(xq), O.fq_act(x, afmt, s).bits)


@pytest.mark.parametrize("name,fmt,group", [("nvfp4", O.FMT_NVFP4, 16), ("int4", O.FMT_INT4, 128),
                                            ("fp8", O.FMT_FP8, None)])
@pytest.mark.parametrize("N,K", [(512, 384), (272, 208), (512, 2048)])
@pytest.mark.parametrize("prequantized", [True, False])
def test_gemm_fwd_tokens_is_the_gathered_fwd(name, fmt, group, N, K, prequantized):
    """Routed row r read as token row perm[r] / topk gives the bits of the
    plain call on the gathered rows, and matches the oracle. K = 2048 (32
    stages over at most 24 tiles) splits the contraction into 4 parts."""
    rng = np.random.default_rng(910 + fmt + N)
    T, topk, E = 400, 4, 6
    if group is not None and K % group:
        group = 16
    g = group or K
    perm, seg = _routing(rng, T, topk, E, hot=2)
    R = int(seg[-1])
    R_max = R + 24
    w = _rand_w(rng, E, N, K)
    s, zp, gs = O.observer_weight(w, fmt, g)
    wq = _wq(fmt, g, s, zp, gs)
    x_tok = O.f32_to_bf16(rng.standard_normal((T, K)).astype(np.float32))
    x_rows = np.zeros((R_max, K), np.uint16)
    x_rows[:R] = x_tok[perm // topk]
    wd = dev_bf16(w)
    wfq = None
    if prequantized:
        wfq = torch.empty_like(wd)
        F.fq_quantize_stacked(wd, (E, N, K), wq, wfq)
    fmts = 0 if prequantized else fmt
    ws = torch.empty(max(F.fq_workspace_bytes(F.FQ_OP_GEMM_FWD, (E, N, K), max(R_max, T), fmts), 1),
                     dtype=torch.uint8, device="cuda")
    y1 = torch.full((R_max, N), 7.0, dtype=torch.bfloat16, device="cuda")
    y2 = torch.full((R_max, N), 7.0, dtype=torch.bfloat16, device="cuda")
    segd, permd = dev_i32(seg), dev_i32(perm)
    F.fq_grouped_gemm_fwd(dev_bf16(x_rows), R_max, segd, (E, N, K), wd, wfq, wq, None, y1, ws)
    F.fq_grouped_gemm_fwd_tokens(dev_bf16(x_tok), T, permd, topk, R_max, segd, (E, N, K), wd, wfq,
                                 wq, y2, ws)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    check_gemm_tol(host_bits(y2)[:R], O.grouped_gemm_fwd(x_rows[:R], seg, w, fmt, g, s, zp, gs), "y")
    assert np.all(bf16_vals(host_bits(y2)[R:]) == 7.0)


@pytest.mark.parametrize("name,fmt,group", [("nvfp4", O.FMT_NVFP4, 16), ("int4", O.FMT_INT4, 128),
                                            ("fp8", O.FMT_FP8, None), ("int8_g32", O.FMT_INT8, 32)])
@pytest.mark.parametrize("N,K,T", [(256, 512, 400), (272, 208, 400), (256, 256, 2800)])
def test_gemm_wgrad_tokens_is_the_gathered_wgrad(name, fmt, group, N, K, T):
    """dScale (and dzero_point) of the routed-X wgrad equal the plain call's
    on the gathered rows bit for bit, and match the oracle. T = 2800 with a
    hot expert puts more than 2048 rows on it (the chunked partial sums)."""
    rng = np.random.default_rng(920 + fmt + N + T)
    topk, E = 2, 4
    if group is not None and K % group:
        group = 16
    g = group or K
    perm, seg = _routing(rng, T, topk, E, hot=3)
    R = int(seg[-1])
    R_max = R + 8
    if T == 2800:
        assert seg[4] - seg[3] > 2048
    w = _rand_w(rng, E, N, K)
    s, zp, gs = O.observer_weight(w, fmt, g)
    wq = _wq(fmt, g, s, zp, gs)
    x_tok = O.f32_to_bf16(rng.standard_normal((T, K)).astype(np.float32))
    x_rows = np.zeros((R_max, K), np.uint16)
    x_rows[:R] = x_tok[perm // topk]
    dy = O.f32_to_bf16(rng.standard_normal((R_max, N)).astype(np.float32))
    ws = torch.empty(F.fq_workspace_bytes(F.FQ_OP_GEMM_BWD, (E, N, K), max(R_max, T), fmt),
                     dtype=torch.uint8, device="cuda")
    wd, segd, dyd = dev_bf16(w), dev_i32(seg), dev_bf16(dy)
    shp = (E, N, K // g)
    ds1 = torch.full(shp, 7.0, device="cuda")
    ds2 = torch.full(shp, 7.0, device="cuda")
    dz1 = torch.full(shp, 7.0, device="cuda") if fmt == O.FMT_INT4 else None
    dz2 = torch.full(shp, 7.0, device="cuda") if fmt == O.FMT_INT4 else None
    F.fq_grouped_gemm_bwd_scale(dyd, dev_bf16(x_rows), R_max, segd, (E, N, K), wd, None, wq, None,
                                None, ds1, dz1, ws)
    F.fq_grouped_gemm_wgrad_tokens(dyd, dev_bf16(x_tok), T, dev_i32(perm), topk, R_max, segd,
                                   (E, N, K), wd, wq, ds2, dz2, ws)
    torch.cuda.synchronize()
    assert torch.equal(ds1, ds2)
    if dz1 is not None:
        assert torch.equal(dz1, dz2)
    _, ds_ref, dz_ref = O.grouped_gemm_bwd(dy, x_rows, seg, w, fmt, g, s, zp, gs)
    check_dscale_tol(ds2.cpu().numpy(), ds_ref, "ds")
    check_dscale_per_expert(ds2.cpu().numpy(), ds_ref, "ds")
    if dz1 is not None:
        check_dscale_tol(dz2.cpu().numpy(), dz_ref, "dzp")


@pytest.mark.parametrize("topk", [1, 8])
def test_gemm_tokens_calls_at_top1_and_top8(topk):
    """Both token-row calls with one routed slot per token (the row divisor
    is 1) and with eight (the bench routing): bitwise the gathered calls."""
    rng = np.random.default_rng(930 + topk)
    T, E, N, K, g = 350, 10, 256, 256, 16
    perm, seg = _routing(rng, T, topk, E)
    R = int(seg[-1])
    R_max = R + 5
    w = _rand_w(rng, E, N, K)
    s, zp, gs = O.observer_weight(w, O.FMT_NVFP4, g)
    wq = _wq(O.FMT_NVFP4, g, s, zp, gs)
    x_tok = O.f32_to_bf16(rng.standard_normal((T, K)).astype(np.float32))
    x_rows = np.zeros((R_max, K), np.uint16)
    x_rows[:R] = x_tok[perm // topk]
    dy = O.f32_to_bf16(rng.standard_normal((R_max, N)).astype(np.float32))
    nb = max(F.fq_workspace_bytes(F.FQ_OP_GEMM_FWD, (E, N, K), max(R_max, T), 0),
             F.fq_workspace_bytes(F.FQ_OP_GEMM_BWD, (E, N, K), max(R_max, T), O.FMT_NVFP4), 1)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    wd, segd, permd = dev_bf16(w), dev_i32(seg), dev_i32(perm)
    wfq = torch.empty_like(wd)
    F.fq_quantize_stacked(wd, (E, N, K), wq, wfq)
    y1 = torch.full((R_max, N), 7.0, dtype=torch.bfloat16, device="cuda")
    y2 = torch.full((R_max, N), 7.0, dtype=torch.bfloat16, device="cuda")
    F.fq_grouped_gemm_fwd(dev_bf16(x_rows), R_max, segd, (E, N, K), wd, wfq, wq, None, y1, ws)
    F.fq_grouped_gemm_fwd_tokens(dev_bf16(x_tok), T, permd, topk, R_max, segd, (E, N, K), wd, wfq,
                                 wq, y2, ws)
    shp = (E, N, K // g)
    ds1 = torch.full(shp, 7.0, device="cuda")
    ds2 = torch.full(shp, 7.0, device="cuda")
    F.fq_grouped_gemm_bwd_scale(dev_bf16(dy), dev_bf16(x_rows), R_max, segd, (E, N, K), wd, None, wq,
                                None, None, ds1, None, ws)
    F.fq_grouped_gemm_wgrad_tokens(dev_bf16(dy), dev_bf16(x_tok), T, permd, topk, R_max, segd,
                                   (E, N, K), wd, wq, ds2, None, ws)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert torch.equal(ds1, ds2)
    check_gemm_tol(host_bits(y2)[:R], O.grouped_gemm_fwd(x_rows[:R], seg, w, O.FMT_NVFP4, g, s, zp,
                                                         gs), "y")
    _, ds_ref, _ = O.grouped_gemm_bwd(dy, x_rows, seg, w, O.FMT_NVFP4, g, s, zp, gs)
    check_dscale_per_expert(ds2.cpu().numpy(), ds_ref, "ds")


# ------------------------------------------------------- error handling --
def test_errors_are_reported_before_launch():
    E, N, K = 2, 256, 250      # K not a multiple of 16
    w = torch.zeros(E, N, K, dtype=torch.bfloat16, device="cuda")
    q = F.WeightQ(F.FMT_NVFP4, 16, torch.ones(E, N, 16, device="cuda"),
                  None, torch.ones(E, device="cuda"))
    with pytest.raises(F.FQError) as ei:
        F.fq_quantize_stacked(w, (E, N, K), q, torch.empty_like(w))
    assert ei.value.status == F.FQ_ERR_INVALID_ARGUMENT
    with pytest.raises(F.FQError) as ei:
        F.fq_moe_permute(torch.zeros(4, 8, dtype=torch.int32, device="cuda"), 4, 8, 0, 16,
                         torch.empty(32, dtype=torch.int32, device="cuda"),
                         torch.empty(4, 8, dtype=torch.int32, device="cuda"),
                         torch.empty(17, dtype=torch.int32, device="cuda"),
                         torch.empty(4, dtype=torch.uint8, device="cuda"))
    assert ei.value.status == F.FQ_ERR_WORKSPACE_TOO_SMALL
