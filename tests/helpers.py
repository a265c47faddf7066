"""Shared helpers of the test suite (bf16 bits <-> torch device tensors,
tolerance checks)."""
import numpy as np
import torch

GEMM_TOL = 2e-2      # max|gpu - ref| <= 2e-2 * max|ref|  (GEMM outputs, dX)
DSCALE_TOL = 1e-3    # max|gpu - ref| / max|ref| <= 1e-3  (dScale, normwise)
# A learnable activation scale's gradient is one fp32 sum of n products,
# accumulated per thread and then in fixed-order trees: its rounding error is
# below (16 + log2 n) * 2^-24 * sum|terms| < 1e-5 * sum|terms| for any n < 2^100.
ACT_DSCALE_TOL = 1e-5


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.cuda()


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_vals(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def dev_f32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, np.float32))).cuda()


def dev_i32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, np.int32))).cuda()


def check_gemm_tol(gpu_bits, ref_bits, what=""):
    g, r = bf16_vals(gpu_bits), bf16_vals(ref_bits)
    err = np.abs(g - r).max() if g.size else 0.0
    scale = np.abs(r).max() if r.size else 0.0
    assert err <= GEMM_TOL * scale, f"{what}: max|err| {err:.4g} > {GEMM_TOL} * {scale:.4g}"
    return err / max(scale, 1e-30)


def check_dscale_tol(gpu, ref, what=""):
    g = np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    scale = np.abs(r).max()
    err = np.abs(g - r).max()
    assert err <= DSCALE_TOL * scale, f"{what}: max|err| {err:.4g} > {DSCALE_TOL} * {scale:.4g}"
    return err / max(scale, 1e-30)


def check_act_dscale_tol(gpu, ref, abs_terms, what="", tol=ACT_DSCALE_TOL):
    """|gpu - ref| <= tol * sum|g * dv/ds| (abs_terms), the sum's own scale."""
    err = abs(float(gpu) - float(ref))
    assert err <= tol * abs_terms, f"{what}: |err| {err:.4g} > {tol} * {abs_terms:.4g}"
    return err / max(abs_terms, 1e-30)


def dscale_p99(gpu, ref):
    """99th percentile of the element-wise error |gpu - ref| / max|ref| (the
    normwise check bounds its maximum; R-15 reports the percentile too)."""
    g = np.asarray(gpu, np.float64).reshape(-1)
    r = np.asarray(ref, np.float64).reshape(-1)
    scale = np.abs(r).max() if r.size else 0.0
    if scale == 0.0:
        return 0.0
    return float(np.percentile(np.abs(g - r), 99) / scale)


def check_dscale_per_expert(gpu, ref, what=""):
    """Normwise dScale tolerance for each expert's slice [e, ...] on its own
    scale, so that an error in a cold expert cannot hide under the hottest
    expert's magnitude; an expert whose reference is all zero must be exactly
    zero. Prints the worst ratio and the tensor's p99 element-wise error."""
    g = np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    worst = 0.0
    for e in range(r.shape[0]):
        se = np.abs(r[e]).max()
        ee = np.abs(g[e] - r[e]).max()
        if se == 0.0:
            assert ee == 0.0, f"{what}: expert {e} reference is zero, gpu max|.| {ee:.4g}"
            continue
        assert ee <= DSCALE_TOL * se, \
            f"{what}: expert {e} max|err| {ee:.4g} > {DSCALE_TOL} * {se:.4g}"
        worst = max(worst, ee / se)
    p99 = dscale_p99(g, r)
    print(f"[dscale] {what}: worst per-expert max|err|/max|ref| {worst:.3g}, "
          f"p99 element-wise |err|/max|ref| {p99:.3g}", flush=True)
    return worst, p99
