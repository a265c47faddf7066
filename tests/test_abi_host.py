"""Host-side tests of the C ABI (no GPU needed).

- libfq.so loads and exports, under its plain C name, every function that
  include/fq.h declares, and the Python binding exposes the same names;
- the pure host queries (version, workspace sizes) answer as documented;
- argument checks reject bad calls with the documented status before any
  launch. These use placeholder pointers and therefore run only where no GPU
  is visible; the GPU suite repeats the error cases with real tensors.
"""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fq.h")
LIB_PATH = os.path.join(ROOT, "moe_fake_quant_amd", "libfq.so")


def _declared():
    """Names of the functions fq.h declares (prototypes start at column 0)."""
    names = []
    with open(HEADER) as f:
        for line in f:
            m = re.match(r"^(?!typedef|#|\s)[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", line)
            if m:
                names.append(m.group(1))
    return names


@pytest.fixture(scope="module")
def pkg():
    if not os.path.exists(LIB_PATH):
        # by path: importing the package needs the library being built
        import importlib.util
        spec = importlib.util.spec_from_file_location("_fq_build", os.path.join(
            os.path.dirname(LIB_PATH), "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
    import moe_fake_quant_amd as F
    return F


def _no_gpu_visible():
    try:
        import torch
        return torch.cuda.device_count() == 0
    except Exception:
        return True


host_only = pytest.mark.skipif(not _no_gpu_visible(),
                               reason="placeholder pointers: host-check cases run where no GPU is "
                                      "visible; the GPU suite covers them with device tensors")


def test_header_declares_the_boundary():
    names = _declared()
    for required in ("fq_quantize_stacked", "fq_grouped_gemm_fwd", "fq_grouped_gemm_bwd_scale",
                     "observer_absmax_init", "fq_moe_permute", "fq_workspace_bytes",
                     "fq_last_error", "fq_abi_version"):
        assert required in names
    assert len(names) == len(set(names))


def test_library_exports_every_declared_symbol(pkg):
    lib = ctypes.CDLL(LIB_PATH)
    for name in _declared():
        assert hasattr(lib, name), f"libfq.so does not export {name}"
    # exported as unmangled dynamic symbols
    out = subprocess.run(["nm", "-D", "--defined-only", LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    dyn = {ln.split()[-1] for ln in out.splitlines() if ln.strip()}
    missing = [n for n in _declared() if n not in dyn]
    assert not missing, missing


def test_binding_matches_header(pkg):
    assert set(pkg.EXPORTED) == set(_declared())
    for name in pkg.EXPORTED:
        if name in ("fq_last_error", "fq_abi_version"):
            continue
        assert callable(getattr(pkg, name)), name


def test_version_and_error_string(pkg):
    lib = pkg.lib()
    assert lib.fq_abi_version() == 2
    assert isinstance(lib.fq_last_error(), bytes)


def _ws(pkg, op, shape, R, wfmt=0, afmt=0):
    return pkg.lib().fq_workspace_bytes(op, pkg.fq_shape(*shape), R, wfmt | (afmt << 8))


def _up(x):
    return (x + 255) // 256 * 256


def test_workspace_sizes(pkg):
    # enough rows for the 256 x 256 tiles to fill a 256-CU (or 304-CU) part:
    # no call splits its contraction, the sizes are the plain buffers
    E, N, K, R = 8, 512, 256, 40000
    # forward: prequantized weights and no activation FQ need nothing
    assert _ws(pkg, pkg.FQ_OP_GEMM_FWD, (E, N, K), R) == 0
    # weight FQ inside the call: one bf16 W_fq stack; act FQ: one bf16 [R, K]
    assert _ws(pkg, pkg.FQ_OP_GEMM_FWD, (E, N, K), R, pkg.FMT_NVFP4) == _up(E * N * K * 2)
    assert _ws(pkg, pkg.FQ_OP_GEMM_FWD, (E, N, K), R, pkg.FMT_NVFP4, pkg.FMT_FP8_E4M3) == \
        _up(E * N * K * 2) + _up(R * K * 2)
    # backward: dScale partials (scale and zero point) per wgrad row chunk of
    # at most 2048 rows (every expert has at least one) and 16-block of K,
    # plus the chunk prefix, plus (per-tensor scales) the scale repeated per
    # channel and the per-channel dScale
    def bwd_plain(R):
        chunks = (R + 2047) // 2048 + E
        part = _up(chunks * N * (K // 16) * 4)
        return 2 * part + _up((E + 1) * 4) + 2 * _up(E * N * 4)
    assert _ws(pkg, pkg.FQ_OP_GEMM_BWD, (E, N, K), R) == bwd_plain(R)
    # a small call with a long contraction (1000 rows: at most 44 forward and
    # 88 dX tiles; 32 and 16 stages of 64) also holds the fp32 sums of the
    # parts its tiles' contraction is split into: 2 to 8 parts of [rows, N]
    # (forward) or [rows, K] (dX)
    E, N, K, r = 8, 1024, 2048, 1000
    fwd = _ws(pkg, pkg.FQ_OP_GEMM_FWD, (E, N, K), r)
    assert fwd % _up(r * N * 4) == 0 and 2 <= fwd // _up(r * N * 4) <= 8
    bwd = _ws(pkg, pkg.FQ_OP_GEMM_BWD, (E, N, K), r) - bwd_plain(r)
    assert bwd % _up(r * K * 4) == 0 and 2 <= bwd // _up(r * K * 4) <= 8
    # a short contraction (256: 4 stages) is not split
    assert _ws(pkg, pkg.FQ_OP_GEMM_FWD, (E, N, 256), r) == 0
    # permute: grows with the pair count, positive for any expert count
    a = _ws(pkg, pkg.FQ_OP_PERMUTE, (4, 0, 0), 1000)
    b = _ws(pkg, pkg.FQ_OP_PERMUTE, (4, 0, 0), 100000)
    assert 0 < a <= b
    assert _ws(pkg, 99, (E, N, K), R) == 0


# ----------------------------------------------------------------- checks --
FAKE = 0x100000  # 16-byte aligned placeholder, never dereferenced: every case fails a check


def _status(pkg, fn, *args):
    return getattr(pkg.lib(), fn)(*args)


def _wq(pkg, fmt, group, scale=FAKE, zp=None, g=None):
    return ctypes.byref(pkg.fq_weight_q(fmt, group, scale, zp, g))


@host_only
def test_quantize_stacked_rejects_bad_arguments(pkg):
    S = pkg.fq_shape
    bad = [
        (S(0, 16, 16), _wq(pkg, pkg.FMT_INT8, 16), pkg.FQ_ERR_INVALID_ARGUMENT),   # empty shape
        (S(1, 16, 32), _wq(pkg, pkg.FMT_NVFP4, 32, g=FAKE), pkg.FQ_ERR_INVALID_ARGUMENT),  # nvfp4 group
        (S(1, 16, 32), _wq(pkg, pkg.FMT_NVFP4, 16), pkg.FQ_ERR_INVALID_ARGUMENT),  # no global scale
        (S(1, 16, 256), _wq(pkg, pkg.FMT_INT4, 128), pkg.FQ_ERR_INVALID_ARGUMENT),  # no zero point
        (S(1, 16, 48), _wq(pkg, pkg.FMT_INT8, 32), pkg.FQ_ERR_INVALID_ARGUMENT),   # group !| K
        (S(1, 16, 32), _wq(pkg, 7, 32), pkg.FQ_ERR_INVALID_ARGUMENT),             # unknown format
    ]
    for shape, q, want in bad:
        assert _status(pkg, "fq_quantize_stacked", FAKE, shape, q, FAKE, None, None) == want
        assert pkg.lib().fq_last_error()
    # neither output requested
    assert _status(pkg, "fq_quantize_stacked", FAKE, S(1, 16, 32), _wq(pkg, pkg.FMT_INT8, 32),
                   None, None, None) == pkg.FQ_ERR_INVALID_ARGUMENT
    # misaligned input
    assert _status(pkg, "fq_quantize_stacked", FAKE + 2, S(1, 16, 32), _wq(pkg, pkg.FMT_INT8, 32),
                   FAKE, None, None) == pkg.FQ_ERR_INVALID_ARGUMENT


@host_only
def test_grouped_gemm_rejects_unsupported_shapes(pkg):
    S = pkg.fq_shape
    q = _wq(pkg, pkg.FMT_FP8_E4M3, 256)
    # N and K must be multiples of 16 (the block of the grids)
    st = _status(pkg, "fq_grouped_gemm_fwd", FAKE, 64, FAKE, S(2, 120, 256), None, FAKE, q, None,
                 FAKE, None, 0, None)
    assert st == pkg.FQ_ERR_UNSUPPORTED
    assert b"16" in pkg.lib().fq_last_error()
    # other multiples of 16 run zero-padded to the tile shape, in workspace
    # memory: with none given the call says how much it needs
    st = _status(pkg, "fq_grouped_gemm_fwd", FAKE, 64, FAKE, S(2, 128, 256), None, FAKE, q, None,
                 FAKE, None, 0, None)
    assert st == pkg.FQ_ERR_WORKSPACE_TOO_SMALL
    need = pkg.lib().fq_workspace_bytes(pkg.FQ_OP_GEMM_FWD, S(2, 128, 256), 64, 0)
    assert need >= 2 * 256 * 256 * 2 + 64 * 256 * 2 * 2          # padded W_fq, x and y
    assert pkg.lib().fq_workspace_bytes(pkg.FQ_OP_GEMM_FWD, S(2, 256, 256), 64, 0) == 0
    # more experts than the tile scheduler holds
    st = _status(pkg, "fq_grouped_gemm_fwd", FAKE, 64, FAKE, S(1025, 256, 256), None, FAKE, q,
                 None, FAKE, None, 0, None)
    assert st == pkg.FQ_ERR_UNSUPPORTED
    # backward: K a multiple of 16; dScale group must be reducible by the epilogue
    st = _status(pkg, "fq_grouped_gemm_bwd_scale", FAKE, FAKE, 64, FAKE, S(2, 256, 200), FAKE,
                 FAKE, _wq(pkg, pkg.FMT_FP8_E4M3, 200), None, FAKE, None, None, FAKE, 1 << 30, None)
    assert st in (pkg.FQ_ERR_UNSUPPORTED, pkg.FQ_ERR_INVALID_ARGUMENT)   # refused before launch
    assert pkg.lib().fq_workspace_bytes(pkg.FQ_OP_GEMM_BWD, S(2, 80, 48), 64, 0) > \
        pkg.lib().fq_workspace_bytes(pkg.FQ_OP_GEMM_BWD, S(2, 256, 256), 64, 0)
    st = _status(pkg, "fq_grouped_gemm_bwd_scale", FAKE, FAKE, 64, FAKE, S(2, 256, 768), FAKE,
                 FAKE, _wq(pkg, pkg.FMT_INT8, 48), None, None, FAKE, None, FAKE, 1 << 30, None)
    assert st == pkg.FQ_ERR_UNSUPPORTED
    # dzero_point exists only for int4, and needs dscale
    st = _status(pkg, "fq_grouped_gemm_bwd_scale", FAKE, FAKE, 64, FAKE, S(2, 256, 256), FAKE,
                 FAKE, _wq(pkg, pkg.FMT_INT8, 256), None, None, None, FAKE, FAKE, 1 << 30, None)
    assert st == pkg.FQ_ERR_INVALID_ARGUMENT
    # workspace too small for weight FQ inside the call
    st = _status(pkg, "fq_grouped_gemm_fwd", FAKE, 64, FAKE, S(2, 256, 256), FAKE, None, q, None,
                 FAKE, FAKE, 16, None)
    assert st == pkg.FQ_ERR_WORKSPACE_TOO_SMALL
    # activation FQ format without a scale
    aq = ctypes.byref(pkg.fq_act_q(pkg.FMT_NVFP4, None))
    st = _status(pkg, "fq_grouped_gemm_fwd", FAKE, 64, FAKE, S(2, 256, 256), None, FAKE, q, aq,
                 FAKE, FAKE, 1 << 30, None)
    assert st == pkg.FQ_ERR_INVALID_ARGUMENT


@host_only
def test_permute_and_elementwise_reject_bad_arguments(pkg):
    L = pkg.lib()
    assert L.fq_moe_permute(FAKE, 16, 0, 0, 4, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == \
        pkg.FQ_ERR_INVALID_ARGUMENT                                   # topk 0
    assert L.fq_moe_permute(FAKE, 16, 8, 0, 4, FAKE, FAKE, None, FAKE, 1 << 20, None) == \
        pkg.FQ_ERR_INVALID_ARGUMENT                                   # no seg_offsets
    assert L.fq_moe_permute(FAKE, 16, 8, 0, 4, FAKE, FAKE, FAKE, FAKE, 8, None) == \
        pkg.FQ_ERR_WORKSPACE_TOO_SMALL
    # the allocation-free variant: same checks, and a request beyond its
    # static scratch fails before anything touches a device
    assert L.fq_moe_permute_noalloc(FAKE, 16, 0, 0, 4, FAKE, FAKE, FAKE, None) == \
        pkg.FQ_ERR_INVALID_ARGUMENT                                   # topk 0
    assert L.fq_moe_permute_noalloc(FAKE, 16, 8, 0, 4, FAKE, FAKE, None, None) == \
        pkg.FQ_ERR_INVALID_ARGUMENT                                   # no seg_offsets
    assert L.fq_moe_permute_noalloc(FAKE, 262144, 8, 0, 1024, FAKE, FAKE, FAKE, None) == \
        pkg.FQ_ERR_WORKSPACE_TOO_SMALL                                # 33.6 MB > 4 MiB
    assert b"static scratch" in L.fq_last_error()
    S = pkg.fq_shape
    assert L.fq_validate(None, 0, 0, 0, None, 0, 0, S(1, 1, 1), None, None, None, None) == \
        pkg.FQ_ERR_INVALID_ARGUMENT                                   # no status word
    assert L.fq_validate(FAKE, 16, 0, 8, None, 0, 0, S(1, 1, 1), None, None, FAKE, None) == \
        pkg.FQ_ERR_INVALID_ARGUMENT                                   # routing with topk 0
    assert L.fq_validate(None, 0, 0, 0, FAKE, 0, 10, S(1, 1, 1), None, None, FAKE, None) == \
        pkg.FQ_ERR_INVALID_ARGUMENT                                   # segments of 0 experts
    assert L.fq_moe_gather_actfq(FAKE, 16, 40, FAKE, 8, None, FAKE, None) == \
        pkg.FQ_ERR_INVALID_ARGUMENT                                   # H % 16
    assert L.fq_moe_gather_actfq(FAKE, 16, 64, None, 8, None, FAKE, None) == \
        pkg.FQ_ERR_INVALID_ARGUMENT                                   # no row map
    assert L.fq_swiglu_actfq(FAKE, 128, None, 64, None, None, FAKE, None) == \
        pkg.FQ_ERR_INVALID_ARGUMENT                                   # no n_rows
    assert L.fq_swiglu_bwd(FAKE, FAKE, 128, FAKE, 24, None, FAKE, None, None, 0, None) == \
        pkg.FQ_ERR_INVALID_ARGUMENT                                   # F % 16
    assert L.fq_moe_combine(FAKE, FAKE, FAKE, 16, 8, 64, FAKE + 8, None) == \
        pkg.FQ_ERR_INVALID_ARGUMENT                                   # misaligned out
    assert L.fq_moe_combine_bwd(FAKE, FAKE, FAKE, 16, 0, 64, FAKE, None) == \
        pkg.FQ_ERR_INVALID_ARGUMENT                                   # topk 0
    # 2^35 elements and more are refused before launch (32-bit vector counts
    # of 8 elements inside the kernels)
    big_t, h = (1 << 35) // 2048, 2048
    assert L.fq_moe_gather_actfq(FAKE, big_t, h, FAKE, 8, None, FAKE, None) == \
        pkg.FQ_ERR_INVALID_ARGUMENT
    assert b"too many elements" in L.fq_last_error()
    assert L.fq_swiglu_actfq(FAKE, big_t, FAKE, h, None, None, FAKE, None) == \
        pkg.FQ_ERR_INVALID_ARGUMENT
    assert b"too many elements" in L.fq_last_error()
    assert L.fq_moe_combine_bwd(FAKE, FAKE, FAKE, big_t, 8, h, FAKE, None) == \
        pkg.FQ_ERR_INVALID_ARGUMENT
    assert b"too many elements" in L.fq_last_error()
    aq = ctypes.byref(pkg.fq_act_q(pkg.FMT_FP8_E4M3, FAKE))
    assert L.fq_moe_unpermute_reduce(FAKE, FAKE, None, 16, 8, 64, aq, FAKE, None, None, 0,
                                     None) == pkg.FQ_ERR_INVALID_ARGUMENT  # act mask needs x
    assert L.observer_absmax_init(FAKE, pkg.fq_shape(1, 4, 12), pkg.FMT_INT8, 12, 0, FAKE, None,
                                  None, None, 0, None) == pkg.FQ_ERR_INVALID_ARGUMENT  # K % 8


@host_only
def test_per_tensor_weight_scale_arguments(pkg):
    """FQ_GROUP_TENSOR: int8 / fp8 only, scale required."""
    L = pkg.lib()
    shape = pkg.fq_shape(2, 256, 256)
    for fmt, scale, want in ((pkg.FMT_INT4, FAKE, pkg.FQ_ERR_INVALID_ARGUMENT),
                             (pkg.FMT_NVFP4, FAKE, pkg.FQ_ERR_INVALID_ARGUMENT),
                             (pkg.FMT_FP8_E4M3, None, pkg.FQ_ERR_INVALID_ARGUMENT)):
        q = pkg.fq_weight_q(fmt, pkg.FQ_GROUP_TENSOR, scale, FAKE, FAKE)
        assert L.fq_quantize_stacked(FAKE, shape, ctypes.byref(q), FAKE, None, None) == want
    assert L.observer_absmax_init(FAKE, shape, pkg.FMT_INT4, pkg.FQ_GROUP_TENSOR, 0, FAKE, FAKE,
                                  None, None, 0, None) == pkg.FQ_ERR_INVALID_ARGUMENT


@host_only
def test_export_arguments(pkg):
    """fq_export_scales only converts nvfp4 / int4 parameters; the decode checks
    its format, group and the pointers that format needs."""
    L = pkg.lib()
    shape = pkg.fq_shape(2, 64, 256)
    q8 = pkg.fq_weight_q(pkg.FMT_INT8, 256, FAKE, None, None)
    assert L.fq_export_scales(shape, ctypes.byref(q8), FAKE, FAKE, None) == \
        pkg.FQ_ERR_INVALID_ARGUMENT
    qn = pkg.fq_weight_q(pkg.FMT_NVFP4, 16, FAKE, None, FAKE)
    assert L.fq_export_scales(shape, ctypes.byref(qn), None, None, None) == \
        pkg.FQ_ERR_INVALID_ARGUMENT                                   # no scale_bytes
    dq = L.fq_dequantize_stacked
    assert dq(FAKE, shape, pkg.FMT_NVFP4, 32, None, FAKE, None, FAKE, FAKE, None) == \
        pkg.FQ_ERR_INVALID_ARGUMENT                                   # nvfp4 group
    assert dq(FAKE, shape, pkg.FMT_INT4, 128, FAKE, None, None, None, FAKE, None) == \
        pkg.FQ_ERR_INVALID_ARGUMENT                                   # no zero-point bytes
    assert dq(FAKE, shape, pkg.FMT_INT4, pkg.FQ_GROUP_TENSOR, FAKE, None, FAKE, None, FAKE,
              None) == pkg.FQ_ERR_INVALID_ARGUMENT                    # per tensor: int8 / fp8
    assert dq(FAKE + 4, shape, pkg.FMT_FP8_E4M3, 256, FAKE, None, None, None, FAKE, None) == \
        pkg.FQ_ERR_INVALID_ARGUMENT                                   # codes alignment
    assert dq(FAKE, pkg.fq_shape(2, 64, 40), pkg.FMT_FP8_E4M3, 40, FAKE, None, None, None, FAKE,
              None) == pkg.FQ_ERR_INVALID_ARGUMENT                    # K % 16


@host_only
def test_topk_kl_and_teacher_arguments(pkg):
    L = pkg.lib()
    kl = L.fq_topk_kl
    ok = (FAKE, FAKE, 16, 4096, 100, 0, None, FAKE, FAKE, FAKE, FAKE, FAKE, 256, None)
    for i, bad, want in ((3, 4100, pkg.FQ_ERR_INVALID_ARGUMENT),      # V % 8
                         (4, 0, pkg.FQ_ERR_INVALID_ARGUMENT),         # K = 0
                         (4, 5000, pkg.FQ_ERR_INVALID_ARGUMENT),      # K > V
                         (12, 16, pkg.FQ_ERR_WORKSPACE_TOO_SMALL),
                         (10, None, pkg.FQ_ERR_INVALID_ARGUMENT)):    # no loss_mean
        args = list(ok)
        args[i] = bad
        assert kl(*args) == want, i
    args = list(ok)
    args[3], args[4] = 16384, 4097
    assert kl(*args) == pkg.FQ_ERR_UNSUPPORTED                        # K above 4096
    # a forward GEMM without a quantizer needs the weights to use as given
    st = _status(pkg, "fq_grouped_gemm_fwd", FAKE, 64, FAKE, pkg.fq_shape(2, 256, 256), FAKE,
                 None, None, None, FAKE, None, 0, None)
    assert st == pkg.FQ_ERR_INVALID_ARGUMENT


@host_only
def test_learnable_act_scale_arguments(pkg):
    """A learnable activation scale needs a static per-tensor format and a
    workspace of one float per block (sized by FQ_OP_ACT_SCALE_GRAD)."""
    L = pkg.lib()
    T, H, R, F = 300, 256, 1200, 768
    need_x = _ws(pkg, pkg.FQ_OP_ACT_SCALE_GRAD, (1, T, H), 0)
    need_a = _ws(pkg, pkg.FQ_OP_ACT_SCALE_GRAD, (1, R, F), 0)
    # one fp32 partial per 256-thread block of 16-element chunks
    assert need_x == _up(4 * -(-T * H // 16 // 256))
    assert need_a == _up(4 * -(-R * F // 16 // 256))
    fp8 = ctypes.byref(pkg.fq_act_q(pkg.FMT_FP8_E4M3, FAKE))
    nv = ctypes.byref(pkg.fq_act_q(pkg.FMT_NVFP4, FAKE))
    for aq, ws, nb, want in ((nv, FAKE, need_x, pkg.FQ_ERR_UNSUPPORTED),
                             (None, FAKE, need_x, pkg.FQ_ERR_UNSUPPORTED),
                             (fp8, FAKE, need_x - 256, pkg.FQ_ERR_WORKSPACE_TOO_SMALL),
                             (fp8, None, need_x, pkg.FQ_ERR_WORKSPACE_TOO_SMALL)):
        assert L.fq_moe_unpermute_reduce(FAKE, FAKE, FAKE, T, 8, H, aq, FAKE, FAKE, ws, nb,
                                         None) == want
    for aq, ws, nb, want in ((nv, FAKE, need_a, pkg.FQ_ERR_UNSUPPORTED),
                             (fp8, FAKE, need_a - 256, pkg.FQ_ERR_WORKSPACE_TOO_SMALL)):
        assert L.fq_swiglu_bwd(FAKE, FAKE, R, FAKE, F, aq, FAKE, FAKE, ws, nb, None) == want
