"""Python binding of libfq, the gfx950 C-ABI library for scale-only fake-quant
MoE grouped GEMM (argument marshalling only: every step runs in libfq's HIP
kernels; torch provides device memory and the current stream).

Each function has the name and argument order of its C entry point in
include/fq.h, takes device tensors (or None for a NULL pointer), enqueues on
``torch.cuda.current_stream()`` and raises ``FQError`` for a non-OK status.
Importing this package loads ``libfq.so`` from this directory and fails
loudly when it is missing; there is no fallback.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfq.so")

FQ_OK = 0
FQ_ERR_INVALID_ARGUMENT = 1
FQ_ERR_UNSUPPORTED = 2
FQ_ERR_WORKSPACE_TOO_SMALL = 3
FQ_ERR_HIP = 4

FMT_NONE = 0
FMT_INT8 = 1
FMT_INT4 = 2
FMT_FP8_E4M3 = 3
FMT_NVFP4 = 4
FMT_BY_NAME = {"none": FMT_NONE, "int8": FMT_INT8, "int4": FMT_INT4, "fp8": FMT_FP8_E4M3,
               "nvfp4": FMT_NVFP4}

FQ_OP_PERMUTE = 1
FQ_OP_GEMM_FWD = 2
FQ_OP_GEMM_BWD = 3
FQ_OP_ACT_SCALE_GRAD = 4
FQ_OP_TOPK_KL = 5
FQ_GROUP_TENSOR = -1     # one weight scale per expert matrix (int8 / fp8)

EXPORTED = (
    "observer_absmax_init", "fq_quantize_stacked", "fq_moe_permute", "fq_grouped_gemm_fwd",
    "fq_grouped_gemm_bwd_scale", "fq_moe_gather_actfq", "fq_swiglu_actfq", "fq_swiglu_bwd",
    "fq_moe_combine", "fq_moe_combine_bwd", "fq_moe_unpermute_reduce", "fq_workspace_bytes",
    "fq_last_error", "fq_abi_version", "fq_export_scales", "fq_dequantize_stacked", "fq_topk_kl",
    "fq_moe_permute_noalloc", "fq_validate", "fq_actfq", "fq_grouped_gemm_fwd_tokens",
    "fq_grouped_gemm_wgrad_tokens",
)

FQ_BAD_EXPERT_ID = 0x01
FQ_BAD_SEG_START = 0x02
FQ_BAD_SEG_ORDER = 0x04
FQ_BAD_SEG_END = 0x08
FQ_BAD_SCALE = 0x10
FQ_BAD_ZERO_POINT = 0x20
FQ_BAD_GLOBAL_SCALE = 0x40
FQ_BAD_ACT_SCALE = 0x80


class FQError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"libfq status {status}: {msg}")
        self.status = status


class fq_shape(ctypes.Structure):
    _fields_ = [("E", ctypes.c_int32), ("N", ctypes.c_int32), ("K", ctypes.c_int32)]


class fq_weight_q(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("group", ctypes.c_int32), ("scale", ctypes.c_void_p),
                ("zero_point", ctypes.c_void_p), ("global_scale", ctypes.c_void_p)]


class fq_act_q(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("scale", ctypes.c_void_p)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libfq.so not found at {LIB_PATH}; build it with "
                          "`python moe_fake_quant_amd/build.py` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    st = ctypes.c_int
    sig = {
        "observer_absmax_init": (st, [P, fq_shape, I32, I32, I32, P, P, P, P, SZ, P]),
        "fq_quantize_stacked": (st, [P, fq_shape, ctypes.POINTER(fq_weight_q), P, P, P]),
        "fq_moe_permute": (st, [P, I32, I32, I32, I32, P, P, P, P, SZ, P]),
        "fq_moe_permute_noalloc": (st, [P, I32, I32, I32, I32, P, P, P, P]),
        "fq_validate": (st, [P, I32, I32, I32, P, I32, I32, fq_shape, ctypes.POINTER(fq_weight_q),
                             ctypes.POINTER(fq_act_q), P, P]),
        "fq_grouped_gemm_fwd": (st, [P, I32, P, fq_shape, P, P, ctypes.POINTER(fq_weight_q),
                                     ctypes.POINTER(fq_act_q), P, P, SZ, P]),
        "fq_grouped_gemm_bwd_scale": (st, [P, P, I32, P, fq_shape, P, P,
                                           ctypes.POINTER(fq_weight_q), ctypes.POINTER(fq_act_q),
                                           P, P, P, P, SZ, P]),
        "fq_actfq": (st, [P, I32, I32, ctypes.POINTER(fq_act_q), P, P]),
        "fq_grouped_gemm_fwd_tokens": (st, [P, I32, P, I32, I32, P, fq_shape, P, P,
                                            ctypes.POINTER(fq_weight_q), P, P, SZ, P]),
        "fq_grouped_gemm_wgrad_tokens": (st, [P, P, I32, P, I32, I32, P, fq_shape, P,
                                              ctypes.POINTER(fq_weight_q), P, P, P, SZ, P]),
        "fq_moe_gather_actfq": (st, [P, I32, I32, P, I32, ctypes.POINTER(fq_act_q), P, P]),
        "fq_swiglu_actfq": (st, [P, I32, P, I32, ctypes.POINTER(fq_act_q), P, P, P]),
        "fq_swiglu_bwd": (st, [P, P, I32, P, I32, ctypes.POINTER(fq_act_q), P, P, P, SZ, P]),
        "fq_moe_combine": (st, [P, P, P, I32, I32, I32, P, P]),
        "fq_moe_combine_bwd": (st, [P, P, P, I32, I32, I32, P, P]),
        "fq_moe_unpermute_reduce": (st, [P, P, P, I32, I32, I32, ctypes.POINTER(fq_act_q), P, P,
                                         P, SZ, P]),
        "fq_export_scales": (st, [fq_shape, ctypes.POINTER(fq_weight_q), P, P, P]),
        "fq_dequantize_stacked": (st, [P, fq_shape, I32, I32, P, P, P, P, P, P]),
        "fq_topk_kl": (st, [P, P, I32, I32, I32, I32, P, P, P, P, P, P, SZ, P]),
        "fq_workspace_bytes": (SZ, [I32, fq_shape, I32, I32]),
        "fq_last_error": (ctypes.c_char_p, []),
        "fq_abi_version": (I32, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def lib() -> ctypes.CDLL:
    return _lib


def abi_version() -> int:
    return _lib.fq_abi_version()


def _check(status: int):
    if status != FQ_OK:
        raise FQError(status, _lib.fq_last_error().decode())


def _p(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libfq takes device tensors")
    if not t.is_contiguous():
        raise ValueError("libfq takes contiguous tensors")
    return t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


@dataclasses.dataclass
class WeightQ:
    """Weight quantizer: fmt, group, scale [E,N,K/group] (nvfp4: theta),
    zero_point (int4), global_scale [E] (nvfp4)."""
    fmt: int
    group: int
    scale: Optional[torch.Tensor] = None
    zero_point: Optional[torch.Tensor] = None
    global_scale: Optional[torch.Tensor] = None

    def c(self) -> fq_weight_q:
        return fq_weight_q(self.fmt, self.group, _p(self.scale), _p(self.zero_point),
                           _p(self.global_scale))


@dataclasses.dataclass
class ActQ:
    """Activation quantizer: fmt and a one-element device scale (s_a or g_a)."""
    fmt: int = FMT_NONE
    scale: Optional[torch.Tensor] = None

    def c(self) -> fq_act_q:
        return fq_act_q(self.fmt, _p(self.scale))


def _shape(E, N, K) -> fq_shape:
    return fq_shape(int(E), int(N), int(K))


def _aq(aq: Optional[ActQ]):
    return ctypes.byref(aq.c()) if aq is not None else None


def _nbytes(ws: Optional[torch.Tensor]) -> int:
    return 0 if ws is None else ws.numel() * ws.element_size()


def fq_workspace_bytes(op: int, shape, R_max: int, fmts: int) -> int:
    return int(_lib.fq_workspace_bytes(op, _shape(*shape), int(R_max), int(fmts)))


def observer_absmax_init(x, shape, fmt, group, per_tensor, scale, zero_point=None,
                         global_scale=None, ws=None):
    _check(_lib.observer_absmax_init(_p(x), _shape(*shape), fmt, group, int(per_tensor), _p(scale),
                                     _p(zero_point), _p(global_scale), _p(ws), _nbytes(ws),
                                     _stream()))


def fq_quantize_stacked(w, shape, q: WeightQ, w_fq=None, codes=None):
    _check(_lib.fq_quantize_stacked(_p(w), _shape(*shape), ctypes.byref(q.c()), _p(w_fq),
                                    _p(codes), _stream()))


def fq_moe_permute(expert_ids, T, topk, expert_begin, E_local, perm, row_of, seg_offsets, ws):
    _check(_lib.fq_moe_permute(_p(expert_ids), int(T), int(topk), int(expert_begin),
                               int(E_local), _p(perm), _p(row_of), _p(seg_offsets), _p(ws),
                               _nbytes(ws), _stream()))


def fq_moe_permute_noalloc(expert_ids, T, topk, expert_begin, E_local, perm, row_of,
                           seg_offsets):
    _check(_lib.fq_moe_permute_noalloc(_p(expert_ids), int(T), int(topk), int(expert_begin),
                                       int(E_local), _p(perm), _p(row_of), _p(seg_offsets),
                                       _stream()))


def fq_validate(status, expert_ids=None, T=0, topk=0, n_experts=0, seg_offsets=None, E=0,
                R_max=0, shape=(1, 1, 1), wq: Optional[WeightQ] = None, aq: Optional[ActQ] = None):
    """Enqueue the device-data checks; `status` (one int32/uint32 device
    element) receives the OR of the FQ_BAD_* bits of failed conditions."""
    _check(_lib.fq_validate(_p(expert_ids), int(T), int(topk), int(n_experts), _p(seg_offsets),
                            int(E), int(R_max), _shape(*shape),
                            ctypes.byref(wq.c()) if wq is not None else None,
                            ctypes.byref(aq.c()) if aq is not None else None, _p(status),
                            _stream()))


def fq_grouped_gemm_fwd(x, R_max, seg_offsets, shape, w, w_fq, wq: Optional[WeightQ],
                        aq: Optional[ActQ], y, ws=None):
    _check(_lib.fq_grouped_gemm_fwd(_p(x), int(R_max), _p(seg_offsets), _shape(*shape), _p(w),
                                    _p(w_fq), ctypes.byref(wq.c()) if wq is not None else None,
                                    _aq(aq), _p(y), _p(ws),
                                    _nbytes(ws), _stream()))


def fq_grouped_gemm_bwd_scale(dy, x, R_max, seg_offsets, shape, w, w_fq, wq: WeightQ,
                              aq: Optional[ActQ], dx, dscale, dzero_point=None, ws=None):
    _check(_lib.fq_grouped_gemm_bwd_scale(_p(dy), _p(x), int(R_max), _p(seg_offsets),
                                          _shape(*shape), _p(w), _p(w_fq), ctypes.byref(wq.c()),
                                          _aq(aq), _p(dx), _p(dscale), _p(dzero_point), _p(ws),
                                          _nbytes(ws), _stream()))


def fq_actfq(x, rows, K, aq: Optional[ActQ], xq):
    _check(_lib.fq_actfq(_p(x), int(rows), int(K), _aq(aq), _p(xq), _stream()))


def fq_grouped_gemm_fwd_tokens(x_tok, T, perm, topk, R_max, seg_offsets, shape, w, w_fq,
                               wq: Optional[WeightQ], y, ws=None):
    _check(_lib.fq_grouped_gemm_fwd_tokens(_p(x_tok), int(T), _p(perm), int(topk), int(R_max),
                                           _p(seg_offsets), _shape(*shape), _p(w), _p(w_fq),
                                           ctypes.byref(wq.c()) if wq is not None else None,
                                           _p(y), _p(ws), _nbytes(ws), _stream()))


def fq_grouped_gemm_wgrad_tokens(dy, x_tok, T, perm, topk, R_max, seg_offsets, shape, w,
                                 wq: WeightQ, dscale, dzero_point=None, ws=None):
    _check(_lib.fq_grouped_gemm_wgrad_tokens(_p(dy), _p(x_tok), int(T), _p(perm), int(topk),
                                             int(R_max), _p(seg_offsets), _shape(*shape), _p(w),
                                             ctypes.byref(wq.c()), _p(dscale), _p(dzero_point),
                                             _p(ws), _nbytes(ws), _stream()))


def fq_moe_gather_actfq(x, T, H, row_of, topk, aq: Optional[ActQ], xq):
    _check(_lib.fq_moe_gather_actfq(_p(x), int(T), int(H), _p(row_of), int(topk), _aq(aq),
                                    _p(xq), _stream()))


def fq_swiglu_actfq(h, R_max, n_rows, F, aq: Optional[ActQ], a, aq_out):
    _check(_lib.fq_swiglu_actfq(_p(h), int(R_max), _p(n_rows), int(F), _aq(aq), _p(a),
                                _p(aq_out), _stream()))


def fq_swiglu_bwd(daq, h, R_max, n_rows, F, aq: Optional[ActQ], dh, dscale_a=None, ws=None):
    _check(_lib.fq_swiglu_bwd(_p(daq), _p(h), int(R_max), _p(n_rows), int(F), _aq(aq), _p(dh),
                              _p(dscale_a), _p(ws), _nbytes(ws), _stream()))


def fq_moe_combine(o, probs, row_of, T, topk, H, out):
    _check(_lib.fq_moe_combine(_p(o), _p(probs), _p(row_of), int(T), int(topk), int(H), _p(out),
                               _stream()))


def fq_moe_combine_bwd(dout, probs, row_of, T, topk, H, dO):
    _check(_lib.fq_moe_combine_bwd(_p(dout), _p(probs), _p(row_of), int(T), int(topk), int(H),
                                   _p(dO), _stream()))


def fq_moe_unpermute_reduce(dxq, row_of, x, T, topk, H, aq: Optional[ActQ], dx, dscale_a=None,
                            ws=None):
    _check(_lib.fq_moe_unpermute_reduce(_p(dxq), _p(row_of), _p(x), int(T), int(topk), int(H),
                                        _aq(aq), _p(dx), _p(dscale_a), _p(ws), _nbytes(ws),
                                        _stream()))


def fq_export_scales(shape, q: WeightQ, scale_bytes=None, zero_point_bytes=None):
    _check(_lib.fq_export_scales(_shape(*shape), ctypes.byref(q.c()), _p(scale_bytes),
                                 _p(zero_point_bytes), _stream()))


def fq_dequantize_stacked(codes, shape, fmt, group, w_bf16, scale=None, scale_bytes=None,
                          zero_point_bytes=None, global_scale=None):
    _check(_lib.fq_dequantize_stacked(_p(codes), _shape(*shape), int(fmt), int(group), _p(scale),
                                      _p(scale_bytes), _p(zero_point_bytes), _p(global_scale),
                                      _p(w_bf16), _stream()))


def fq_topk_kl(student, teacher, T, V, K, reverse, valid, topk_idx, grad, loss_tok, loss_mean, ws):
    _check(_lib.fq_topk_kl(_p(student), _p(teacher), int(T), int(V), int(K), int(bool(reverse)),
                           _p(valid), _p(topk_idx), _p(grad), _p(loss_tok), _p(loss_mean), _p(ws),
                           _nbytes(ws), _stream()))


from .layer import MoEFakeQuantLayer  # noqa: E402,F401
