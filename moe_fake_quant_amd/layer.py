"""One MoE layer's routed-expert path through libfq (orchestration only).

The AngelSlim mcore_qad article (section 二.4) replaces a layer's experts with
3D stacks, fake-quantizes each stack in one pass and runs all experts as one
grouped GEMM; weights are frozen and only quantizer scales train (section 一).
This class holds the device buffers of that path and calls the C ABI in
order; it computes nothing itself.

Forward:  FQ pass on both stacks -> permute -> act FQ of each token row ->
          gate_up GEMM (routed row r read as token row perm[r] / topk, so the
          gathered [R, H] input is never formed) -> SwiGLU + act FQ -> down
          GEMM -> combine
Backward: combine bwd -> down dgrad + dScale -> SwiGLU bwd (with the act-FQ
          mask; + dS_a2) -> gate_up dgrad + dScale -> unpermute-reduce (with
          the input act-FQ mask; + dS_a1)
Activation scales are frozen after calibration unless ``learn_act_scales``
(FP8 / INT8 activations), in which case the backward also returns their
gradients in ``ds_a1`` (input of gate_up) and ``ds_a2`` (input of down).
All buffers are allocated once; a step allocates nothing.

With ``overlap_wgrad`` (the default) the two wgrad -> dScale calls run on a
second stream of the same priority, each behind the producer of its inputs,
while the dgrad chain continues on the caller's stream: their persistent
grids then take over the CUs that a dgrad kernel's last partial round of
tiles leaves idle. The second stream has a workspace of its own.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import (ActQ, FMT_FP8_E4M3, FMT_INT4, FMT_INT8, FMT_NONE, FMT_NVFP4, FQ_GROUP_TENSOR,
               FQ_OP_ACT_SCALE_GRAD, FQ_OP_GEMM_BWD, FQ_OP_GEMM_FWD, FQ_OP_PERMUTE, WeightQ,
               fq_actfq, fq_grouped_gemm_bwd_scale, fq_grouped_gemm_fwd,
               fq_grouped_gemm_fwd_tokens, fq_grouped_gemm_wgrad_tokens, fq_moe_combine,
               fq_moe_combine_bwd, fq_moe_permute, fq_moe_unpermute_reduce, fq_quantize_stacked,
               fq_swiglu_actfq, fq_swiglu_bwd, fq_workspace_bytes, observer_absmax_init)


def _weight_q(E, N, K, fmt, group, dev) -> WeightQ:
    shape = (E,) if group == FQ_GROUP_TENSOR else (E, N, K // group)
    q = WeightQ(fmt=fmt, group=group, scale=torch.empty(shape, dtype=torch.float32, device=dev))
    if fmt == FMT_INT4:
        q.zero_point = torch.empty(shape, dtype=torch.float32, device=dev)
    if fmt == FMT_NVFP4:
        q.global_scale = torch.empty(E, dtype=torch.float32, device=dev)
    return q


class MoEFakeQuantLayer:
    def __init__(self, w_gu: torch.Tensor, w_d: torch.Tensor, wfmt: int, afmt: int, T_max: int,
                 topk: int, expert_begin: int = 0, group: Optional[int] = None,
                 learn_act_scales: bool = False):
        """w_gu [E, 2F, H], w_d [E, H, F] bf16 on the device (frozen). group None =
        one scale per output channel (group = K of each stack); FQ_GROUP_TENSOR =
        one scale per expert matrix (int8 / fp8). learn_act_scales:
        the backward also produces the activation-scale gradients (FP8 / INT8)."""
        assert w_gu.dtype == torch.bfloat16 and w_d.dtype == torch.bfloat16
        self.dev = w_gu.device
        self.E, F2, self.H = w_gu.shape
        self.F = F2 // 2
        assert tuple(w_d.shape) == (self.E, self.H, self.F)
        self.wfmt, self.afmt = wfmt, afmt
        self.topk, self.expert_begin = topk, expert_begin
        self.T_max = T_max
        self.R_max = T_max * topk
        self.w_gu, self.w_d = w_gu.contiguous(), w_d.contiguous()
        self.shape_gu = (self.E, 2 * self.F, self.H)
        self.shape_d = (self.E, self.H, self.F)
        g_gu = group or self.H
        g_d = group or self.F
        self.q_gu = _weight_q(*self.shape_gu, wfmt, g_gu, self.dev)
        self.q_d = _weight_q(*self.shape_d, wfmt, g_d, self.dev)
        f32 = dict(dtype=torch.float32, device=self.dev)
        bf = dict(dtype=torch.bfloat16, device=self.dev)
        i32 = dict(dtype=torch.int32, device=self.dev)
        self.aq1 = ActQ(afmt, torch.ones(1, **f32))
        self.aq2 = ActQ(afmt, torch.ones(1, **f32))
        self.wfq_gu = torch.empty(self.shape_gu, **bf)
        self.wfq_d = torch.empty(self.shape_d, **bf)
        R, H, F = self.R_max, self.H, self.F
        self.perm = torch.empty(R, **i32)
        self.row_of = torch.empty(T_max, topk, **i32)
        self.seg = torch.empty(self.E + 1, **i32)
        self.n_rows = self.seg[self.E:]
        # the expert input as token rows: FQ_a(x) once per token; the gate_up
        # GEMMs read routed row r as token row perm[r] / topk
        self.xq_tok = torch.empty(T_max, H, **bf)
        self._x_tok = None
        self.h = torch.empty(R, 2 * F, **bf)
        self.a = torch.empty(R, F, **bf)
        self.aq = torch.empty(R, F, **bf)
        self.o = torch.empty(R, H, **bf)
        self.out = torch.empty(T_max, H, **bf)
        self.do = torch.empty(R, H, **bf)
        self.daq = torch.empty(R, F, **bf)
        self.dh = torch.empty(R, 2 * F, **bf)
        self.dxq = torch.empty(R, H, **bf)
        self.dx = torch.empty(T_max, H, **bf)
        self.ds_gu = torch.empty_like(self.q_gu.scale)
        self.ds_d = torch.empty_like(self.q_d.scale)
        self.dzp_gu = torch.empty_like(self.q_gu.scale) if wfmt == FMT_INT4 else None
        self.dzp_d = torch.empty_like(self.q_d.scale) if wfmt == FMT_INT4 else None
        if learn_act_scales and afmt not in (FMT_FP8_E4M3, FMT_INT8):
            raise ValueError("learnable activation scales need fp8 or int8 activations")
        self.learn_act_scales = learn_act_scales
        self.ds_a1 = torch.zeros(1, **f32) if learn_act_scales else None
        self.ds_a2 = torch.zeros(1, **f32) if learn_act_scales else None
        ws = max(fq_workspace_bytes(FQ_OP_PERMUTE, (self.E, 0, 0), self.R_max, 0),
                 fq_workspace_bytes(FQ_OP_ACT_SCALE_GRAD, (1, T_max, H), 0, 0),
                 fq_workspace_bytes(FQ_OP_ACT_SCALE_GRAD, (1, R, F), 0, 0),
                 fq_workspace_bytes(FQ_OP_GEMM_FWD, self.shape_gu, R, 0),
                 fq_workspace_bytes(FQ_OP_GEMM_FWD, self.shape_d, R, 0),
                 fq_workspace_bytes(FQ_OP_GEMM_BWD, self.shape_gu, R, 0),
                 fq_workspace_bytes(FQ_OP_GEMM_BWD, self.shape_d, R, 0), 256)
        self.ws = torch.empty(ws, dtype=torch.uint8, device=self.dev)
        self.ws2 = torch.empty(ws, dtype=torch.uint8, device=self.dev)
        self.side = torch.cuda.Stream(device=self.dev)   # default priority
        self.ev_do = torch.cuda.Event()
        self.ev_dh = torch.cuda.Event()
        self.overlap_wgrad = True
        self.T = 0

    # ------------------------------------------------------------- setup --
    def init_weight_scales(self):
        """Observer init of both stacks' learnable scales."""
        for w, shape, q in ((self.w_gu, self.shape_gu, self.q_gu), (self.w_d, self.shape_d, self.q_d)):
            observer_absmax_init(w, shape, q.fmt, q.group, 0, q.scale, q.zero_point, q.global_scale)

    def quantize_weights(self):
        """One fake-quant pass over each whole stack."""
        fq_quantize_stacked(self.w_gu, self.shape_gu, self.q_gu, self.wfq_gu)
        fq_quantize_stacked(self.w_d, self.shape_d, self.q_d, self.wfq_d)

    def route(self, expert_ids: torch.Tensor):
        T = expert_ids.shape[0]
        assert T <= self.T_max and expert_ids.shape[1] == self.topk
        self.T = T
        fq_moe_permute(expert_ids, T, self.topk, self.expert_begin, self.E, self.perm,
                       self.row_of[:T], self.seg, self.ws)

    def calibrate(self, x: torch.Tensor, expert_ids: torch.Tensor):
        """Frozen activation scales from one calibration forward (reads R on the host)."""
        if self.afmt == FMT_NONE:
            return
        T = x.shape[0]
        observer_absmax_init(x, (1, T, self.H), self.afmt, 16, 1, self.aq1.scale)
        self.quantize_weights()
        self.route(expert_ids)
        R = int(self.seg[self.E].item())
        self._gate_up_fwd(x, T)
        fq_swiglu_actfq(self.h, self.R_max, self.n_rows, self.F, None, self.a, self.aq)
        if R > 0:
            observer_absmax_init(self.a[:R], (1, R, self.F), self.afmt, 16, 1, self.aq2.scale)

    # ---------------------------------------------------------- hot path --
    def _gate_up_fwd(self, x: torch.Tensor, T: int):
        """FQ_a of each token row once (the rows themselves without an
        activation format), then the gate_up GEMM over the routed rows."""
        if self.afmt == FMT_NONE:
            self._x_tok = x
        else:
            fq_actfq(x, T, self.H, self.aq1, self.xq_tok)
            self._x_tok = self.xq_tok
        fq_grouped_gemm_fwd_tokens(self._x_tok, T, self.perm, self.topk, self.R_max, self.seg,
                                   self.shape_gu, None, self.wfq_gu, self.q_gu, self.h, self.ws)

    def forward(self, x: torch.Tensor, expert_ids: torch.Tensor, probs: torch.Tensor,
                keep_a: bool = False) -> torch.Tensor:
        T = x.shape[0]
        self.route(expert_ids)
        self._gate_up_fwd(x, T)
        fq_swiglu_actfq(self.h, self.R_max, self.n_rows, self.F, self.aq2,
                        self.a if keep_a else None, self.aq)
        fq_grouped_gemm_fwd(self.aq, self.R_max, self.seg, self.shape_d, None, self.wfq_d,
                            self.q_d, None, self.o, self.ws)
        fq_moe_combine(self.o, probs, self.row_of[:T], T, self.topk, self.H, self.out[:T])
        return self.out[:T]

    def teacher_forward(self, x: torch.Tensor, expert_ids: torch.Tensor,
                        probs: torch.Tensor) -> torch.Tensor:
        """The self-teacher: this layer with quantization off (the raw token
        rows through the routing, the frozen bf16 weights as the GEMM operands,
        SwiGLU, combine), into buffers of its own so a student forward's saved
        activations survive."""
        T = x.shape[0]
        if not hasattr(self, "t_h"):
            bf = dict(dtype=torch.bfloat16, device=self.dev)
            R, H, F = self.R_max, self.H, self.F
            self.t_h = torch.empty(R, 2 * F, **bf)
            self.t_a = torch.empty(R, F, **bf)
            self.t_o = torch.empty(R, H, **bf)
            self.t_out = torch.empty(self.T_max, H, **bf)
        self.route(expert_ids)
        fq_grouped_gemm_fwd_tokens(x, T, self.perm, self.topk, self.R_max, self.seg,
                                   self.shape_gu, None, self.w_gu, None, self.t_h, self.ws)
        fq_swiglu_actfq(self.t_h, self.R_max, self.n_rows, self.F, None, None, self.t_a)
        fq_grouped_gemm_fwd(self.t_a, self.R_max, self.seg, self.shape_d, None, self.w_d, None,
                            None, self.t_o, None)
        fq_moe_combine(self.t_o, probs, self.row_of[:T], T, self.topk, self.H, self.t_out[:T])
        return self.t_out[:T]

    def _wgrad(self, ready, launch):
        """One wgrad -> dScale call, launch(ws): on the side stream once event
        `ready` (recorded right after its dy's producer) has passed
        (overlap_wgrad), else inline on the caller's stream."""
        if not self.overlap_wgrad:
            launch(self.ws)
            return
        self.side.wait_event(ready)
        with torch.cuda.stream(self.side):
            launch(self.ws2)

    def backward(self, x: torch.Tensor, probs: torch.Tensor, dout: torch.Tensor):
        T = x.shape[0]
        main = torch.cuda.current_stream(self.dev)
        if self.overlap_wgrad:
            # the side stream's previous step (and anything else the caller
            # enqueued before this backward) is complete before it reuses ws2
            self.side.wait_stream(main)
        fq_moe_combine_bwd(dout, probs, self.row_of[:T], T, self.topk, self.H, self.do)
        self.ev_do.record(main)
        # dgrad and wgrad -> dScale as separate calls (one GEMM kernel each);
        # the dgrad is enqueued first: it leads the chain to dX
        fq_grouped_gemm_bwd_scale(self.do, None, self.R_max, self.seg, self.shape_d, self.w_d,
                                  self.wfq_d, self.q_d, None, self.daq, None, None, self.ws)
        self._wgrad(self.ev_do, lambda ws: fq_grouped_gemm_bwd_scale(
            self.do, self.aq, self.R_max, self.seg, self.shape_d, self.w_d, self.wfq_d, self.q_d,
            None, None, self.ds_d, self.dzp_d, ws))
        fq_swiglu_bwd(self.daq, self.h, self.R_max, self.n_rows, self.F, self.aq2, self.dh,
                      self.ds_a2, self.ws)
        self.ev_dh.record(main)
        fq_grouped_gemm_bwd_scale(self.dh, None, self.R_max, self.seg, self.shape_gu, self.w_gu,
                                  self.wfq_gu, self.q_gu, None, self.dxq, None, None, self.ws)
        x_tok = self._x_tok
        self._wgrad(self.ev_dh, lambda ws: fq_grouped_gemm_wgrad_tokens(
            self.dh, x_tok, T, self.perm, self.topk, self.R_max, self.seg, self.shape_gu,
            self.w_gu, self.q_gu, self.ds_gu, self.dzp_gu, ws))
        fq_moe_unpermute_reduce(self.dxq, self.row_of[:T], x, T, self.topk, self.H, self.aq1,
                                self.dx[:T], self.ds_a1, self.ws)
        if self.overlap_wgrad:
            # the caller's stream sees both dScale results, and the next step's
            # forward cannot overwrite xq_tok / aq / do / dh under a wgrad still running
            main.wait_stream(self.side)
        return self.dx[:T], self.ds_gu, self.ds_d

    def step(self, x, expert_ids, probs, dout):
        """The whole hot path once: FQ pass, forward, scale-only backward."""
        self.quantize_weights()
        self.forward(x, expert_ids, probs)
        return self.backward(x, probs, dout)
