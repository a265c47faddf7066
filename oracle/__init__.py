"""CPU oracle for scale-only fake-quant MoE grouped GEMM -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously-correct NumPy implementation of what the HIP path
computes. Only the test suite, the smoke check and the benchmark's CPU-baseline
leg may import it; the product path (``moe_fake_quant_amd``) never does, and
this package imports nothing from it. The two share only the seeded input
generators in ``workloads``, which hold none of the method's arithmetic.

Sources (cited by page title and section):
  * "AngelSlim mcore_qad" article (hnwysp.cn news 88453): frozen BF16 weights,
    fake-quant (quantize->dequantize) of weights and activations, only the
    quantizer scales trainable (section 一); weights fake-quantized through a
    parametrization and inputs through a forward pre-hook, gradient reaching
    the scales by autograd (section 二.3); each MoE layer's experts stacked into
    one 3D tensor, fake-quantized as a whole, then one grouped GEMM (section
    二.4); the formats nvfp4 / fp8 / w4a16 / w8a8 (section 三).
  * "QAT + DeepSpeed ZeRO-3" page of the AngelSlim docs: the PTQ weight scale
    max|W|/448 (section "Quantizer 初始值"), fake_quant casting its output back
    to the input dtype and F.linear on bf16 operands (section "Quantizer 的变更"),
    learnable flags weight_scale true / act_scale false (example yaml).
  * msmodelslim multi-card quantisation page: observers keep per-channel
    min / max and turn them into quantisation parameters (FA3 observer section).
  * Format grids: OCP Microscaling Formats spec v1.0 (E4M3, E2M1), the
    standard definitions of the formats the pages name; the pages give no bit
    layouts.

Every point the pages leave open is a numbered reading; the code names the
reading where it applies:
  R-1  z = x * r with r = 1/s rounded once per scale (not x / s per element)
  R-2  integer formats dequantize to +0.0; FP formats keep the sign of z
  R-3  int8 symmetric range [-128, 127]
  R-4  an all-zero row / group / tensor gets scale 1
  R-5  int4 asymmetric: min / max widened to include 0, integer zero point
  R-6  E4M3 saturates at +-448, subnormals kept
  R-7  E2M1 ties go to the even code
  R-8  NVFP4: learnable fp32 theta re-rounded to E4M3 each forward; tensor
       scale g per expert per stack; one activation g_a per projection input
  R-9  a zero NVFP4 block scale makes the block +0.0 with mask and grad 0
  R-10 gate is the first F rows of the fused gate_up stack
  R-11 routing: softmax, top-k (ties to the lower id), renormalised
  R-12 no gradient into the router (logits are given data)
  R-13 STE mask lo <= z <= hi on the unrounded z, inclusive
  R-14 no LSQ gradient-scale factor
  R-15 dScale compared normwise (max |diff| / max |ref|)
  R-16 chained tests feed the GPU-calibrated activation scales to the oracle
  R-17 MoE weights drawn N(0, 0.02)
  R-18 the skewed local-share workload forces experts {3, 7, 11, 15} empty
  R-19 FP8 scales: weights per output channel amax/448, activations one
       frozen per-tensor amax/448 per projection input
  R-20 every stored intermediate is bf16; accumulation in fp64 here
  R-21 empty experts get dScale (and dZP) exactly 0
  R-22 in the layer, dA is masked by the act-FQ mask of A and dX by that of
       X; dynamic NVFP4 activation block scales are constants
  R-23 a learnable activation scale exists for the static per-tensor formats
       (FP8, INT8) only; its gradient uses the weights' STE factor, summed
       over every element the quantizer saw in the step. NVFP4 activations
       derive their block scales from the data and keep g_a at calibration.
  R-24 a per-tensor weight scale is one scale per expert matrix [N, K] of a
       stack (each expert is its own linear); INT8 / FP8 only
  R-25 top-K KL: the teacher's K largest logits per token (equal logits: lower
       index first), both distributions renormalised over that set, mean
       over valid tokens; only the student's logits get a gradient

Parity status: every function here is pinned by the ``-m "not gpu"`` tests
(exhaustive code grids, tie tables, library special cases, closed forms,
brute force, an independent torch-autograd derivation of the STE gradients),
except SwiGLU's exp and the routing generator, which are compared by
tolerance only ("parity unpinned" beyond the stated tolerances).
"""
from .numerics import bf16_to_f32, f32_to_bf16, f64_to_bf16  # noqa: F401
from .codecs import (  # noqa: F401
    FMT_NONE, FMT_INT8, FMT_INT4, FMT_FP8, FMT_NVFP4, FMT_NAMES, GROUP_TENSOR,
    E4M3_POS, E2M1_POS, E4M3_MAX, E2M1_MAX,
    e4m3_round, e2m1_round, e4m3_value_of_code, e2m1_value_of_code,
    fq_int8, fq_int4, fq_fp8, fq_nvfp4, fq_nvfp4_act_dynamic, nvfp4_dynamic_theta,
    fq_weight_stack, fq_act,
)
from .observer import observer_weight, observer_act  # noqa: F401
from .permute import moe_permute  # noqa: F401
from .gemm import grouped_gemm_fwd, grouped_gemm_bwd  # noqa: F401
from .export import pack_codes, unpack_codes, export_scales, dequantize  # noqa: F401
from .distill import topk_set, topk_kl  # noqa: F401
from .moe import (  # noqa: F401
    gather_actfq, swiglu_fwd, swiglu_actfq, swiglu_bwd, combine, combine_bwd,
    unpermute_reduce, unpermute_sum, act_scale_grad, moe_layer, teacher_forward,
)
