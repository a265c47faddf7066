"""Benchmark of the scale-only fake-quant MoE hot path on one MI355X.

One step = the whole routed-expert path of one MoE layer: the stacked
fake-quant pass over both weight stacks, permutation, activation FQ of each
token row, gate_up grouped GEMM (routed rows read as token rows through the
routing), SwiGLU + activation FQ, down grouped GEMM, combine, and
the backward to dX and the weight-scale gradients (dScale) only.

Workload (default): Qwen3-30B-A3B-shaped layer, 128 experts, hidden 2048,
expert FFN 768, 16384 tokens x top-8, NVFP4 weights and activations,
synthetic seeded inputs. Inputs are resident in HBM before timing starts.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 1..5]

Prints one JSON line (rank 0). The headline step time comes from HIP events
around the K timed steps only; the per-call breakdown comes from a separate
pass with HIP events around every call, so the headline carries no
instrumentation. --config 1 / 2 time the dense single-linear workloads (FQ
pass + forward + scale-only backward through the same grouped-GEMM calls with
one expert).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MI355X_BF16_PEAK_TFLOPS = 2500.0     # dense bf16 MFMA
MI355X_HBM_PEAK_GBS = 8000.0
FLOPS_PER_ROW = 6 * (2 * 768 * 2048 + 2048 * 768)   # 28,311,552 per routed row (fwd+bwd GEMMs)

# HBM bytes per GEMM launch from rocprofv3 FETCH_SIZE / WRITE_SIZE runs,
# scaled by a plain copy kernel's readings, recorded with a hash of the GEMM
# sources they were taken on; a kernel changed since then reports null.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_gemm_{workload}.json")
GEMM_SOURCES = ("gemm.hip", "codec.hpp", "common.hpp", "internal.hpp")


def gemm_source_hash() -> str:
    """SHA-256 of the GEMM sources' code: comments removed and whitespace
    collapsed, so that a change to the comments alone keeps the hash."""
    import hashlib
    import re
    h = hashlib.sha256()
    for name in GEMM_SOURCES:
        with open(os.path.join(ROOT, "moe_fake_quant_amd", "csrc", name)) as f:
            txt = f.read()
        txt = re.sub(r"/\*.*?\*/", " ", txt, flags=re.S)
        txt = re.sub(r"//[^\n]*", "", txt)
        h.update(" ".join(txt.split()).encode())
    return h.hexdigest()


def hbm_pass_bytes(T, H, Fh, R, topk):
    """Algorithmic HBM bytes of each elementwise call: every operand read
    once, every output written once (bf16 2 B, fp32 / int32 4 B)."""
    return {
        "fq_moe_permute": 12 * T * topk,
        "fq_actfq": 4 * T * H,
        "fq_swiglu_actfq": R * (4 * Fh + 2 * Fh),
        "fq_moe_combine": 2 * R * H + 8 * T * topk + 2 * T * H,
        "fq_moe_combine_bwd": 2 * T * H + 8 * T * topk + 2 * R * H,
        "fq_swiglu_bwd": R * (2 * Fh + 4 * Fh + 4 * Fh),
        "fq_moe_unpermute_reduce": 2 * R * H + 4 * T * topk + 2 * T * H + 2 * T * H,
    }


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=4, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--breakdown-steps", type=int, default=10,
                    help="steps of the separate instrumented pass (per-call times)")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the measured MFMA-chain and copy peaks")
    ap.add_argument("--no-overlap", action="store_true",
                    help="keep the wgrad calls on the launch stream in the timed steps too "
                         "(for kernel traces whose per-kernel durations are their own)")
    ap.add_argument("--act-scales", choices=["frozen", "learnable"], default="frozen",
                    help="learnable: the backward also forms the activation-scale gradients "
                         "(fp8 workload only)")
    ap.add_argument("--weight-scales", choices=["default", "per-tensor"], default="default",
                    help="per-tensor: one scale per expert matrix (fp8 workload only)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the graph-replay figure of the MoE step")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the measurements outside the step (export decode, self-teacher "
                         "forward, top-K KL)")
    ap.add_argument("--cpu-sample-experts", type=int, default=6)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="after timing, run one plain device copy of this many MiB (a known "
                         "traffic reference for HBM byte counters)")
    return ap.parse_args()


class KernelTimer:
    """HIP events (torch.cuda.Event on the current stream, which is the stream
    every libfq call is enqueued on) around named ABI calls."""

    def __init__(self, torch):
        self.torch = torch
        self.pending = []
        self.enabled = False

    def wrap(self, key, fn):
        def inner(*a, **k):
            if not self.enabled:
                return fn(*a, **k)
            s = self.torch.cuda.Event(enable_timing=True)
            e = self.torch.cuda.Event(enable_timing=True)
            s.record()
            r = fn(*a, **k)
            e.record()
            self.pending.append((key(a), s, e))
            return r
        return inner

    def collect(self):
        out = {}
        for name, s, e in self.pending:
            out.setdefault(name, []).append(s.elapsed_time(e))
        self.pending = []
        return out


def measure_export(torch, F, layer, fmt, reps=10):
    """Real-quantized export of both stacks, outside the training step: the
    codes from the FQ pass, the stored scale bytes, and the decode back to
    bf16. Reports the decode kernel's HBM rate (codes + scale bytes read,
    bf16 written) over `reps` launches per stack."""
    out = {}
    total_b, total_ms = 0, 0.0
    for name, w, shape, q in (("gate_up", layer.w_gu, layer.shape_gu, layer.q_gu),
                              ("down", layer.w_d, layer.shape_d, layer.q_d)):
        E, N, K = shape
        nel = E * N * K
        four_bit = fmt in (F.FMT_NVFP4, F.FMT_INT4)
        codes = torch.empty(nel // 2 if four_bit else nel, dtype=torch.uint8, device=w.device)
        sb = torch.empty(nel // 16, dtype=torch.uint8, device=w.device) \
            if fmt == F.FMT_NVFP4 else None
        F.fq_quantize_stacked(w, shape, q, None, codes)
        if sb is not None:
            F.fq_export_scales(shape, q, sb, None)
        dec = torch.empty_like(w)
        scale = None if fmt == F.FMT_NVFP4 else q.scale
        F.fq_dequantize_stacked(codes, shape, fmt, q.group, dec, scale, sb, None, q.global_scale)
        torch.cuda.synchronize()
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(reps):
            F.fq_dequantize_stacked(codes, shape, fmt, q.group, dec, scale, sb, None,
                                    q.global_scale)
        e.record()
        torch.cuda.synchronize()
        ms = s.elapsed_time(e) / reps
        nbytes = codes.numel() + (sb.numel() if sb is not None else q.scale.numel() * 4) + 2 * nel
        out[name] = {"bytes": nbytes, "ms": round(ms, 4),
                     "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1)}
        total_b += nbytes
        total_ms += ms
    out["decode_GB/s"] = round(total_b / (total_ms * 1e-3) / 1e9, 1)
    out["pct_hbm_peak"] = round(100 * out["decode_GB/s"] / MI355X_HBM_PEAK_GBS, 1)
    return out


def measure_distill(torch, F, W, layer, x, ids, probs, reps=10):
    """The self-distillation pieces, outside the training step: the layer's
    quantization-off teacher forward on the same batch, and the top-K KL
    kernel on synthetic [4096, 151936] logits (teacher top-1000). The KL
    kernel's algorithmic bytes per token: the teacher row once (2V), the
    student at the K entries (2K), the outputs (8K + 4)."""
    for _ in range(2):
        layer.teacher_forward(x, ids, probs)
    torch.cuda.synchronize()
    s0 = torch.cuda.Event(enable_timing=True)
    e0 = torch.cuda.Event(enable_timing=True)
    s0.record()
    for _ in range(reps):
        layer.teacher_forward(x, ids, probs)
    e0.record()
    torch.cuda.synchronize()
    t_ms = s0.elapsed_time(e0) / reps
    R = int(layer.seg[layer.E].item())
    fwd_flops = 2 * R * (2 * layer.F * layer.H + layer.H * layer.F)

    T, V, K = W.KD_TOKENS, W.KD_VOCAB, W.KD_TOPK
    st, te = W.kd_logits(T, V, seed=0, device="cuda")
    idx = torch.empty(T, K, dtype=torch.int32, device="cuda")
    g = torch.empty(T, K, device="cuda")
    lt = torch.empty(T, device="cuda")
    lm = torch.empty(1, device="cuda")
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    out = {"teacher_forward": {"ms": round(t_ms, 4),
                               "TFLOP/s": round(fwd_flops / (t_ms * 1e-3) / 1e12, 2)}}
    nbytes = T * (2 * V + 2 * K + 8 * K + 4)
    for reverse in (False, True):
        F.fq_topk_kl(st, te, T, V, K, reverse, None, idx, g, lt, lm, ws)
        torch.cuda.synchronize()
        s1 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        s1.record()
        for _ in range(reps):
            F.fq_topk_kl(st, te, T, V, K, reverse, None, idx, g, lt, lm, ws)
        e1.record()
        torch.cuda.synchronize()
        ms = s1.elapsed_time(e1) / reps
        out["r_kl_top_K" if reverse else "kl_top_K"] = {
            "workload": W.KD_NAME, "ms": round(ms, 4), "bytes": nbytes,
            "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "pct_hbm_peak": round(100 * nbytes / (ms * 1e-3) / 1e9 / MI355X_HBM_PEAK_GBS, 1),
            "loss_mean": round(float(lm.cpu()[0]), 6)}
    floor = kl_pattern_floor(torch, te, st, idx, T, V, K, reps)
    if floor is not None:
        out["kl_pattern_floor"] = floor
        for key in ("kl_top_K", "r_kl_top_K"):
            out[key]["pct_of_pattern_floor"] = round(100 * floor["ms"] / out[key]["ms"], 1)
    del st, te
    return out


def kl_pattern_floor(torch, teacher, student, idx, T, V, K, reps):
    """The floor of the top-K KL kernel's memory pattern: a plain kernel that
    reads each teacher row once, the student at the K indices the KL kernel
    selected, and writes 8K + 4 bytes per token, with no selection or softmax
    work. Bytes = T (2V + 2K + 4K + 8K + 4) (it also reads the indices)."""
    import ctypes
    lib_path = os.path.join(ROOT, "moe_fake_quant_amd", "libfqpeaks.so")
    if not os.path.exists(lib_path):
        return None
    # the probe reads student[t, idx[t, k]]: every index must lie in the row
    lo, hi = int(idx.min().item()), int(idx.max().item())
    if lo < 0 or hi >= V:
        return None
    lib = ctypes.CDLL(lib_path)
    lib.fqp_stream_gather.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int] * 3 + \
        [ctypes.c_void_p] * 4
    dev = teacher.device
    oi = torch.empty(T, K, dtype=torch.int32, device=dev)
    of = torch.empty(T, K, device=dev)
    ol = torch.empty(T, dtype=torch.int32, device=dev)
    st = torch.cuda.current_stream().cuda_stream
    args = (teacher.data_ptr(), student.data_ptr(), idx.data_ptr(), T, V, K, oi.data_ptr(),
            of.data_ptr(), ol.data_ptr(), st)
    assert lib.fqp_stream_gather(*args) == 0
    torch.cuda.synchronize()
    s0 = torch.cuda.Event(enable_timing=True)
    e0 = torch.cuda.Event(enable_timing=True)
    s0.record()
    for _ in range(reps):
        assert lib.fqp_stream_gather(*args) == 0
    e0.record()
    torch.cuda.synchronize()
    ms = s0.elapsed_time(e0) / reps
    nbytes = T * (2 * V + 2 * K + 4 * K + 8 * K + 4)
    del oi, of, ol
    return {"ms": round(ms, 4), "bytes": nbytes, "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1)}


def measured_peaks(torch, dev):
    """The part's own ceilings, measured in the same run: a register-only chain
    of bf16 MFMA 32x32x16 on every CU (1 wave per SIMD, 8 independent
    accumulators; random operand bits and constant 1.0, since the clock under
    MFMA load depends on the operand bits), a plain 1 GiB device copy with
    one 16-byte vector per thread (read + write bytes), and the grouped
    GEMM's operand stream without its MFMAs."""
    import ctypes
    lib_path = os.path.join(ROOT, "moe_fake_quant_amd", "libfqpeaks.so")
    if not os.path.exists(lib_path):
        return None
    lib = ctypes.CDLL(lib_path)
    lib.fqp_mfma_chain.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_void_p]
    lib.fqp_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    st = torch.cuda.current_stream().cuda_stream
    n_cu = torch.cuda.get_device_properties(dev).multi_processor_count
    blocks, iters = n_cu, 8000   # one 4-wave block per CU: one wave per SIMD
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    res = {}
    for name, rnd in (("random_operands", 1), ("constant_operands", 0)):
        assert lib.fqp_mfma_chain(out.data_ptr(), blocks, 20, rnd, st) == 0
        torch.cuda.synchronize()
        s0 = torch.cuda.Event(enable_timing=True)
        e0 = torch.cuda.Event(enable_timing=True)
        s0.record()
        assert lib.fqp_mfma_chain(out.data_ptr(), blocks, iters, rnd, st) == 0
        e0.record()
        torch.cuda.synchronize()
        ms = s0.elapsed_time(e0)
        flops = 32 * 32 * 16 * 2 * 8 * iters * blocks * 4
        res[name] = round(flops / (ms * 1e-3) / 1e12, 1)
    nbytes = 1 << 30
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    assert lib.fqp_copy(src.data_ptr(), dst.data_ptr(), nbytes, st) == 0
    torch.cuda.synchronize()
    s1 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    s1.record()
    for _ in range(5):
        assert lib.fqp_copy(src.data_ptr(), dst.data_ptr(), nbytes, st) == 0
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * nbytes * 5 / (s1.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst, out
    # the grouped GEMM's operand stream alone (its two-stage LDS ring, 64 KiB per
    # 64-deep stage of a 256 x 256 tile, panels shared as the forward shares
    # them): the rate a tile of this design cannot beat, as TFLOP/s of the tile
    lib.fqp_operand_stream.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_void_p]
    panels, ntiles = 512, 12
    xs = torch.empty(panels << 20, dtype=torch.uint8, device=dev)
    ws = torch.empty(panels << 20, dtype=torch.uint8, device=dev)
    xs.fill_(0x3c)
    ws.fill_(0x3c)
    assert lib.fqp_operand_stream(xs.data_ptr(), ws.data_ptr(), panels, n_cu, 2, st) == 0
    torch.cuda.synchronize()
    s2 = torch.cuda.Event(enable_timing=True)
    e2 = torch.cuda.Event(enable_timing=True)
    s2.record()
    for _ in range(3):
        assert lib.fqp_operand_stream(xs.data_ptr(), ws.data_ptr(), panels, n_cu, ntiles, st) == 0
    e2.record()
    torch.cuda.synchronize()
    ms_s = s2.elapsed_time(e2) / 3
    del xs, ws
    stages = ntiles * 32
    tile_tflops = 2 * 256 * 256 * 64 * n_cu * stages / (ms_s * 1e-3) / 1e12
    return {"mfma_bf16_chain_TFLOP/s": res,
            "mfma_bf16_chain_pct_of_spec": round(100 * res["random_operands"] / MI355X_BF16_PEAK_TFLOPS, 1),
            "copy_GB/s": round(copy_gbs, 1),
            "copy_pct_of_spec": round(100 * copy_gbs / MI355X_HBM_PEAK_GBS, 1),
            "gemm_operand_stream": {"us_per_stage": round(ms_s * 1e3 / stages, 3),
                                    "tile_TFLOP/s": round(tile_tflops, 1)}}


def library_gemm(torch, dev, shapes, reps=20):
    """A vendor-library reference: torch's bf16 GEMM (hipBLASLt) timed in the
    same run. shapes: (batch, M, N, K) each, a batched product over `batch`
    equal problems (random operands, both contiguous: [batch, M, K] and
    [batch, K, N]); the rate is over all of them together."""
    ops = []
    for b, m, n, k in shapes:
        a = torch.randn(b, m, k, device=dev, dtype=torch.bfloat16)
        w = torch.randn(b, k, n, device=dev, dtype=torch.bfloat16)
        ops.append((a, w))
    def run():
        for a, w in ops:
            torch.bmm(a, w)
    for _ in range(3):
        run()
    torch.cuda.synchronize()
    s0 = torch.cuda.Event(enable_timing=True)
    e0 = torch.cuda.Event(enable_timing=True)
    s0.record()
    for _ in range(reps):
        run()
    e0.record()
    torch.cuda.synchronize()
    ms = s0.elapsed_time(e0) / reps
    flops = sum(2.0 * b * m * n * k for b, m, n, k in shapes)
    del ops
    return {"TFLOP/s": round(flops / (ms * 1e-3) / 1e12, 1), "ms": round(ms, 4),
            "shapes_batch_m_n_k": [list(t) for t in shapes]}


def scattered_rows_floor(torch, dev, rows, row_of, T, topk, H):
    """The floor of the per-token passes over routed rows: a plain kernel with
    their access pattern timed on the same buffers, 16 bytes per thread. Read
    direction (combine, unpermute-reduce): per token row written, its topk
    routed rows read at the real routing positions. Write direction (combine
    backward): per token row read, written to its topk routed rows. Bytes =
    2RH + 2TH + 4Tk either way."""
    import ctypes
    lib_path = os.path.join(ROOT, "moe_fake_quant_amd", "libfqpeaks.so")
    if not os.path.exists(lib_path):
        return None
    lib = ctypes.CDLL(lib_path)
    lib.fqp_scattered_rows.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    st = torch.cuda.current_stream().cuda_stream
    out = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
    args = (rows.data_ptr(), row_of.data_ptr(), T, topk, 2 * H, out.data_ptr(), st)
    assert lib.fqp_scattered_rows(*args) == 0
    torch.cuda.synchronize()
    s0 = torch.cuda.Event(enable_timing=True)
    e0 = torch.cuda.Event(enable_timing=True)
    s0.record()
    for _ in range(10):
        assert lib.fqp_scattered_rows(*args) == 0
    e0.record()
    torch.cuda.synchronize()
    ms = s0.elapsed_time(e0) / 10
    R = int((row_of[:T] >= 0).sum().item())
    nbytes = 2 * R * H + 2 * T * H + 4 * T * topk
    # write direction: the token rows of `out` to fresh routed rows
    lib.fqp_scattered_rows_w.argtypes = lib.fqp_scattered_rows.argtypes
    dst = torch.empty_like(rows)
    wargs = (out.data_ptr(), row_of.data_ptr(), T, topk, 2 * H, dst.data_ptr(), st)
    assert lib.fqp_scattered_rows_w(*wargs) == 0
    torch.cuda.synchronize()
    s0.record()
    for _ in range(10):
        assert lib.fqp_scattered_rows_w(*wargs) == 0
    e0.record()
    torch.cuda.synchronize()
    ms_w = s0.elapsed_time(e0) / 10
    del out, dst
    return {"ms": round(ms, 4), "bytes": nbytes, "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "write_ms": round(ms_w, 4), "write_GB/s": round(nbytes / (ms_w * 1e-3) / 1e9, 1)}


def host_description():
    """CPU model and the cores this process may run on (the GPU machine's host)."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        cpus = len(os.sched_getaffinity(0))
    except AttributeError:
        cpus = os.cpu_count()
    return model, cpus


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([p["num_threads"] for p in threadpool_info() if p.get("user_api") == "blas"]
                   or [1])
    except Exception:
        return 1


def time_steps(torch, step, steps):
    """HIP events around `steps` calls of step() on the current stream."""
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for _ in range(steps):
        step()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps, time.perf_counter() - t0


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): the library has no "
              "multi-GPU path (expert parallelism across GPUs is designed, not implemented).",
              file=sys.stderr)
        sys.exit(2)
    if args.config in (1, 2):
        return dense_main(args)
    import torch
    import moe_fake_quant_amd as F
    import workloads as W

    dev = torch.device("cuda:0")
    fmt = {3: F.FMT_FP8_E4M3, 4: F.FMT_NVFP4, 5: F.FMT_NVFP4}[args.config]
    learn = args.act_scales == "learnable"
    per_tensor = args.weight_scales == "per-tensor"
    if (learn or per_tensor) and fmt != F.FMT_FP8_E4M3:
        print("learnable activation scales and per-tensor weight scales exist for the fp8 "
              "workload (--config 3) only", file=sys.stderr)
        sys.exit(2)
    group = (F.FQ_GROUP_TENSOR if per_tensor else None) if fmt == F.FMT_FP8_E4M3 else 16
    t_gen = time.time()
    case = W.config(args.config, seed=args.seed)
    bf = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)  # noqa: E731
    w_gu, w_d = bf(case.w_gu), bf(case.w_d)
    x = bf(case.x)
    ids = torch.from_numpy(case.expert_ids).to(dev)
    probs = torch.from_numpy(case.probs).to(dev)
    dout = bf(case.dout)
    t_gen = time.time() - t_gen

    # the part's own ceilings first, before the workload has heated it
    peaks = None if args.no_peaks else measured_peaks(torch, dev)
    if peaks:
        # each GEMM kind of both stacks with every expert given the mean row
        # count: no routing, no ragged tails, no fake-quant, and for wgrad the
        # plain dW product without the dScale epilogue
        E_l, F2, H_ = case.w_gu.shape
        local = (case.expert_ids >= case.expert_begin) & (case.expert_ids < case.expert_begin + E_l)
        r = max(int(local.sum()) // E_l, 1)
        peaks["library_batched_gemm"] = {
            "gemm_fwd": library_gemm(torch, dev, [(E_l, r, F2, H_), (E_l, r, H_, F2 // 2)]),
            "gemm_dgrad": library_gemm(torch, dev, [(E_l, r, H_, F2), (E_l, r, F2 // 2, H_)]),
            "gemm_wgrad_dscale": library_gemm(torch, dev, [(E_l, F2, H_, r), (E_l, H_, F2 // 2, r)])}
    layer = F.MoEFakeQuantLayer(w_gu, w_d, fmt, fmt, case.T, case.topk, case.expert_begin, group,
                                learn_act_scales=learn)
    layer.init_weight_scales()
    layer.calibrate(x, ids)
    torch.cuda.synchronize()
    R = int(layer.seg[layer.E].item())
    E, H, Fh = layer.E, layer.H, layer.F

    # Events around every ABI call the layer makes, in the breakdown pass
    # only. Each GEMM call launches one kernel: fwd -> k_grouped_gemm<FWD>,
    # bwd with dx -> <DGRAD>, bwd with dscale -> <WGRAD> (dScale epilogue);
    # the FQ pass is one kernel per stack.
    timer = KernelTimer(torch)
    import moe_fake_quant_amd.layer as LM
    keys = {
        "fq_grouped_gemm_fwd": lambda a: "gemm_fwd",
        "fq_grouped_gemm_fwd_tokens": lambda a: "gemm_fwd",
        "fq_grouped_gemm_bwd_scale": lambda a: "gemm_dgrad" if a[9] is not None else "gemm_wgrad_dscale",
        "fq_grouped_gemm_wgrad_tokens": lambda a: "gemm_wgrad_dscale",
        "fq_quantize_stacked": lambda a: "fq_quantize_stacked",
    }
    for name in ("fq_quantize_stacked", "fq_moe_permute", "fq_actfq",
                 "fq_grouped_gemm_fwd", "fq_grouped_gemm_fwd_tokens", "fq_swiglu_actfq",
                 "fq_moe_combine", "fq_moe_combine_bwd", "fq_grouped_gemm_bwd_scale",
                 "fq_grouped_gemm_wgrad_tokens", "fq_swiglu_bwd", "fq_moe_unpermute_reduce"):
        setattr(LM, name, timer.wrap(keys.get(name, lambda a, n=name: n), getattr(LM, name)))

    layer.overlap_wgrad = not args.no_overlap
    overlap = layer.overlap_wgrad
    step = lambda: layer.step(x, ids, probs, dout)  # noqa: E731
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # headline: K whole steps bracketed by device syncs, events on the stream,
    # nothing else recorded inside
    timer.enabled = False
    ms_step, wall = time_steps(torch, step, args.steps)

    # the same step captured once in a HIP graph and replayed (reported beside
    # the eager headline, after a bit-for-bit check against the eager step)
    graph = None
    if not args.no_graph:
        outs = (layer.out[:case.T], layer.dx[:case.T], layer.ds_gu, layer.ds_d, layer.wfq_gu,
                layer.wfq_d)
        graph = graph_replay(torch, step, outs, args.steps, FLOPS_PER_ROW * R)
        graph["ms_per_step"] = round(graph.pop("us_per_step") / 1e3, 4)

    # breakdown: a separate pass with events around each call, the backward's
    # wgrad calls serialized on the launch stream so that every call's events
    # bracket its kernels alone
    nb = max(args.breakdown_steps, 1)
    layer.overlap_wgrad = False
    timer.enabled = True
    ms_step_instr, _ = time_steps(torch, step, nb)
    timer.enabled = False
    layer.overlap_wgrad = overlap
    per = timer.collect()

    flops_step = FLOPS_PER_ROW * R
    tflops = flops_step / (ms_step * 1e-3) / 1e12
    # each GEMM kind runs twice per step (gate_up and down); together
    # 2*R*(2F*H + H*F) flops
    kind_flops = 2 * R * (2 * Fh * H + H * Fh)
    kernels = {}
    for kind in ("gemm_fwd", "gemm_dgrad", "gemm_wgrad_dscale"):
        t = per.get(kind, [])
        ms = sum(t) / nb
        kernels[kind] = {"launches_per_step": len(t) // nb, "ms_per_step": round(ms, 4),
                         "avg_launch_ms": round(sum(t) / max(len(t), 1), 4),
                         "TFLOP/s": round(kind_flops / (ms * 1e-3) / 1e12, 2)}
    dom = max(kernels, key=lambda k: kernels[k]["ms_per_step"])
    achieved = kernels[dom]["TFLOP/s"]
    if peaks and peaks.get("gemm_operand_stream"):
        # the forward against the stream its own tiles need (both stacks' launches,
        # partial last rounds and ragged tails included)
        kernels["gemm_fwd"]["pct_of_operand_stream"] = round(
            100 * kernels["gemm_fwd"]["TFLOP/s"] / peaks["gemm_operand_stream"]["tile_TFLOP/s"], 1)
    if peaks and peaks.get("library_batched_gemm"):
        for k, ref in peaks["library_batched_gemm"].items():
            kernels[k]["pct_of_library_batched_gemm"] = round(100 * kernels[k]["TFLOP/s"] / ref["TFLOP/s"], 1)

    # FQ pass over both stacks: read bf16 + write bf16 + read the scales
    nel = E * (2 * Fh * H + H * Fh)
    if fmt == F.FMT_NVFP4:
        scale_bytes = (nel // 16) * 4 + 2 * E * 4
    elif per_tensor:
        scale_bytes = 2 * E * 4
    else:
        scale_bytes = E * (2 * Fh + H) * 4
    fq_bytes = nel * 4 + scale_bytes
    fq_ms = sum(per.get("fq_quantize_stacked", [0.0])) / nb
    fq_gbs = fq_bytes / (fq_ms * 1e-3) / 1e9

    traffic = None
    tfile = TRAFFIC_FILE.format(workload=W.CONFIG_NAMES[args.config])
    if os.path.exists(tfile):
        with open(tfile) as f:
            tr = json.load(f)
        if tr.get("gemm_sources_sha256") == gemm_source_hash() and dom in tr.get("kernels", {}):
            traffic = tr["kernels"][dom]["hbm_bytes_per_launch"]

    passes = {}
    for name, nbytes in hbm_pass_bytes(case.T, H, Fh, R, case.topk).items():
        ms = sum(per.get(name, [0.0])) / nb
        if ms > 0:
            passes[name] = {"bytes": nbytes, "ms": round(ms, 4),
                            "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
                            "pct_hbm_peak": round(100 * nbytes / (ms * 1e-3) / 1e9 / MI355X_HBM_PEAK_GBS, 1)}
    gemm_ms = sum(kernels[k]["ms_per_step"] for k in kernels)

    breakdown = {n: round(sum(v) / nb, 4) for n, v in sorted(per.items())}
    floor = None if args.no_peaks else scattered_rows_floor(torch, dev, layer.o, layer.row_of,
                                                            case.T, case.topk, H)
    if floor:
        for name, key in (("fq_moe_combine", "GB/s"), ("fq_moe_unpermute_reduce", "GB/s"),
                          ("fq_moe_combine_bwd", "write_GB/s")):
            if name in passes:
                passes[name]["pct_of_scattered_rows_floor"] = round(
                    100 * passes[name]["GB/s"] / floor[key], 1)
        if peaks is not None:
            peaks["scattered_rows_GB/s"] = floor["GB/s"]
            peaks["scattered_rows_write_GB/s"] = floor["write_GB/s"]

    if args.copy_calibration_mb > 0:
        n = args.copy_calibration_mb * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    export = distill = None
    if not args.no_extras:
        export = measure_export(torch, F, layer, fmt)
        distill = measure_distill(torch, F, W, layer, x, ids, probs)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(case, fmt, group, args.cpu_sample_experts)

    line = {
        "metric": "MoE fake-quant grouped-GEMM fwd+bwd TFLOP/s; % bf16 MFMA peak; FQ pass GB/s",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": W.CONFIG_NAMES[args.config],
            "experts": E, "hidden": H, "expert_ffn": Fh, "tokens": case.T, "topk": case.topk,
            "routed_rows": R, "weight_format": {3: "fp8_e4m3", 4: "nvfp4", 5: "nvfp4"}[args.config],
            "act_format": {3: "fp8_e4m3", 4: "nvfp4", 5: "nvfp4"}[args.config],
            "weight_scales": ("per-tensor" if per_tensor else "per-channel")
            if fmt == F.FMT_FP8_E4M3 else "block16",
            "act_scales": args.act_scales,
            "flops_per_step": flops_step,
        },
        "pct_bf16_peak": round(100 * tflops / MI355X_BF16_PEAK_TFLOPS, 2),
        "fq_pass": {"GB/s": round(fq_gbs, 1), "pct_hbm_peak": round(100 * fq_gbs / MI355X_HBM_PEAK_GBS, 2),
                    "bytes_per_step": fq_bytes, "ms_per_step": round(fq_ms, 4)},
        "roofline": {
            "kernel": dom,
            "bound": "mfma",
            "achieved": achieved,
            "peak": MI355X_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / MI355X_BF16_PEAK_TFLOPS, 4),
            "traffic": traffic,
        },
        "timing": {"headline": "HIP events around the timed steps, no per-call events; the wgrad "
                               + ("calls on a second stream" if overlap else
                                  "calls on the launch stream (--no-overlap)"),
                   "breakdown": "a separate pass with events around each call, all on one stream",
                   "breakdown_steps": nb, "breakdown_ms_per_step": round(ms_step_instr, 4)},
        "graph_replay": graph,
        "gemm_kernels": kernels,
        "gemm_only": {"ms_per_step": round(gemm_ms, 4),
                      "TFLOP/s": round(flops_step / (gemm_ms * 1e-3) / 1e12, 2)},
        "hbm_passes": passes,
        "measured_peaks": peaks,
        "export_decode": export,
        "distill": distill,
        "ms_per_step_by_call": breakdown,
        "cpu_baseline": cpu,
        "input_gen_s": round(t_gen, 1),
        "wall_s_timed": round(wall, 3),
    }
    print(json.dumps(line), flush=True)


def graph_replay(torch, step, outs, steps, flops_step):
    """The same step captured once in a HIP graph (torch.cuda.CUDAGraph over
    the ABI calls) and replayed `steps` times between the same device syncs:
    the rate without the host's per-kernel launch cost, which is most of a
    small step. The replay's outputs are compared bit for bit with the eager
    step's before it is timed."""
    torch.cuda.synchronize()
    eager = [t.clone() for t in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for t in outs:
        t.zero_()
    g.replay()
    torch.cuda.synchronize()
    same = all(torch.equal(a.view(torch.uint8), b.view(torch.uint8)) for a, b in zip(outs, eager))
    for _ in range(3):
        g.replay()
    ms, _ = time_steps(torch, g.replay, steps)
    return {"us_per_step": round(ms * 1e3, 2), "TFLOP/s": round(flops_step / (ms * 1e-3) / 1e12, 3),
            "bitwise_equal_to_eager": same}


def dense_main(args):
    """The dense single-linear workloads (one expert, seg = [0, M]): one step =
    FQ pass over W, forward Y = X . FQ(W)^T, backward dX and dScale (weights
    frozen), through the same grouped-GEMM calls as the MoE path."""
    import torch
    import moe_fake_quant_amd as F
    import workloads as W

    dev = torch.device("cuda:0")
    case = W.config(args.config, seed=args.seed)
    fmt = {1: F.FMT_INT8, 2: F.FMT_INT4}[args.config]
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)  # noqa: E731
    N, K = case.w.shape
    M = case.x.shape[0]
    shape = (1, N, K)
    group = case.group
    G = K // group
    w, x, dy = bf(case.w[None]), bf(case.x), bf(case.dy)
    s = torch.empty(1, N, G, device=dev)
    zp = torch.empty(1, N, G, device=dev) if fmt == F.FMT_INT4 else None
    F.observer_absmax_init(w, shape, fmt, group, 0, s, zp, None)
    q = F.WeightQ(fmt, group, s, zp, None)
    seg = torch.tensor([0, M], dtype=torch.int32, device=dev)
    wfq = torch.empty_like(w)
    ws = torch.empty(max(F.fq_workspace_bytes(F.FQ_OP_GEMM_FWD, shape, M, 0),
                         F.fq_workspace_bytes(F.FQ_OP_GEMM_BWD, shape, M, 0), 256),
                     dtype=torch.uint8, device=dev)
    y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    dx = torch.empty(M, K, dtype=torch.bfloat16, device=dev)
    ds = torch.empty(1, N, G, device=dev)
    dzp = torch.empty(1, N, G, device=dev) if fmt == F.FMT_INT4 else None

    calls = {
        "fq_quantize_stacked": lambda: F.fq_quantize_stacked(w, shape, q, wfq),
        "gemm_fwd": lambda: F.fq_grouped_gemm_fwd(x, M, seg, shape, None, wfq, q, None, y, ws),
        "gemm_dgrad": lambda: F.fq_grouped_gemm_bwd_scale(dy, x, M, seg, shape, w, wfq, q, None,
                                                          dx, None, None, ws),
        "gemm_wgrad_dscale": lambda: F.fq_grouped_gemm_bwd_scale(dy, x, M, seg, shape, w, wfq, q,
                                                                 None, None, ds, dzp, ws),
    }

    def step():
        for fn in calls.values():
            fn()

    peaks = None if args.no_peaks else measured_peaks(torch, dev)
    if peaks:
        peaks["library_batched_gemm"] = {
            "gemm_fwd": library_gemm(torch, dev, [(1, M, N, K)]),
            "gemm_dgrad": library_gemm(torch, dev, [(1, M, K, N)]),
            "gemm_wgrad_dscale": library_gemm(torch, dev, [(1, N, K, M)])}
    steps = args.steps * (50 if args.config == 1 else 1)   # the latency case: more reps
    for _ in range(args.warmup):
        step()
    ms_step, wall = time_steps(torch, step, steps)
    # per-call breakdown in a separate pass
    per = {}
    nb = max(args.breakdown_steps, 1) * (50 if args.config == 1 else 1)
    for name, fn in calls.items():
        ms, _ = time_steps(torch, fn, nb)
        per[name] = ms
    flops_step = 6 * M * N * K
    tflops = flops_step / (ms_step * 1e-3) / 1e12
    graph = graph_replay(torch, step, tuple(t for t in (wfq, y, dx, ds, dzp) if t is not None),
                         steps, flops_step)
    kind_flops = 2 * M * N * K
    kernels = {k: {"ms_per_step": round(per[k], 4), "avg_launch_ms": round(per[k], 4),
                   "TFLOP/s": round(kind_flops / (per[k] * 1e-3) / 1e12, 2)}
               for k in ("gemm_fwd", "gemm_dgrad", "gemm_wgrad_dscale")}
    dom = max(kernels, key=lambda k: kernels[k]["ms_per_step"])
    if peaks and peaks.get("library_batched_gemm"):
        for k, ref in peaks["library_batched_gemm"].items():
            kernels[k]["pct_of_library_batched_gemm"] = round(100 * kernels[k]["TFLOP/s"] / ref["TFLOP/s"], 1)
    nel = N * K
    scale_bytes = N * G * 4 * (2 if fmt == F.FMT_INT4 else 1)
    fq_bytes = nel * 4 + scale_bytes
    fq_gbs = fq_bytes / (per["fq_quantize_stacked"] * 1e-3) / 1e9
    cpu = None if args.no_cpu_baseline else cpu_baseline_dense(case, args.config)
    line = {
        "metric": "MoE fake-quant grouped-GEMM fwd+bwd TFLOP/s; % bf16 MFMA peak; FQ pass GB/s",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "us_per_step": round(ms_step * 1e3, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": W.CONFIG_NAMES[args.config], "M": M, "N": N, "K": K,
                   "weight_format": {1: "int8", 2: "int4"}[args.config],
                   "weight_scales": "per-channel" if group == K else f"group{group}",
                   "act_format": "none", "flops_per_step": flops_step},
        "pct_bf16_peak": round(100 * tflops / MI355X_BF16_PEAK_TFLOPS, 3),
        "fq_pass": {"GB/s": round(fq_gbs, 1), "pct_hbm_peak": round(100 * fq_gbs / MI355X_HBM_PEAK_GBS, 2),
                    "bytes_per_step": fq_bytes, "ms_per_step": round(per["fq_quantize_stacked"], 5)},
        "roofline": {"kernel": dom, "bound": "mfma", "achieved": kernels[dom]["TFLOP/s"],
                     "peak": MI355X_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(kernels[dom]["TFLOP/s"] / MI355X_BF16_PEAK_TFLOPS, 4),
                     "traffic": None},
        "timing": {"headline": "HIP events around the timed steps, no per-call events",
                   "breakdown": "each call timed alone over the same number of reps"},
        "gemm_kernels": kernels,
        "graph_replay": graph,
        "measured_peaks": peaks,
        "ms_per_step_by_call": {k: round(v, 5) for k, v in per.items()},
        "cpu_baseline": cpu,
        "wall_s_timed": round(wall, 3),
    }
    print(json.dumps(line), flush=True)


def cpu_baseline(case, fmt, group, n_experts):
    """The oracle, untuned, on the host cores: the same layer restricted to the
    first n_experts experts and their routed rows (a bounded sample)."""
    import oracle as O
    import workloads as W
    E = n_experts
    sub = W.MoECase(name=case.name, fmt=case.fmt, n_experts_global=case.n_experts_global,
                    expert_begin=0, w_gu=case.w_gu[:E], w_d=case.w_d[:E], x=case.x,
                    expert_ids=case.expert_ids, probs=case.probs, dout=case.dout)
    wfmt = O.FMT_NVFP4 if fmt == 4 else O.FMT_FP8
    _, _, seg = O.moe_permute(case.expert_ids, 0, E)
    R = int(seg[-1])
    model, cpus = host_description()
    t0 = time.perf_counter()
    # group: 16 (nvfp4 blocks), None (one scale per output channel) or the
    # per-tensor marker, the same values the oracle takes
    O.moe_layer(sub, wfmt, group, wfmt)
    dt = time.perf_counter() - t0
    flops = FLOPS_PER_ROW * R
    # the oracle's weight codec alone (the FQ pass) on the same sampled
    # stacks, scales from the observer beforehand; bytes as the GPU FQ pass
    # counts them: 2 B read + 2 B written per element, plus the NVFP4 theta
    stacks = []
    for w in (sub.w_gu, sub.w_d):
        g = group or w.shape[2]
        stacks.append((w, g, O.observer_weight(w, wfmt, g)))
    t1 = time.perf_counter()
    for w, g, wq in stacks:
        O.fq_weight_stack(w, wfmt, g, *wq)
    dt_codec = time.perf_counter() - t1
    n_el = sum(w.size for w, _, _ in stacks)
    codec_bytes = 4 * n_el + (n_el // 16 * 4 if wfmt == O.FMT_NVFP4 else 0)
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": blas_threads(),
            "kind": "oracle", "seconds": round(dt, 2), "cpu_model": model,
            "affinity_cpus": cpus,
            "sample": f"experts 0..{E - 1} of the same layer and their {R} routed rows "
                      f"(full fwd+bwd incl. observer init), {flops / 1e9:.1f} GFLOP",
            "codec_GB/s": round(codec_bytes / dt_codec / 1e9, 3),
            "codec_sample": f"the oracle's weight FQ over the same {E} experts' gate_up and down "
                            f"stacks, {codec_bytes / 1e9:.3f} GB in {dt_codec:.2f} s"}


def cpu_baseline_dense(case, cfg):
    """The oracle on the whole dense workload: observer, FQ pass, forward and
    the scale-only backward (float64 GEMMs through NumPy's BLAS)."""
    import oracle as O
    fmt = {1: O.FMT_INT8, 2: O.FMT_INT4}[cfg]
    N, K = case.w.shape
    M = case.x.shape[0]
    model, cpus = host_description()
    seg = np.array([0, M])
    t0 = time.perf_counter()
    wq = O.observer_weight(case.w[None], fmt, case.group)
    O.fq_weight_stack(case.w[None], fmt, case.group, *wq)
    O.grouped_gemm_fwd(case.x, seg, case.w[None], fmt, case.group, *wq)
    O.grouped_gemm_bwd(case.dy, case.x, seg, case.w[None], fmt, case.group, *wq)
    dt = time.perf_counter() - t0
    flops = 6 * M * N * K
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": blas_threads(),
            "kind": "oracle", "seconds": round(dt, 3), "cpu_model": model,
            "affinity_cpus": cpus,
            "sample": f"the whole workload (M={M}, N={N}, K={K}): observer, FQ pass, forward, "
                      f"dX and dScale, {flops / 1e9:.2f} GFLOP"}


if __name__ == "__main__":
    main()
