"""bf16 <-> fp32 conversions for the oracle (test infrastructure only).

The fake-quant output is cast back to the input dtype, bf16 (AngelSlim QAT +
ZeRO-3 page, section "Quantizer 的变更"); GEMM operands are bf16 (same
section, F.linear after aligning the input dtype to the weight's).

bf16 -> fp32 is exact (the 16 bits become the high half). fp32 -> bf16 is
round-to-nearest-even on the 16 dropped bits (inputs are finite here).
"""
import numpy as np


def bf16_to_f32(bits) -> np.ndarray:
    """Raw bf16 bits (uint16) -> exact float32 values."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16(x) -> np.ndarray:
    """float32 -> bf16 bits, round half to even on the dropped 16 bits."""
    u = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    u = u + np.uint64(0x7FFF) + lsb
    return (u >> np.uint64(16)).astype(np.uint16)


def f64_to_bf16(x) -> np.ndarray:
    """float64 -> bf16 bits via float32 (each step RNE).

    The GPU rounds its fp32 accumulator to bf16; the oracle accumulates in
    float64 and rounds through fp32 the same way. The two differ only at
    double-rounding ties, far inside the GEMM tolerance.
    """
    return f32_to_bf16(np.asarray(x, dtype=np.float64).astype(np.float32))
