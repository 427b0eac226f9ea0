#!/usr/bin/env python3
"""Benchmark of the dense linear-layer GEMM on one MI355X.

Placeholder: formulas only (the timed driver is added with the GPU path).
"""
from __future__ import annotations

# --------------------------------------------------------------- formulas
# Dense peaks and HBM bandwidth of one MI355X (AMD's published figures; dense,
# no sparsity): 256 CUs at 2.4 GHz.
PEAK_TFLOPS = {"bf16": 2516.6, "fp8": 5033.2}
PEAK_HBM_GBPS = 8000.0


def flops(M: int, N: int, K: int) -> float:
    """2*M*N*K: each multiply-add is two flops ("GEMM Optimization Guide"
    page, section 8.1)."""
    return 2.0 * M * N * K


def alg_bytes(M: int, N: int, K: int, dtype: str, scales: str = "per_tensor") -> float:
    """Algorithmic HBM bytes: every operand read once and C written once.

    bf16: 2*(M*K + N*K + M*N) (the 16-bit operand/output reading of the
    FLOPS/Byte column on the TraceLens GEMM analysis page).  fp8: the
    "GEMM Optimization Guide" page, section 8.2 (1-byte A and B, bf16 C) with
    the scales as stored: two fp32 per-tensor scales (8 bytes) here, or
    (M + N) fp32 per-token scales as on that page."""
    if dtype == "bf16":
        return 2.0 * (M * K + N * K + M * N)
    if dtype == "fp8":
        sc = 8.0 if scales == "per_tensor" else 4.0 * (M + N)
        return 1.0 * M * K + 1.0 * N * K + 2.0 * M * N + sc
    raise ValueError(dtype)


def tflops_at(M: int, N: int, K: int, us: float) -> float:
    return flops(M, N, K) / (us * 1e-6) / 1e12


def roofline_us(M: int, N: int, K: int, dtype: str) -> float:
    """Lower bound on time: max of the MFMA time and the HBM time."""
    t_c = flops(M, N, K) / (PEAK_TFLOPS[dtype] * 1e12)
    t_m = alg_bytes(M, N, K, dtype) / (PEAK_HBM_GBPS * 1e9)
    return max(t_c, t_m) * 1e6
