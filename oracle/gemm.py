"""The GEMM itself (oracle; test infrastructure only).

GEMM Optimization Guide §1.1 states the problem as C = A x B^T with A of M
rows and B read, per §12.1, as N rows of K contiguous elements; so

    C[m, n] = sum_k  dec(A[m, k]) * dec(B[n, k])

Per-element epilogue (§7.1): the accumulator is multiplied by the per-row
scale of A and the per-column scale of B (FP8, fp32 scales, §8.2 "per-token
scales"). MXFP4 (§6.2, §8.2): every 32-element K block of a row of A or B
carries one E8M0 scale that multiplies its elements.

Accumulation is exact: int64 for INT8 (checked to fit int32) and float64
otherwise. FP8 products are multiples of 2^-18 and the sums stay far below
2^35, so they are exact in float64; BF16 and FP4 sums carry at most about
K * 2^-53 relative error, far below the bf16 output rounding. The float64
product is numpy's matmul, used as a library primitive; there is no blocking,
reordering or fusion beyond decode-then-multiply.

`rows` / `cols` select a subset of outputs (used to check sampled outputs of
large problems): the result is C[rows][:, cols].
"""
from __future__ import annotations

import numpy as np

from .formats import decode_int8, decode_bf16, decode_e4m3, decode_e2m1, decode_e8m0, unpack_fp4


def _take(x, idx):
    return x if idx is None else np.asarray(x)[np.asarray(idx)]


def gemm_int8(a, b, rows=None, cols=None) -> np.ndarray:
    """int8 [M,K] x int8 [N,K]^T -> int32 [M,N], exact."""
    A = decode_int8(_take(a, rows))
    B = decode_int8(_take(b, cols))
    acc = A @ B.T
    if acc.size and np.abs(acc).max() >= 2**31:
        raise OverflowError("INT8 GEMM result does not fit int32")
    return acc.astype(np.int32)


def gemm_fp8(a, b, scale_a, scale_b, rows=None, cols=None) -> np.ndarray:
    """E4M3 codes [M,K] x [N,K]^T, times scale_a[m] * scale_b[n] -> float64."""
    A = decode_e4m3(_take(a, rows))
    B = decode_e4m3(_take(b, cols))
    sa = np.asarray(_take(scale_a, rows), dtype=np.float32).astype(np.float64)
    sb = np.asarray(_take(scale_b, cols), dtype=np.float32).astype(np.float64)
    return (A @ B.T) * sa[:, None] * sb[None, :]


def gemm_bf16(a, b, rows=None, cols=None) -> np.ndarray:
    """bf16 bits [M,K] x [N,K]^T -> float64."""
    A = decode_bf16(_take(a, rows))
    B = decode_bf16(_take(b, cols))
    return A @ B.T


def _dec_mx(packed, scale):
    vals = decode_e2m1(unpack_fp4(packed))                  # [R, K]
    s = decode_e8m0(scale)                                  # [R, K/32]
    return vals * np.repeat(s, 32, axis=1)


def gemm_mxfp4(a, scale_a, b, scale_b, rows=None, cols=None) -> np.ndarray:
    """Packed E2M1 [M,K/2] with E8M0 [M,K/32] x the same for B -> float64."""
    A = _dec_mx(_take(a, rows), _take(scale_a, rows))
    B = _dec_mx(_take(b, cols), _take(scale_b, cols))
    return A @ B.T


def gemm(dtype: str, inputs: dict, rows=None, cols=None) -> np.ndarray:
    """Dispatch on the workload dtype with the input dict of workloads.make_inputs."""
    if dtype == "int8":
        return gemm_int8(inputs["a"], inputs["b"], rows, cols)
    if dtype == "fp8":
        return gemm_fp8(inputs["a"], inputs["b"], inputs["scale_a"], inputs["scale_b"], rows, cols)
    if dtype == "bf16":
        return gemm_bf16(inputs["a"], inputs["b"], rows, cols)
    if dtype == "mxfp4":
        return gemm_mxfp4(inputs["a"], inputs["scale_a"], inputs["b"], inputs["scale_b"], rows, cols)
    raise ValueError(dtype)
