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

FP16 (§6.2's f16 instruction) decodes IEEE binary16; W4A8 (§8.2's INT4
weights) multiplies int8 A by int4 B exactly in int64 and applies fp32
per-row / per-column scales like FP8.

Fused epilogues (Kernel Tuning Guide §6 lists bias, bias+ReLU, bias+SiLU and
bias+GELU): after the scales, an fp32 bias per output column is added and
the activation applied, all in float64:
    relu(x) = max(x, 0)
    silu(x) = x * sigmoid(x) = x / (1 + exp(-x))
    gelu(x) = x * Phi(x) = x/2 * (1 + erf(x / sqrt(2)))     (the exact, erf form)
The pages name the activations only; these are their standard definitions.

`rows` / `cols` select a subset of outputs (used to check sampled outputs of
large problems): the result is C[rows][:, cols].
"""
from __future__ import annotations

import numpy as np

from .formats import (decode_int8, decode_bf16, decode_e4m3, decode_e2m1, decode_e8m0, decode_f16,
                      decode_int4, unpack_fp4, unpack_nibbles)

ACTS = ("none", "relu", "silu", "gelu")


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


def gemm_f16(a, b, rows=None, cols=None) -> np.ndarray:
    """fp16 bits [M,K] x [N,K]^T -> float64."""
    A = decode_f16(_take(a, rows))
    B = decode_f16(_take(b, cols))
    return A @ B.T


def gemm_w4a8(a, b, scale_a, scale_b, rows=None, cols=None) -> np.ndarray:
    """int8 [M,K] x packed int4 [N,K/2]^T (exact int64), times scale_a[m] * scale_b[n] -> float64."""
    A = decode_int8(_take(a, rows))
    B = decode_int4(unpack_nibbles(_take(b, cols)))
    sa = np.asarray(_take(scale_a, rows), dtype=np.float32).astype(np.float64)
    sb = np.asarray(_take(scale_b, cols), dtype=np.float32).astype(np.float64)
    return (A @ B.T).astype(np.float64) * sa[:, None] * sb[None, :]


def activation(x: np.ndarray, act: str) -> np.ndarray:
    """The epilogue activation in float64 (definitions in the module docstring)."""
    from scipy.special import erf

    x = np.asarray(x, dtype=np.float64)
    if act == "none":
        return x
    if act == "relu":
        return np.maximum(x, 0.0)
    if act == "silu":
        with np.errstate(over="ignore"):
            return x / (1.0 + np.exp(-x))
    if act == "gelu":
        return 0.5 * x * (1.0 + erf(x / np.sqrt(2.0)))
    raise ValueError(act)


def apply_epilogue(r: np.ndarray, bias=None, act: str = "none", cols=None) -> np.ndarray:
    """act(R + bias[n]) with bias fp32 [N] (or None)."""
    out = np.asarray(r, dtype=np.float64)
    if bias is not None:
        out = out + np.asarray(_take(bias, cols), dtype=np.float32).astype(np.float64)[None, :]
    return activation(out, act)


def _dec_mx(packed, scale):
    vals = decode_e2m1(unpack_fp4(packed))                  # [R, K]
    s = decode_e8m0(scale)                                  # [R, K/32]
    return vals * np.repeat(s, 32, axis=1)


def gemm_mxfp4(a, scale_a, b, scale_b, rows=None, cols=None) -> np.ndarray:
    """Packed E2M1 [M,K/2] with E8M0 [M,K/32] x the same for B -> float64."""
    A = _dec_mx(_take(a, rows), _take(scale_a, rows))
    B = _dec_mx(_take(b, cols), _take(scale_b, cols))
    return A @ B.T


def _gemm(dtype, inputs, rows, cols):
    if dtype == "int8":
        return gemm_int8(inputs["a"], inputs["b"], rows, cols)
    if dtype == "fp8":
        return gemm_fp8(inputs["a"], inputs["b"], inputs["scale_a"], inputs["scale_b"], rows, cols)
    if dtype == "bf16":
        return gemm_bf16(inputs["a"], inputs["b"], rows, cols)
    if dtype == "fp16":
        return gemm_f16(inputs["a"], inputs["b"], rows, cols)
    if dtype == "mxfp4":
        return gemm_mxfp4(inputs["a"], inputs["scale_a"], inputs["b"], inputs["scale_b"], rows, cols)
    if dtype == "w4a8":
        return gemm_w4a8(inputs["a"], inputs["b"], inputs["scale_a"], inputs["scale_b"], rows, cols)
    raise ValueError(dtype)


def gemm(dtype: str, inputs: dict, rows=None, cols=None, act=None) -> np.ndarray:
    """Dispatch on the workload dtype with the input dict of workloads.make_inputs.

    With `act` given (one of ACTS), the fused epilogue is applied: the bias
    inputs["bias"] (if present) is added and the activation taken."""
    r = _gemm(dtype, inputs, rows, cols)
    if act is None:
        return r
    if dtype == "int8":
        raise ValueError("the INT8 -> int32 path has no fused epilogue")
    return apply_epilogue(r, inputs.get("bias"), act, cols)
