"""Comparison of a bf16 / fp16 GPU result with the float64 oracle (test infrastructure).

Tolerances for the floating-point paths (FP8, BF16, MXFP4, W4A8 with bf16
output; FP16 with fp16 output):
  * normwise   ||C - R||_F / ||R||_F <= 2e-3
  * elementwise max_i |C_i - R_i| / max(|R_i|, tau) <= 1e-2,
    tau = 1e-2 * RMS(R).
The floor tau is needed because the literal |C_i - R_i| / |R_i| is unbounded
for outputs that cancel to nearly zero: fp32 accumulation leaves an absolute
error of order sqrt(K) * 2^-24 * RMS(products), which is a large relative
error when |R_i| is tiny, even for a correctly rounded kernel. For every other
output, bf16 round-to-nearest-even alone contributes at most 2^-9 relative
(fp16: 2^-12).
The literal value is reported alongside.
"""
from __future__ import annotations

import numpy as np

from .formats import decode_bf16, decode_f16

NORMWISE_TOL = 2e-3
ELEM_TOL = 1e-2
FLOOR_FRAC = 1e-2


def bf16_rne(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 (ties to even), returned as float64.

    Rounds once, straight from float64, by adding the rounding increment to
    the binary64 significand (used for diagnostics only).
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                     # x = m * 2^e, 0.5 <= |m| < 1
    scaled = np.ldexp(m, 8)                # 8 significant bits of bf16
    r = np.round(scaled)                   # numpy rounds half to even
    return np.ldexp(r, e - 8)


def f16_rne(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest fp16 (ties to even, normal range), as float64."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    scaled = np.ldexp(m, 11)               # 11 significant bits of fp16
    return np.ldexp(np.round(scaled), e - 11)


def compare_bf16(c_bits: np.ndarray, ref: np.ndarray) -> dict:
    """Metrics of a bf16 result (uint16 bit patterns) against float64 ref."""
    return compare_values(decode_bf16(np.asarray(c_bits).view(np.uint16)), ref)


def compare_f16(c_bits: np.ndarray, ref: np.ndarray) -> dict:
    """Metrics of an fp16 result (uint16 bit patterns) against float64 ref."""
    return compare_values(decode_f16(np.asarray(c_bits).view(np.uint16)), ref)


def compare_values(c: np.ndarray, ref: np.ndarray) -> dict:
    """Metrics of decoded result values (float64) against float64 ref."""
    c = np.asarray(c, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    if c.shape != r.shape:
        raise ValueError(f"shape mismatch {c.shape} vs {r.shape}")
    diff = np.abs(c - r)
    rn = np.sqrt(np.sum(r * r))
    rms = np.sqrt(np.mean(r * r)) if r.size else 0.0
    tau = FLOOR_FRAC * rms
    normwise = float(np.sqrt(np.sum(diff * diff)) / rn) if rn > 0 else float(np.sqrt(np.sum(diff * diff)))
    denom = np.maximum(np.abs(r), tau)
    with np.errstate(divide="ignore", invalid="ignore"):
        elem = np.where(denom > 0, diff / denom, np.where(diff > 0, np.inf, 0.0))
        lit = np.where(np.abs(r) > 0, diff / np.abs(r), np.where(diff > 0, np.inf, 0.0))
    return {
        "normwise": normwise,
        "elem_floored": float(elem.max()) if elem.size else 0.0,
        "elem_literal": float(lit.max()) if lit.size else 0.0,
        "n_literal_over": int(np.sum(lit > ELEM_TOL)),
        "nonfinite": int(np.sum(~np.isfinite(c))),
        "ok": bool(normwise <= NORMWISE_TOL and (elem.max() if elem.size else 0.0) <= ELEM_TOL
                   and np.all(np.isfinite(c))),
    }
