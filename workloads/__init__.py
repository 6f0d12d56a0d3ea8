"""Seeded synthetic inputs for the preshuffle GEMM workloads.

This module is shared by the CPU oracle and by the GPU path. It only draws
random numbers and encodes them into the input formats (INT8, FP8 E4M3 with
per-row fp32 scales, BF16, FP16, MXFP4 with E8M0 block scales, int8 x INT4
with per-row fp32 scales) and draws the optional epilogue bias. It holds none of the
GEMM's arithmetic: no decoding of those formats, no products, no sums, no
layout shuffle.

The workload shapes are the ones the GEMM Optimization Guide (rocm
gemm-optimization skill) tiles in §1.3 (small batch, medium batch, large batch,
FP4) and measures with the formulas of §8.1-§8.2. The pages publish no input
values; every input here is drawn from numpy's PCG64 with a fixed seed, A
before B, row-major.

Recipes:
  int8   integers uniform on {-8, ..., 8}.
  fp8    fp32 N(0,1); per row s = absmax(row) / 448 (fp32); code = E4M3FN(x / s)
         with round-to-nearest-even (torch's float8_e4m3fn cast after clamping
         to +-448); an all-zero row gets s = 1.
  bf16   fp32 N(0,1) rounded to bf16 with round-to-nearest-even (torch cast).
  fp16   fp32 N(0,1) rounded to IEEE fp16 with round-to-nearest-even (numpy cast).
  w4a8   A: fp32 N(0,1); per row s = absmax(row) / 127 (fp32), code = round-half-
         even(x / s) clamped to [-127, 127], int8. B: fp32 N(0,1); per row
         s = absmax(row) / 7, code = round-half-even(x / s) clamped to [-8, 7],
         two's complement nibbles, two per byte, the even k in the low nibble.
         fp32 scale_a[M], scale_b[N] as for FP8.
  bias   (fused epilogues, optional) fp32 N(0,1) * sqrt(K) per output column,
         drawn after A and B (so A and B do not change); sqrt(K) puts it on the
         scale of the GEMM output for N(0,1) operands.
  mxfp4  fp32 N(0,1); per 32-element K block: shared exponent
         e = floor(log2(amax)) - 2, clamped so that e + 127 lies in [0, 254]
         (a zero block gets e = 0); element = E2M1(x / 2^e) round-to-nearest-even,
         saturating at +-6; two elements per byte, the even k in the low nibble;
         the E8M0 scale byte is e + 127.
"""
from __future__ import annotations

import numpy as np

# name -> (dtype, M, N, K, seed, named tile (tile_m, tile_n, tile_k) or None)
CONFIGS = {
    "int8_128x256x512": ("int8", 128, 256, 512, 1, None),
    "fp8_16x7168x2048": ("fp8", 16, 7168, 2048, 2, None),
    "fp8_512x4096x4096": ("fp8", 512, 4096, 4096, 3, (64, 256, 128)),
    "bf16_8192x8192x8192": ("bf16", 8192, 8192, 8192, 4, (128, 256, 64)),
    "mxfp4_4096x4096x8192": ("mxfp4", 4096, 4096, 8192, 5, None),
    # next rows: FP16 inputs (fp16 out) and INT4 weights with int8 activations
    "fp16_8192x8192x8192": ("fp16", 8192, 8192, 8192, 7, None),
    "w4a8_16x7168x2048": ("w4a8", 16, 7168, 2048, 6, None),
    # W4A8 at a medium batch (the tile kernel's INT4 path), the FP8 medium shape
    "w4a8_512x4096x4096": ("w4a8", 512, 4096, 4096, 8, None),
}

# activations of the fused epilogues (with a bias; "none" = bias only)
EPILOGUE_ACTS = ("none", "relu", "silu", "gelu")

_FP8_MAX = 448.0
# E2M1 magnitudes of codes 0..7 (OCP MX v1.0 element format) used only to pick
# the nearest code when encoding; ties go to the even code.
_E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _normal(rng, shape) -> np.ndarray:
    return rng.standard_normal(shape, dtype=np.float32)


def _encode_fp8_rows(x: np.ndarray):
    import torch

    amax = np.abs(x).max(axis=1)
    s = (amax / np.float32(_FP8_MAX)).astype(np.float32)
    s[s == 0] = 1.0
    q = np.clip(x / s[:, None], -_FP8_MAX, _FP8_MAX).astype(np.float32)
    codes = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return np.ascontiguousarray(codes), s


def _encode_int_rows(x: np.ndarray, qmax: int, qmin: int):
    amax = np.abs(x).max(axis=1)
    s = (amax / np.float32(qmax)).astype(np.float32)
    s[s == 0] = 1.0
    q = np.clip(np.rint(x / s[:, None]), qmin, qmax).astype(np.int8)
    return q, s


def _pack_int4(q: np.ndarray) -> np.ndarray:
    u = (q.astype(np.int16) & 0xF).astype(np.uint8)
    return np.ascontiguousarray(u[:, 0::2] | (u[:, 1::2] << 4))


def _encode_bf16(x: np.ndarray) -> np.ndarray:
    import torch

    t = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy()
    return np.ascontiguousarray(t.view(np.uint16))


def _encode_e2m1(y: np.ndarray) -> np.ndarray:
    """Nearest E2M1 code (sign in bit 3), ties to even code, saturating."""
    mag = np.minimum(np.abs(y), 6.0)
    # index of the largest magnitude <= mag
    lo = np.searchsorted(_E2M1_MAG, mag, side="right") - 1
    hi = np.minimum(lo + 1, 7)
    dlo = mag - _E2M1_MAG[lo]
    dhi = _E2M1_MAG[hi] - mag
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0) & (hi != lo))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    sign = ((y < 0) & (code != 0)).astype(np.uint8) << 3
    return code | sign


def _encode_mxfp4(x: np.ndarray):
    rows, K = x.shape
    blk = x.reshape(rows, K // 32, 32).astype(np.float64)
    amax = np.abs(blk).max(axis=2)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 2
    e = np.where(amax > 0, e, 0.0)
    e = np.clip(e, -127, 127)
    scale_code = (e + 127).astype(np.uint8)
    codes = _encode_e2m1(blk / np.exp2(e)[:, :, None]).reshape(rows, K)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return np.ascontiguousarray(packed), np.ascontiguousarray(scale_code)


def make_inputs(dtype: str, M: int, N: int, K: int, seed: int, bias: bool = False) -> dict:
    """Draw A (M x K) then B (N x K) and encode them (then the bias, if asked).

    Returns numpy arrays:
      int8:  a int8[M,K], b int8[N,K]
      fp8:   a uint8[M,K], b uint8[N,K] (E4M3FN codes), scale_a f32[M], scale_b f32[N]
      bf16:  a uint16[M,K], b uint16[N,K] (bf16 bit patterns)
      mxfp4: a uint8[M,K/2], b uint8[N,K/2] (packed E2M1), scale_a uint8[M,K/32],
             scale_b uint8[N,K/32] (E8M0 codes)
      fp16:  a uint16[M,K], b uint16[N,K] (fp16 bit patterns)
      w4a8:  a int8[M,K], b uint8[N,K/2] (packed int4), scale_a f32[M], scale_b f32[N]
    plus bias f32[N] when `bias` is set.
    """
    rng = _rng(seed)
    out = _draw(rng, dtype, M, N, K)
    if bias:
        out["bias"] = (rng.standard_normal(N, dtype=np.float32) * np.float32(np.sqrt(K))).astype(np.float32)
    return out


def _draw(rng, dtype, M, N, K) -> dict:
    if dtype == "int8":
        a = rng.integers(-8, 9, size=(M, K), dtype=np.int8)
        b = rng.integers(-8, 9, size=(N, K), dtype=np.int8)
        return {"a": a, "b": b}
    if dtype == "fp8":
        a, sa = _encode_fp8_rows(_normal(rng, (M, K)))
        b, sb = _encode_fp8_rows(_normal(rng, (N, K)))
        return {"a": a, "b": b, "scale_a": sa, "scale_b": sb}
    if dtype == "bf16":
        a = _encode_bf16(_normal(rng, (M, K)))
        b = _encode_bf16(_normal(rng, (N, K)))
        return {"a": a, "b": b}
    if dtype == "fp16":
        a = _normal(rng, (M, K)).astype(np.float16).view(np.uint16)
        b = _normal(rng, (N, K)).astype(np.float16).view(np.uint16)
        return {"a": np.ascontiguousarray(a), "b": np.ascontiguousarray(b)}
    if dtype == "w4a8":
        assert K % 2 == 0
        a, sa = _encode_int_rows(_normal(rng, (M, K)), 127, -127)
        q, sb = _encode_int_rows(_normal(rng, (N, K)), 7, -8)
        return {"a": a, "b": _pack_int4(q), "scale_a": sa, "scale_b": sb}
    if dtype == "mxfp4":
        assert K % 32 == 0
        a, sa = _encode_mxfp4(_normal(rng, (M, K)))
        b, sb = _encode_mxfp4(_normal(rng, (N, K)))
        return {"a": a, "scale_a": sa, "b": b, "scale_b": sb}
    raise ValueError(f"unknown dtype {dtype!r}")


def make_config(name: str, bias: bool = False) -> dict:
    dtype, M, N, K, seed, _ = CONFIGS[name]
    return make_inputs(dtype, M, N, K, seed, bias=bias)


def elem_bytes(dtype: str) -> float:
    """Bytes per B element (A is int8 for W4A8)."""
    return {"int8": 1, "fp8": 1, "bf16": 2, "fp16": 2, "mxfp4": 0.5, "w4a8": 0.5}[dtype]
