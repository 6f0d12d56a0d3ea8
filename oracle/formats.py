"""Element-format decoders (oracle; test infrastructure only).

The GEMM Optimization Guide names the input types in §6.2 (FP8, INT8, BF16,
FP16, FP4 on gfx950), the FP4 block-scale bytes in §8.2 and INT4 weights in
§8.2 (the W4A8 bytes formula). The pages do not spell the bit layouts out; the
readings used here are the open standards the gfx950 matrix cores implement:
  * FP8 is OCP E4M3FN (bias 7, no infinities, S.1111.111 is NaN, max 448);
  * FP4 is OCP MX E2M1 (bias 1, no NaN/Inf, max 6), two codes per byte with
    the even K index in the low nibble;
  * the MX block scale is E8M0 (2^(e-127), 0xFF is NaN);
  * BF16 is the upper half of an IEEE binary32;
  * FP16 is IEEE binary16 (bias 15, subnormals, infinities, NaN);
  * INT4 is a two's complement nibble (-8 .. 7), two per byte, the even K
    index in the low nibble (the same packing as FP4).
Each decoder evaluates its format's sign/exponent/mantissa fields directly,
in float64, so every value is exact.
"""
from __future__ import annotations

import numpy as np


def decode_int8(x: np.ndarray) -> np.ndarray:
    """Two's complement bytes -> int64."""
    return np.asarray(x).view(np.int8).astype(np.int64)


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64 (exact)."""
    u = np.asarray(bits).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return u.view(np.float32).astype(np.float64)


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    """FP8 E4M3FN codes (uint8) -> float64; NaN for 0x7F / 0xFF."""
    c = np.asarray(codes).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    subnormal = (m / 8.0) * np.exp2(1.0 - 7.0)
    v = sign * np.where(e == 0, subnormal, normal)
    return np.where((e == 15) & ((c & 0x7) == 7), np.nan, v)


def decode_e2m1(codes: np.ndarray) -> np.ndarray:
    """FP4 E2M1 codes (values 0..15) -> float64."""
    c = np.asarray(codes).astype(np.int64)
    sign = np.where(c & 0x8, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = (c & 0x1).astype(np.float64)
    normal = (1.0 + m / 2.0) * np.exp2(e.astype(np.float64) - 1.0)
    subnormal = (m / 2.0) * np.exp2(1.0 - 1.0)
    return sign * np.where(e == 0, subnormal, normal)


def decode_e8m0(codes: np.ndarray) -> np.ndarray:
    """E8M0 scale codes (uint8) -> float64 2^(code-127); NaN for 0xFF."""
    c = np.asarray(codes).astype(np.int64)
    return np.where(c == 255, np.nan, np.exp2(c.astype(np.float64) - 127.0))


def decode_f16(bits: np.ndarray) -> np.ndarray:
    """IEEE binary16 bit patterns (uint16) -> float64 (exact); inf / NaN kept."""
    c = np.asarray(bits).astype(np.int64)
    sign = np.where(c & 0x8000, -1.0, 1.0)
    e = (c >> 10) & 0x1F
    m = (c & 0x3FF).astype(np.float64)
    normal = (1.0 + m / 1024.0) * np.exp2(e.astype(np.float64) - 15.0)
    subnormal = (m / 1024.0) * np.exp2(1.0 - 15.0)
    v = np.where(e == 0, subnormal, normal)
    v = np.where(e == 31, np.where(m == 0, np.inf, np.nan), v)
    return sign * v


def decode_int4(codes: np.ndarray) -> np.ndarray:
    """INT4 codes (nibbles 0..15, two's complement) -> int64 in [-8, 7]."""
    c = np.asarray(codes).astype(np.int64) & 0xF
    return np.where(c >= 8, c - 16, c)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    """[R, K/2] bytes -> [R, K] 4-bit codes; element 2i is the low nibble of byte i."""
    p = np.asarray(packed).astype(np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


unpack_fp4 = unpack_nibbles
