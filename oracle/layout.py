"""B preshuffle layout (oracle; test infrastructure only).

GEMM Optimization Guide §1.4 and §12.1 store B (N rows, K-contiguous) as a
five-axis array [N/16][K/64][4][16][kpack_bytes] where the 16-axis is the 16
lanes of one MFMA column block and the 4-axis is the lane group of four that
each take a 16-byte (dwordx4) piece. The pages' kpack wording is
self-inconsistent; the reading that keeps the byte count equal to N*Kb is a
16-byte innermost pack and a K/64 axis that counts 64-BYTE blocks of K:

    Bs[n0][k0][g][j][b] = B[16*n0 + j][64*k0 + 16*g + b]

with Kb = K * element bytes (K/64 elements for INT8/FP8, K/32 for BF16, K/128
for packed FP4). The permutation acts on bytes, so it is the same for every
element type.
"""
from __future__ import annotations

import numpy as np


def preshuffle_index(n: int, kb: int, Kb: int) -> int:
    """Flat byte offset in the preshuffled buffer of byte B[n][kb]."""
    n0, j = divmod(n, 16)
    k0, r = divmod(kb, 64)
    g, b = divmod(r, 16)
    return (((n0 * (Kb // 64) + k0) * 4 + g) * 16 + j) * 16 + b


def preshuffle(b: np.ndarray) -> np.ndarray:
    """B as bytes [N, Kb] -> preshuffled flat bytes [N*Kb]."""
    bb = np.ascontiguousarray(b).view(np.uint8)
    N, Kb = bb.shape
    if N % 16 or Kb % 64:
        raise ValueError("preshuffle needs N % 16 == 0 and K bytes % 64 == 0")
    t = bb.reshape(N // 16, 16, Kb // 64, 4, 16)       # n0, j, k0, g, b
    return np.ascontiguousarray(t.transpose(0, 2, 3, 1, 4)).reshape(-1)


def unshuffle(bs: np.ndarray, N: int, Kb: int) -> np.ndarray:
    """Inverse of preshuffle: flat bytes -> [N, Kb] bytes."""
    t = np.ascontiguousarray(bs).view(np.uint8).reshape(N // 16, Kb // 64, 4, 16, 16)
    return np.ascontiguousarray(t.transpose(0, 3, 1, 2, 4)).reshape(N, Kb)


# INT4 weights (W4A8). The byte permutation above gives each lane 16 bytes =
# 32 consecutive K elements of one column. The int8 matrix instruction takes
# 16 K elements per lane, so a lane's 32 elements feed two instructions. The
# INT4 layout additionally reorders the nibbles inside every 16-byte piece so
# that its low nibbles hold elements 0..15 of the piece and its high nibbles
# elements 16..31 (element t in byte t % 16, nibble t // 16): each half then
# widens to 16 int8 values in K order with a mask and a shift per dword. The
# pages fix no INT4 nibble order; this one is the layout's own definition.

def repack_int4_pieces(b: np.ndarray) -> np.ndarray:
    """Row-major packed INT4 bytes [N, Kb] (element 2i in the low nibble of
    byte i) -> [N, Kb] bytes with every 16-byte piece reordered as above."""
    bb = np.ascontiguousarray(b).view(np.uint8)
    N, Kb = bb.shape
    if Kb % 16:
        raise ValueError("INT4 rows must be whole 16-byte pieces")
    nib = np.empty((N, Kb * 2), dtype=np.uint8)           # element order
    nib[:, 0::2] = bb & 0xF
    nib[:, 1::2] = bb >> 4
    t = nib.reshape(N, Kb // 16, 2, 16)                    # piece, half (t // 16), t % 16
    out = t[:, :, 0, :] | (t[:, :, 1, :] << 4)
    return np.ascontiguousarray(out.reshape(N, Kb))


def unpack_int4_pieces(r: np.ndarray) -> np.ndarray:
    """Inverse of repack_int4_pieces."""
    rr = np.ascontiguousarray(r).view(np.uint8)
    N, Kb = rr.shape
    t = rr.reshape(N, Kb // 16, 16)
    nib = np.stack([t & 0xF, t >> 4], axis=2).reshape(N, Kb * 2)   # element order
    return np.ascontiguousarray((nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8))


def preshuffle_int4(b: np.ndarray) -> np.ndarray:
    """Packed INT4 B [N, Kb] -> the W4A8 preshuffled flat bytes."""
    return preshuffle(repack_int4_pieces(b))


def unshuffle_int4(bs: np.ndarray, N: int, Kb: int) -> np.ndarray:
    return unpack_int4_pieces(unshuffle(bs, N, Kb))
