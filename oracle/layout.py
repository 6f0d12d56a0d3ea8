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
