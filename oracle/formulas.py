"""The pages' planning and roofline formulas (oracle; test infrastructure only).

GEMM Optimization Guide:
  §1.2  derived tile parameters m_repeat, n_per_wave, num_acc_n, k_unroll;
  §1.5  MFMA count per tile, k_unroll * m_repeat * num_acc_n * 2 (the factor 2
        is two K32 instructions per 64-byte K step on gfx942);
  §2.4  LDS budget, 2 * tile_m * tile_k * elem_bytes (+ tile_m * tile_n * 2
        with a CShuffle epilogue);
  §8.1  flops = 2MNK;  §8.2 bytes moved per input type;
  §10.1 VGPR estimate;  §10.2 occupancy min(8, 512 // alignTo(vgprs, 8));
  §14   the worked 5120 x 5120 x 8320 FP8 example.

gfx950 instruction counts: the gfx950 matrix cores take 64 K-bytes per
16x16 instruction for INT8 (16x16x64), BF16 (16x16x32) and FP4 (16x16x128 at
half a byte), and 128 K-bytes for FP8 (16x16x128); the 32x32 forms take half
the K (32x32x32 INT8, 32x32x16 BF16, 32x32x64 FP8/FP4). Whatever the
instruction, the count of ms x ms x K_instr instructions for a whole problem
is (M/ms)(N/ms)(K/K_instr) and each does 2*ms*ms*K_instr flops, which must add
up to 2MNK.
"""
from __future__ import annotations

ELEM_BYTES = {"int8": 1.0, "fp8": 1.0, "bf16": 2.0, "fp16": 2.0, "mxfp4": 0.5, "int4": 0.5}
# K elements per gfx950 instruction; W4A8 widens INT4 to int8 and runs the int8 ones
K_INSTR_GFX950 = {"int8": 64, "fp8": 128, "bf16": 32, "fp16": 32, "mxfp4": 128, "w4a8": 64}   # 16x16 blocks
K_INSTR_GFX950_32 = {"int8": 32, "fp8": 64, "bf16": 16, "fp16": 16, "mxfp4": 64, "w4a8": 32}  # 32x32 blocks


def derived(tile_m: int, tile_n: int, tile_k: int, elem_bytes: float = 1.0) -> dict:
    """§1.2: m_repeat, n_per_wave, num_acc_n, k_unroll (64-byte K steps per tile)."""
    tile_k_bytes = int(tile_k * elem_bytes)
    return {
        "m_repeat": tile_m // 16,
        "n_per_wave": tile_n // 4,
        "num_acc_n": tile_n // 4 // 16,
        "k_unroll": tile_k_bytes // 64,
    }


def mfma_per_tile_pages(tile_m: int, tile_n: int, tile_k: int, elem_bytes: float = 1.0) -> int:
    """§1.5 with the gfx942 K32 instruction: two instructions per 64-byte K step."""
    d = derived(tile_m, tile_n, tile_k, elem_bytes)
    return d["k_unroll"] * d["m_repeat"] * d["num_acc_n"] * 2


def mfma_total_pages(K: int, tile_m: int, tile_n: int, tile_k: int, elem_bytes: float = 1.0) -> int:
    """§14 step 2: MFMAs per tile times the number of K tiles."""
    return mfma_per_tile_pages(tile_m, tile_n, tile_k, elem_bytes) * (K // tile_k)


def grid(M: int, N: int, tile_m: int, tile_n: int) -> int:
    return (M // tile_m) * (N // tile_n)


def lds_bytes(tile_m: int, tile_n: int, tile_k: int, elem_bytes: float, cshuffle: bool = False) -> int:
    """§2.4: double-buffered A tile (+ bf16 C tile for CShuffle)."""
    b = 2 * int(tile_m * tile_k * elem_bytes)
    if cshuffle:
        b += tile_m * tile_n * 2
    return b


def vgpr_estimate(tile_m: int, tile_n: int, tile_k: int, elem_bytes: float, num_a_loads: int) -> dict:
    """§10.1 estimate (FP8 sync copy): accumulators, B tile, A prefetch, A tile regs."""
    d = derived(tile_m, tile_n, tile_k, elem_bytes)
    return {
        "accumulators": d["m_repeat"] * d["num_acc_n"] * 4,
        "b_tile": d["k_unroll"] * 2 * d["num_acc_n"] * 2,
        "a_prefetch": 2 * 2,
        "a_tile": num_a_loads * 4,
    }


def occupancy(total_vgprs: int) -> int:
    """§10.2: waves per SIMD from the combined arch+accum VGPR count (granule 8)."""
    aligned = (total_vgprs + 7) // 8 * 8
    if aligned > 512:
        return 0
    return min(8, 512 // aligned)


def flops(M: int, N: int, K: int) -> int:
    """§8.1."""
    return 2 * M * N * K


def bytes_moved(dtype: str, M: int, N: int, K: int, out_bytes: int = 2) -> int:
    """§8.2 per input type. FP8/INT8 carry fp32 per-token scales; MXFP4 carries
    one scale byte per 32 K elements of every row of A and B. `out_bytes` is 2
    for a bf16 C and 4 for an int32 C (the INT8 path); INT8 has no scales."""
    if dtype == "fp8":
        return M * K + N * K + M * N * out_bytes + (M + N) * 4
    if dtype == "int8":
        return M * K + N * K + M * N * out_bytes
    if dtype in ("int4", "w4a8"):
        return M * K + (N * K) // 2 + M * N * out_bytes + (M + N) * 4
    if dtype == "mxfp4":
        return (M * K) // 2 + (N * K) // 2 + M * N * out_bytes + (M + N) * (K // 32)
    if dtype in ("bf16", "fp16"):
        return 2 * M * K + 2 * N * K + M * N * out_bytes
    raise ValueError(dtype)


def _k_instr(dtype: str, ms: int) -> int:
    return K_INSTR_GFX950[dtype] if ms == 16 else K_INSTR_GFX950_32[dtype]


def mfma_count_gfx950(dtype: str, M: int, N: int, K: int, ms: int = 16) -> int:
    """Number of ms x ms x K_instr gfx950 MFMA instructions for the whole problem."""
    return (M // ms) * (N // ms) * (K // _k_instr(dtype, ms))


def flops_per_mfma_gfx950(dtype: str, ms: int = 16) -> int:
    return 2 * ms * ms * _k_instr(dtype, ms)
