"""CPU oracle for the preshuffle GEMM  C[M,N] = A[M,K] . B[N,K]^T.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this package: only the tests, the smoke check and the benchmark's
CPU-baseline leg do. It shares no code with the HIP library and imports
nothing from it.

It is the plain definition written out, slow and obviously correct:
  * decoders for INT8, INT4, BF16, FP16, FP8 E4M3FN, FP4 E2M1 and E8M0 from
    their bit definitions (formats.py);
  * the B preshuffle layout and its inverse as a byte permutation (layout.py),
    GEMM Optimization Guide §1.4 and §12.1, plus the nibble order of the INT4
    weight layout;
  * the GEMM as decode-then-multiply with exact int64 (INT8) or fp64
    accumulation (gemm.py), GEMM Optimization Guide §1.1 (problem statement)
    and §7.1 (per-row/per-column scales in the epilogue), §8.2 (MXFP4 block
    scale bytes, INT4 weights); the fused bias / activation epilogues of
    Kernel Tuning Guide §6;
  * the comparison metrics (compare.py);
  * the pages' planning formulas: MFMA counts, LDS budget, VGPR estimate,
    occupancy, FLOPs and bytes moved (formulas.py), GEMM Optimization Guide
    §1.2, §1.5, §2.4, §8.1-§8.2, §10, §14.

Every function is pinned by tests under tests/ that run without a GPU.
"""
from .formats import (decode_int8, decode_bf16, decode_e4m3, decode_e2m1,
                      decode_e8m0, decode_f16, decode_int4, unpack_fp4, unpack_nibbles)
from .layout import (preshuffle, unshuffle, preshuffle_index, repack_int4_pieces,
                     unpack_int4_pieces, preshuffle_int4, unshuffle_int4)
from .gemm import (gemm_int8, gemm_fp8, gemm_bf16, gemm_f16, gemm_mxfp4, gemm_w4a8, gemm,
                   activation, apply_epilogue, ACTS)
from .compare import compare_bf16, compare_f16, compare_values, bf16_rne, f16_rne, ELEM_TOL, NORMWISE_TOL

__all__ = [
    "decode_int8", "decode_bf16", "decode_e4m3", "decode_e2m1", "decode_e8m0",
    "decode_f16", "decode_int4", "unpack_fp4", "unpack_nibbles",
    "preshuffle", "unshuffle", "preshuffle_index", "repack_int4_pieces", "unpack_int4_pieces",
    "preshuffle_int4", "unshuffle_int4",
    "gemm_int8", "gemm_fp8", "gemm_bf16", "gemm_f16", "gemm_mxfp4", "gemm_w4a8", "gemm",
    "activation", "apply_epilogue", "ACTS",
    "compare_bf16", "compare_f16", "compare_values", "bf16_rne", "f16_rne", "ELEM_TOL", "NORMWISE_TOL",
]
