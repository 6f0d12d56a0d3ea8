"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

INT8 is bit-exact; FP8 / BF16 / MXFP4 with bf16 output are within
normwise 2e-3 and floored elementwise 1e-2 of the float64 oracle; the
closed-form cases (one-hot B, single products, exhaustive FP8 / FP4 codes,
block-scale placement) are bit-exact for every type.
"""
import numpy as np
import pytest

import oracle
import workloads
from tests._parity import check, gpu_run, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import dense_gemm_preshuffle_amd as gp

    gp.load_library()
    yield


EB = {"int8": 1, "fp8": 1, "bf16": 2, "mxfp4": 0.5, "fp16": 2, "w4a8": 0.5}


# ---------------------------------------------------------------- preshuffle
@pytest.mark.parametrize("dtype,N,K", [("int8", 16, 64), ("fp8", 48, 512), ("bf16", 64, 256),
                                       ("mxfp4", 32, 512), ("fp8", 7168, 2048), ("fp16", 32, 128),
                                       ("w4a8", 48, 512), ("w4a8", 7168, 2048)])
def test_preshuffle_bit_exact(dtype, N, K):
    import torch
    from dense_gemm_preshuffle_amd import gemm_preshuffle_b

    say(f"preshuffle {dtype} N={N} K={K}")
    Kb = int(K * EB[dtype])
    b = np.random.default_rng(N + K).integers(0, 256, size=(N, Kb), dtype=np.uint8)
    out = gemm_preshuffle_b(torch.from_numpy(b).cuda(), dtype)
    torch.cuda.synchronize()
    ref = oracle.preshuffle_int4(b) if dtype == "w4a8" else oracle.preshuffle(b)
    assert np.array_equal(out.cpu().numpy(), ref)


# ---------------------------------------------------------------- random parity over tile shapes
TILE_CASES = [
    # dtype, M, N, K, opts
    ("int8", 64, 128, 128, dict(kernel=1, tile_m=64, tile_n=64, tile_k=128)),      # 1 K tile
    ("int8", 128, 256, 256, dict(kernel=1, tile_m=64, tile_n=128, tile_k=128)),    # 2 K tiles
    ("int8", 128, 256, 384, dict(kernel=1, tile_m=128, tile_n=256, tile_k=128)),   # 3 K tiles (odd)
    ("int8", 64, 192, 640, dict(kernel=1, tile_m=32, tile_n=64, tile_k=128, epilogue=2)),
    ("int8", 32, 128, 512, dict(kernel=1, tile_m=16, tile_n=64, tile_k=256)),
    ("fp8", 128, 512, 384, dict(kernel=1, tile_m=64, tile_n=256, tile_k=128)),
    ("fp8", 128, 512, 640, dict(kernel=1, tile_m=128, tile_n=256, tile_k=128, epilogue=2)),
    ("fp8", 96, 256, 256, dict(kernel=1, tile_m=32, tile_n=256, tile_k=128)),
    ("fp8", 64, 256, 1536, dict(kernel=1, tile_m=16, tile_n=64, tile_k=512, epilogue=2)),
    ("fp8", 128, 256, 768, dict(kernel=1, tile_m=64, tile_n=256, tile_k=256)),
    ("bf16", 256, 512, 192, dict(kernel=1, tile_m=128, tile_n=256, tile_k=64)),
    ("bf16", 128, 512, 320, dict(kernel=1, tile_m=128, tile_n=256, tile_k=32, epilogue=2)),
    ("bf16", 128, 256, 192, dict(kernel=1, tile_m=64, tile_n=128, tile_k=64)),
    ("mxfp4", 128, 512, 768, dict(kernel=1, tile_m=64, tile_n=256, tile_k=256)),
    ("mxfp4", 256, 256, 512, dict(kernel=1, tile_m=128, tile_n=128, tile_k=256, epilogue=2)),
    ("mxfp4", 64, 256, 1024, dict(kernel=1, tile_m=32, tile_n=256, tile_k=256)),
    # 32x32 MFMA blocks (BF16, FP4, INT8)
    ("bf16", 128, 512, 192, dict(kernel=1, tile_m=128, tile_n=256, tile_k=64, mfma=32)),
    ("bf16", 128, 256, 320, dict(kernel=1, tile_m=128, tile_n=256, tile_k=32, mfma=32, epilogue=1)),
    ("bf16", 128, 256, 192, dict(kernel=1, tile_m=64, tile_n=128, tile_k=64, mfma=32, epilogue=2)),
    ("bf16", 256, 256, 128, dict(kernel=1, tile_m=128, tile_n=128, tile_k=64, mfma=32)),
    ("mxfp4", 128, 512, 768, dict(kernel=1, tile_m=128, tile_n=256, tile_k=256, mfma=32)),
    ("mxfp4", 128, 256, 512, dict(kernel=1, tile_m=64, tile_n=256, tile_k=256, mfma=32, epilogue=1)),
    ("mxfp4", 256, 256, 768, dict(kernel=1, tile_m=128, tile_n=128, tile_k=256, mfma=32)),
    # 128 x 512 tiles on 8 waves (each wave 128 x 64, one A tile for all eight)
    ("bf16", 256, 1024, 448, dict(kernel=1, tile_m=128, tile_n=512, tile_k=64, mfma=16, pipeline=3)),
    ("bf16", 128, 512, 320, dict(kernel=1, tile_m=128, tile_n=512, tile_k=64, mfma=32, pipeline=3)),
    ("bf16", 200, 608, 384, dict(kernel=1, tile_m=128, tile_n=512, tile_k=64, mfma=16, pipeline=2)),
    ("bf16", 128, 1024, 256, dict(kernel=1, tile_m=128, tile_n=512, tile_k=64, mfma=16, pipeline=3, epilogue=1)),
    ("fp16", 256, 512, 576, dict(kernel=1, tile_m=128, tile_n=512, tile_k=64, mfma=16, pipeline=3)),
    ("fp16", 144, 528, 320, dict(kernel=1, tile_m=128, tile_n=512, tile_k=64, mfma=32, pipeline=3)),
    ("fp8", 256, 1024, 640, dict(kernel=1, tile_m=128, tile_n=512, tile_k=128, pipeline=3)),
    ("mxfp4", 128, 1024, 4608, dict(kernel=1, tile_m=128, tile_n=512, tile_k=256, mfma=32, pipeline=2)),
    ("mxfp4", 256, 512, 2048, dict(kernel=1, tile_m=128, tile_n=512, tile_k=256, mfma=32, pipeline=1)),
    ("mxfp4", 160, 560, 1280, dict(kernel=1, tile_m=128, tile_n=512, tile_k=256, mfma=32, pipeline=2, epilogue=1)),
    # grouped FP4 scales with 16 x 16 blocks: odd row blocks inside the permuted 32-row scale blocks
    ("mxfp4", 128, 256, 2560, dict(kernel=1, tile_m=64, tile_n=256, tile_k=256, mfma=16)),
    ("mxfp4", 96, 512, 4096, dict(kernel=1, tile_m=32, tile_n=256, tile_k=256, mfma=16)),
    ("mxfp4", 128, 256, 2048, dict(kernel=1, tile_m=64, tile_n=128, tile_k=256, mfma=16, epilogue=2)),
    # 256 x 256 FP4 tiles (one workgroup per CU, accumulators in AGPRs), 2-stage DMA and VGPR-staged A
    ("mxfp4", 256, 512, 2304, dict(kernel=1, tile_m=256, tile_n=256, tile_k=256, mfma=32, pipeline=2)),
    ("mxfp4", 512, 256, 1024, dict(kernel=1, tile_m=256, tile_n=256, tile_k=256, mfma=32, pipeline=1)),
    ("mxfp4", 300, 272, 4352, dict(kernel=1, tile_m=256, tile_n=256, tile_k=256, mfma=32, pipeline=2, epilogue=1)),
    ("int8", 128, 256, 384, dict(kernel=1, tile_m=128, tile_n=256, tile_k=128, mfma=32)),
    ("int8", 128, 512, 256, dict(kernel=1, tile_m=64, tile_n=256, tile_k=128, mfma=32, epilogue=2)),
    # A by LDS DMA, 2 or 3 pipeline stages, K-tile counts 1..5
    ("int8", 128, 256, 768, dict(kernel=1, tile_m=64, tile_n=128, tile_k=256, pipeline=3)),
    ("int8", 128, 512, 384, dict(kernel=1, tile_m=64, tile_n=256, tile_k=128, pipeline=3, epilogue=2)),
    ("int8", 256, 512, 640, dict(kernel=1, tile_m=128, tile_n=256, tile_k=128, pipeline=3)),
    ("bf16", 128, 256, 64, dict(kernel=1, tile_m=128, tile_n=256, tile_k=64, mfma=32, pipeline=3)),
    ("bf16", 128, 256, 128, dict(kernel=1, tile_m=128, tile_n=256, tile_k=64, mfma=32, pipeline=3)),
    ("bf16", 256, 512, 192, dict(kernel=1, tile_m=128, tile_n=256, tile_k=64, mfma=32, pipeline=3)),
    ("bf16", 128, 256, 256, dict(kernel=1, tile_m=128, tile_n=256, tile_k=64, mfma=32, pipeline=3, epilogue=1)),
    ("bf16", 128, 256, 320, dict(kernel=1, tile_m=128, tile_n=256, tile_k=64, mfma=32, pipeline=3)),
    ("bf16", 128, 256, 320, dict(kernel=1, tile_m=128, tile_n=256, tile_k=64, mfma=16, pipeline=3)),
    ("bf16", 128, 256, 192, dict(kernel=1, tile_m=128, tile_n=256, tile_k=64, mfma=32, pipeline=2)),
    ("fp8", 128, 256, 128, dict(kernel=1, tile_m=128, tile_n=256, tile_k=128, pipeline=3)),
    ("fp8", 128, 512, 640, dict(kernel=1, tile_m=128, tile_n=256, tile_k=128, pipeline=3)),
    ("fp8", 128, 256, 256, dict(kernel=1, tile_m=128, tile_n=256, tile_k=128, pipeline=2)),
    ("fp8", 128, 256, 512, dict(kernel=1, tile_m=64, tile_n=256, tile_k=128, pipeline=3)),
    ("fp8", 64, 512, 384, dict(kernel=1, tile_m=32, tile_n=256, tile_k=128, pipeline=3)),
    ("fp8", 64, 256, 640, dict(kernel=1, tile_m=32, tile_n=128, tile_k=128, pipeline=3)),
    ("fp8", 96, 384, 768, dict(kernel=1, tile_m=32, tile_n=128, tile_k=256, pipeline=3)),
    ("fp8", 64, 512, 1280, dict(kernel=1, tile_m=32, tile_n=256, tile_k=256, pipeline=3)),
    # 4- and 6-stage pipelines, K-tile counts 1 .. 13 (prologue clamp, tails)
    ("fp8", 64, 256, 128, dict(kernel=1, tile_m=32, tile_n=256, tile_k=128, pipeline=6)),
    ("fp8", 64, 256, 384, dict(kernel=1, tile_m=32, tile_n=256, tile_k=128, pipeline=6)),
    ("fp8", 64, 512, 896, dict(kernel=1, tile_m=32, tile_n=256, tile_k=128, pipeline=6)),
    ("fp8", 32, 256, 1664, dict(kernel=1, tile_m=32, tile_n=256, tile_k=128, pipeline=4)),
    ("fp8", 96, 256, 768, dict(kernel=1, tile_m=32, tile_n=128, tile_k=256, pipeline=6)),
    ("fp8", 64, 384, 1280, dict(kernel=1, tile_m=32, tile_n=128, tile_k=256, pipeline=4)),
    ("fp8", 128, 512, 640, dict(kernel=1, tile_m=64, tile_n=256, tile_k=128, pipeline=4)),
    ("fp8", 128, 256, 768, dict(kernel=1, tile_m=64, tile_n=128, tile_k=256, pipeline=3)),            # 3 K tiles
    ("fp8", 64, 384, 2560, dict(kernel=1, tile_m=64, tile_n=128, tile_k=256, pipeline=3, epilogue=1)),  # 10 K tiles
    ("mxfp4", 128, 256, 256, dict(kernel=1, tile_m=128, tile_n=256, tile_k=256, mfma=32, pipeline=2)),
    ("mxfp4", 128, 512, 768, dict(kernel=1, tile_m=128, tile_n=256, tile_k=256, mfma=32, pipeline=2)),
    ("mxfp4", 128, 256, 1280, dict(kernel=1, tile_m=128, tile_n=256, tile_k=256, mfma=32, pipeline=2)),   # 5 K tiles: two scale groups, the second partial
    # 4-tile loop trips with a tail of 0-3 tiles after one or two trips
    ("mxfp4", 128, 256, 1536, dict(kernel=1, tile_m=128, tile_n=256, tile_k=256, mfma=32, pipeline=2)),   # 6 K tiles
    ("mxfp4", 128, 256, 1792, dict(kernel=1, tile_m=128, tile_n=256, tile_k=256, mfma=32, pipeline=2)),   # 7
    ("mxfp4", 128, 256, 2048, dict(kernel=1, tile_m=128, tile_n=256, tile_k=256, mfma=32, pipeline=2)),   # 8
    ("mxfp4", 128, 256, 2304, dict(kernel=1, tile_m=128, tile_n=256, tile_k=256, mfma=32, pipeline=2)),   # 9
    ("mxfp4", 64, 128, 2816, dict(kernel=1, tile_m=64, tile_n=128, tile_k=256)),                          # 11, 16 x 16 blocks
    # 256x256 tiles, one workgroup per CU (accumulators in AGPRs)
    ("bf16", 256, 512, 192, dict(kernel=1, tile_m=256, tile_n=256, tile_k=32, mfma=16, pipeline=3)),
    ("bf16", 512, 256, 224, dict(kernel=1, tile_m=256, tile_n=256, tile_k=32, mfma=16, pipeline=4)),
    ("bf16", 512, 256, 320, dict(kernel=1, tile_m=256, tile_n=256, tile_k=64, mfma=32, pipeline=3)),
    ("bf16", 256, 256, 64, dict(kernel=1, tile_m=256, tile_n=256, tile_k=64, mfma=32, pipeline=2, epilogue=1)),
    ("bf16", 256, 512, 160, dict(kernel=1, tile_m=256, tile_n=256, tile_k=32, mfma=32, pipeline=3)),
    # 512-byte K tiles (A rows of 512 bytes: each LDS-DMA instruction has its own source offsets)
    ("fp8", 256, 512, 2048, dict(kernel=1, tile_m=64, tile_n=128, tile_k=512, pipeline=3)),
    ("fp8", 200, 384, 1536, dict(kernel=1, tile_m=64, tile_n=128, tile_k=512, pipeline=2)),
    ("fp8", 64, 128, 512, dict(kernel=1, tile_m=64, tile_n=128, tile_k=512, pipeline=3, epilogue=1)),
    # 128 x 128 tiles with A by LDS DMA (128-byte K tiles); ragged M / N tails
    ("bf16", 256, 384, 576, dict(kernel=1, tile_m=128, tile_n=128, tile_k=64, mfma=16, pipeline=3)),
    ("bf16", 200, 144, 128, dict(kernel=1, tile_m=128, tile_n=128, tile_k=64, mfma=16, pipeline=3, epilogue=1)),
    ("fp16", 128, 256, 320, dict(kernel=1, tile_m=128, tile_n=128, tile_k=64, mfma=16, pipeline=3)),
    ("int8", 256, 256, 640, dict(kernel=1, tile_m=128, tile_n=128, tile_k=128, pipeline=3)),
    ("int8", 96, 208, 384, dict(kernel=1, tile_m=64, tile_n=128, tile_k=128, pipeline=3, epilogue=2)),
    ("mxfp4", 256, 256, 1280, dict(kernel=1, tile_m=128, tile_n=128, tile_k=256, mfma=32, pipeline=2)),
    ("mxfp4", 160, 144, 512, dict(kernel=1, tile_m=128, tile_n=128, tile_k=256, mfma=32, pipeline=2, epilogue=1)),
    # 256 x 256 tiles on 8 waves (each wave 32 columns of all 256 rows): 16 x 16 blocks with 128-byte K tiles
    ("bf16", 512, 512, 640, dict(kernel=1, tile_m=256, tile_n=256, tile_k=64, mfma=16, pipeline=3)),
    ("bf16", 300, 272, 384, dict(kernel=1, tile_m=256, tile_n=256, tile_k=64, mfma=16, pipeline=2)),
    ("bf16", 256, 256, 64, dict(kernel=1, tile_m=256, tile_n=256, tile_k=64, mfma=16, pipeline=3, epilogue=1)),
    ("fp16", 512, 256, 448, dict(kernel=1, tile_m=256, tile_n=256, tile_k=64, mfma=16, pipeline=3)),
    ("fp16", 260, 288, 128, dict(kernel=1, tile_m=256, tile_n=256, tile_k=64, mfma=16, pipeline=3, epilogue=1)),
    # wide kernel: 256x256 tiles, 8 waves, A and B through LDS; K-tile counts 1 .. 7
    ("bf16", 256, 256, 64, dict(kernel=3)),
    ("bf16", 512, 256, 320, dict(kernel=3)),
    ("bf16", 256, 512, 448, dict(kernel=3, mfma=32)),
    ("bf16", 256, 512, 160, dict(kernel=3, tile_k=32, pipeline=3)),
    ("bf16", 512, 256, 224, dict(kernel=3, tile_k=32, mfma=32, pipeline=4)),
    ("bf16", 256, 256, 96, dict(kernel=3, tile_k=32, pipeline=4)),
    ("fp8", 512, 512, 640, dict(kernel=3)),
    ("fp8", 256, 256, 128, dict(kernel=3)),
    ("int8", 256, 512, 384, dict(kernel=3)),
    ("int8", 512, 256, 256, dict(kernel=3, mfma=32)),
    # two K groups of 4 waves (waves=8): K-tile counts 2 .. 12 split in halves
    ("fp8", 128, 256, 1024, dict(kernel=1, tile_m=64, tile_n=128, tile_k=256, pipeline=3, waves=8)),
    ("fp8", 64, 384, 3072, dict(kernel=1, tile_m=64, tile_n=128, tile_k=256, pipeline=3, waves=8, epilogue=1)),
    ("fp8", 64, 512, 512, dict(kernel=1, tile_m=32, tile_n=256, tile_k=256, pipeline=3, waves=8)),
    ("fp8", 128, 512, 1536, dict(kernel=1, tile_m=64, tile_n=256, tile_k=128, pipeline=3, waves=8)),
    ("int8", 128, 256, 512, dict(kernel=1, tile_m=64, tile_n=128, tile_k=128, pipeline=0, waves=8)),
    ("bf16", 256, 512, 256, dict(kernel=1, tile_m=128, tile_n=256, tile_k=64, pipeline=3, waves=8)),
    ("bf16", 128, 256, 384, dict(kernel=1, tile_m=64, tile_n=128, tile_k=64, pipeline=0, waves=8)),
    # small-M split-K kernel
    ("fp8", 16, 512, 2048, dict(kernel=2)),
    ("fp8", 32, 256, 1024, dict(kernel=2, tile_n=32)),
    ("fp8", 16, 256, 2048, dict(kernel=2, waves=8, tile_k=256)),
    ("fp8", 16, 512, 2048, dict(kernel=2, tile_n=32, waves=8, tile_k=256)),
    ("fp8", 32, 256, 4096, dict(kernel=2, tile_n=64, waves=8, tile_k=256)),   # 2 chunks per wave
    ("fp8", 16, 128, 4096, dict(kernel=2, tile_k=128)),   # 8 chunks per wave
    ("fp8", 16, 128, 1536, dict(kernel=2, tile_k=128)),   # 3 chunks (odd)
    ("int8", 16, 64, 1024, dict(kernel=2)),
    ("bf16", 32, 128, 512, dict(kernel=2, tile_n=32)),
    ("mxfp4", 16, 128, 2048, dict(kernel=2)),
    # FP16 (fp16 output): tile, DMA pipeline, 32x32 blocks, split-K, wide
    ("fp16", 128, 256, 256, dict(kernel=1, tile_m=128, tile_n=256, tile_k=64)),
    ("fp16", 128, 512, 320, dict(kernel=1, tile_m=128, tile_n=256, tile_k=64, pipeline=3)),
    ("fp16", 128, 256, 192, dict(kernel=1, tile_m=128, tile_n=256, tile_k=64, mfma=32, pipeline=3)),
    ("fp16", 64, 256, 256, dict(kernel=1, tile_m=64, tile_n=128, tile_k=64, epilogue=1)),
    ("fp16", 32, 128, 512, dict(kernel=2, tile_n=32)),
    ("fp16", 512, 256, 320, dict(kernel=3)),
    # W4A8 (int8 A, INT4 B) on the small-M kernel
    ("w4a8", 16, 512, 2048, dict(kernel=2)),
    ("w4a8", 32, 256, 1024, dict(kernel=2, tile_n=16)),
    ("w4a8", 16, 256, 4096, dict(kernel=2, tile_n=32, waves=8, tile_k=256)),
    ("w4a8", 48, 128, 512, dict(kernel=2, tile_k=128)),
    ("w4a8", 16, 128, 4096, dict(kernel=2, tile_n=32, tile_k=128)),   # 4 chunks per wave
    # small-M kernel with 2 or 4 row blocks per workgroup (B read once per 2 or 4 row blocks)
    ("fp8", 32, 512, 2048, dict(kernel=2, tile_m=32)),
    ("fp8", 64, 256, 1024, dict(kernel=2, tile_m=64)),
    ("fp8", 48, 512, 2048, dict(kernel=2, tile_m=64)),
    ("bf16", 64, 256, 512, dict(kernel=2, tile_m=32)),
    ("int8", 64, 256, 2048, dict(kernel=2, tile_m=32)),
    ("mxfp4", 64, 256, 1024, dict(kernel=2, tile_m=32)),
    ("fp16", 32, 256, 512, dict(kernel=2, tile_m=32)),
    ("w4a8", 64, 256, 1024, dict(kernel=2, tile_m=32)),
    ("w4a8", 32, 512, 2048, dict(kernel=2, tile_m=32)),
    ("fp8", 64, 512, 2048, dict(kernel=2, tile_m=16)),
    ("fp8", 64, 512, 2048, dict(kernel=2, tile_m=32)),
    ("int8", 48, 256, 2048, dict(kernel=2, tile_m=64)),      # 4 row blocks on 8 waves, last one empty
    ("bf16", 64, 512, 4096, dict(kernel=2, tile_m=64)),
    ("w4a8", 40, 512, 2048, dict(kernel=2, tile_m=64)),
    # the planner's own row blocks (16 rows on few columns; 32 on 4096; 64 on 7168)
    ("fp8", 64, 1024, 2048, dict(kernel=2)),
    ("bf16", 40, 1024, 2048, dict(kernel=2)),
    ("int8", 64, 4096, 1024, dict(kernel=2)),
    ("mxfp4", 33, 1024, 7168, dict(kernel=2)),                # 128-byte chunks (7 per wave)
    ("w4a8", 64, 7168, 512, dict(kernel=2)),
    # 128-byte K chunks (K per wave an odd multiple of 128 bytes), explicit and the planner's
    ("bf16", 32, 256, 1280, dict(kernel=2, tile_k=64)),
    ("fp16", 48, 512, 1280, dict(kernel=2, tile_m=32, tile_k=64)),
    ("int8", 40, 256, 1536, dict(kernel=2, tile_n=32, tile_k=128)),
    ("bf16", 113, 1024, 1280, dict()),
    ("fp8", 32, 576, 4352, dict()),                         # one wave would be left: the tile planner
    # above 64 rows, small outputs: the planner's small-M plan (ragged last row blocks)
    ("w4a8", 200, 1024, 2048, dict()),
    ("mxfp4", 640, 256, 2048, dict()),
    ("int8", 130, 1024, 1024, dict()),
    ("bf16", 96, 2048, 1024, dict()),
    ("fp16", 257, 512, 2048, dict()),
    ("fp8", 100, 1024, 2048, dict()),
    # W4A8 on the tile kernel (tile_k in INT4 elements; A tiles twice the B bytes)
    ("w4a8", 128, 256, 512, dict(kernel=1, tile_m=64, tile_n=128, tile_k=128, pipeline=3)),
    ("w4a8", 256, 512, 1024, dict(kernel=1, tile_m=128, tile_n=256, tile_k=128)),
    ("w4a8", 128, 256, 768, dict(kernel=1, tile_m=64, tile_n=128, tile_k=256)),        # 3 K tiles
    ("w4a8", 64, 256, 384, dict(kernel=1, tile_m=32, tile_n=128, tile_k=128, epilogue=1)),
    ("w4a8", 64, 128, 512, dict(kernel=1, tile_m=32, tile_n=64, tile_k=128)),          # A through VGPRs
    ("w4a8", 256, 512, 640, dict(kernel=1, tile_m=64, tile_n=256, tile_k=128, epilogue=2)),
    ("w4a8", 128, 384, 128, dict(kernel=1, tile_m=64, tile_n=128, tile_k=128)),        # one K tile
]


@pytest.mark.parametrize("case", TILE_CASES, ids=lambda c: f"{c[0]}-{c[1]}x{c[2]}x{c[3]}-{c[4]}")
def test_random_parity(case):
    dtype, M, N, K, opts = case
    say(f"parity {dtype} {M}x{N}x{K} {opts}")
    host = workloads.make_inputs(dtype, M, N, K, seed=M * 7 + N * 3 + K)
    out = gpu_run(dtype, host, opts)
    check(dtype, host, out)


@pytest.mark.parametrize("xcd", [1, 2])
def test_xcd_order_does_not_change_result(xcd):
    say(f"xcd {xcd}")
    host = workloads.make_inputs("fp8", 512, 1024, 256, seed=11)
    opts = dict(kernel=1, tile_m=64, tile_n=256, tile_k=128, xcd_swizzle=xcd)
    out = gpu_run("fp8", host, opts)
    check("fp8", host, out)


# ---------------------------------------------------------------- M / N not multiples of the tile
RAGGED_CASES = [
    # edge tiles overlap their neighbours; split-K takes partial 16-row blocks
    ("bf16", 100, 272, 256, dict(kernel=1, tile_m=64, tile_n=128, tile_k=64)),
    ("bf16", 200, 400, 192, dict(kernel=1, tile_m=128, tile_n=256, tile_k=64, pipeline=3)),
    ("bf16", 130, 304, 128, dict(kernel=1, tile_m=128, tile_n=256, tile_k=64, mfma=32, epilogue=1)),
    ("fp8", 77, 336, 512, dict(kernel=1, tile_m=32, tile_n=256, tile_k=128, pipeline=3)),
    ("fp8", 150, 528, 384, dict(kernel=1, tile_m=64, tile_n=256, tile_k=128, epilogue=2)),
    ("fp8", 100, 208, 512, dict(kernel=1, tile_m=64, tile_n=128, tile_k=256, pipeline=3)),
    ("int8", 90, 208, 256, dict(kernel=1, tile_m=64, tile_n=128, tile_k=128)),
    ("int8", 33, 80, 256, dict(kernel=1, tile_m=32, tile_n=64, tile_k=128)),
    ("mxfp4", 160, 288, 512, dict(kernel=1, tile_m=128, tile_n=256, tile_k=256, mfma=32)),
    ("fp16", 70, 144, 256, dict(kernel=1, tile_m=64, tile_n=128, tile_k=64)),
    ("bf16", 300, 272, 128, dict(kernel=3)),
    ("fp8", 100, 208, 1024, dict(kernel=1, tile_m=64, tile_n=128, tile_k=256, pipeline=3, waves=8)),
    ("bf16", 200, 400, 256, dict(kernel=1, tile_m=128, tile_n=256, tile_k=64, pipeline=3, waves=8)),
    ("fp8", 1, 512, 2048, dict(kernel=2)),
    ("fp8", 5, 256, 1024, dict(kernel=2, tile_n=16)),
    ("bf16", 17, 128, 512, dict(kernel=2)),
    ("int8", 29, 64, 1024, dict(kernel=2)),
    ("mxfp4", 7, 128, 2048, dict(kernel=2)),
    ("w4a8", 3, 256, 2048, dict(kernel=2)),
    ("fp8", 20, 256, 1024, dict(kernel=2)),       # two row blocks, the second partial
    ("fp8", 100, 512, 2048, dict(kernel=2)),      # two row blocks per workgroup, 4 workgroup rows, last partial
    ("bf16", 50, 128, 512, dict(kernel=2)),
    ("mxfp4", 40, 128, 2048, dict(kernel=2)),
    ("w4a8", 77, 256, 2048, dict(kernel=2)),
    ("w4a8", 150, 400, 512, dict(kernel=1, tile_m=64, tile_n=128, tile_k=128)),
    ("w4a8", 100, 208, 1024, None),        # planner's choice: the tile kernel with edge tiles
    ("fp8", 200, 48, 1024, None),          # no tile fits 48 columns: the planner takes split-K
    # K a multiple of one 64-byte block but not of the larger K tiles: 64-byte
    # K tiles (planner's choice, and named)
    ("int8", 128, 256, 320, None),
    ("fp16", 128, 256, 160, None),
    ("mxfp4", 128, 256, 384, None),
    ("int8", 100, 208, 448, None),
    ("mxfp4", 256, 512, 384, dict(kernel=1, tile_m=128, tile_n=256, tile_k=128, mfma=16)),
    ("fp16", 256, 512, 96, dict(kernel=1, tile_m=128, tile_n=256, tile_k=32)),
    ("int8", 256, 512, 192, dict(kernel=1, tile_m=128, tile_n=256, tile_k=64)),
    # degenerate: one 16-column block, the shortest K of each type (one wave,
    # one chunk). bf16 outputs keep >= 256 elements: the normwise bound of
    # 2e-3 sits just above the RMS of bf16 rounding alone (about 1.7e-3), so
    # a handful of outputs can cross it with an exact accumulator.
    ("int8", 1, 16, 64, None),
    ("int8", 16, 16, 64, None),
    ("fp8", 16, 16, 128, None),
    ("fp8", 300, 16, 256, None),
    ("bf16", 16, 16, 32, None),
    ("bf16", 1000, 16, 64, None),
    ("fp16", 3, 16, 32, None),
    ("mxfp4", 16, 16, 128, None),
    ("w4a8", 16, 16, 128, None),
    ("bf16", 33, 48, 96, None),
    ("bf16", 100, 272, 256, None),         # planner's own choice
]


@pytest.mark.parametrize("case", RAGGED_CASES, ids=lambda c: f"{c[0]}-{c[1]}x{c[2]}x{c[3]}-{c[4]}")
def test_ragged_parity(case):
    dtype, M, N, K, opts = case
    say(f"ragged {dtype} {M}x{N}x{K} {opts}")
    host = workloads.make_inputs(dtype, M, N, K, seed=M + N + K)
    out = gpu_run(dtype, host, opts)
    check(dtype, host, out)


# ---------------------------------------------------------------- fused epilogues
EPI_CASES = [
    ("fp8", 16, 512, 2048, dict(kernel=2)),
    ("fp8", 128, 512, 640, dict(kernel=1, tile_m=128, tile_n=256, tile_k=128, pipeline=3, epilogue=2)),
    ("fp8", 96, 256, 256, dict(kernel=1, tile_m=32, tile_n=256, tile_k=128, epilogue=1)),
    ("bf16", 256, 512, 192, dict(kernel=1, tile_m=128, tile_n=256, tile_k=64, pipeline=3)),
    ("bf16", 128, 256, 128, dict(kernel=1, tile_m=128, tile_n=256, tile_k=64, mfma=32, epilogue=1)),
    ("mxfp4", 128, 256, 512, dict(kernel=1, tile_m=128, tile_n=256, tile_k=256, mfma=32, pipeline=2)),
    ("mxfp4", 128, 256, 2560, dict(kernel=1, tile_m=128, tile_n=256, tile_k=256, mfma=32, pipeline=2)),  # 3 scale groups
    ("mxfp4", 16, 128, 2048, dict(kernel=2)),
    ("fp16", 128, 256, 256, dict(kernel=1, tile_m=128, tile_n=256, tile_k=64)),
    ("bf16", 512, 256, 320, dict(kernel=3)),
    ("fp8", 512, 512, 640, dict(kernel=3)),
    ("w4a8", 16, 512, 2048, dict(kernel=2)),
    ("fp8", 48, 512, 2048, dict(kernel=2)),      # row blocks: per-row scales of each block
    ("w4a8", 64, 256, 1024, dict(kernel=2)),
    ("bf16", 100, 272, 256, dict(kernel=1, tile_m=64, tile_n=128, tile_k=64)),   # with edge tiles
    ("fp8", 100, 208, 1024, dict(kernel=1, tile_m=64, tile_n=128, tile_k=256, pipeline=3, waves=8)),
    ("bf16", 128, 256, 256, dict(kernel=1, tile_m=64, tile_n=128, tile_k=64, pipeline=0, waves=8)),
    ("w4a8", 128, 256, 512, dict(kernel=1, tile_m=64, tile_n=128, tile_k=128)),
    ("w4a8", 150, 400, 512, dict(kernel=1, tile_m=64, tile_n=128, tile_k=128, epilogue=1)),
    ("bf16", 96, 1024, 2048, dict()),                                # the planner's small-M plan above 64 rows
    ("w4a8", 130, 512, 4096, dict()),
]


@pytest.mark.parametrize("act", ["none", "relu", "silu", "gelu"])
@pytest.mark.parametrize("case", EPI_CASES, ids=lambda c: f"{c[0]}-{c[1]}x{c[2]}x{c[3]}-k{c[4].get('kernel', 0)}")
def test_fused_epilogue_parity(case, act):
    dtype, M, N, K, opts = case
    say(f"epilogue {act} {dtype} {M}x{N}x{K} {opts}")
    host = workloads.make_inputs(dtype, M, N, K, seed=M + 3 * N + K, bias=True)
    out = gpu_run(dtype, host, opts, act=act)
    check(dtype, host, out, act=act)


def test_activation_without_bias_and_int8_refused():
    say("epilogue without bias")
    host = workloads.make_inputs("fp8", 128, 256, 256, seed=41)
    out = gpu_run("fp8", host, dict(kernel=1, tile_m=64, tile_n=256, tile_k=128), act="gelu")
    check("fp8", host, out, act="gelu")
    out = gpu_run("bf16", workloads.make_inputs("bf16", 16, 256, 1024, seed=42), dict(kernel=2), act="silu")
    check("bf16", workloads.make_inputs("bf16", 16, 256, 1024, seed=42), out, act="silu")
    import dense_gemm_preshuffle_amd as gp
    with pytest.raises(gp.GemmError):
        gpu_run("int8", workloads.make_inputs("int8", 64, 128, 128, seed=1), act="relu")


# ---------------------------------------------------------------- closed forms (bit-exact)
def _one_hot_b(dtype, N, K, perm):
    """B[n, k] = 1.0 at k = perm[n], else 0, in the input encoding."""
    if dtype == "int8":
        b = np.zeros((N, K), np.int8)
        b[np.arange(N), perm] = 1
        return {"b": b}
    if dtype == "fp8":
        b = np.zeros((N, K), np.uint8)
        b[np.arange(N), perm] = 0x38
        return {"b": b, "scale_b": np.ones(N, np.float32)}
    if dtype == "bf16":
        b = np.zeros((N, K), np.uint16)
        b[np.arange(N), perm] = 0x3F80
        return {"b": b}
    if dtype == "fp16":
        b = np.zeros((N, K), np.uint16)
        b[np.arange(N), perm] = 0x3C00
        return {"b": b}
    if dtype == "w4a8":
        codes = np.zeros((N, K), np.uint8)
        codes[np.arange(N), perm] = 1            # INT4 1
        return {"b": codes[:, 0::2] | (codes[:, 1::2] << 4), "scale_b": np.exp2(np.arange(N) % 3 - 1).astype(np.float32)}
    codes = np.zeros((N, K), np.uint8)
    codes[np.arange(N), perm] = 2            # E2M1 1.0
    return {"b": codes[:, 0::2] | (codes[:, 1::2] << 4), "scale_b": np.full((N, K // 32), 127, np.uint8)}


PERM_CASES = [("int8", 128, 256, 256, dict(kernel=1, tile_m=64, tile_n=256, tile_k=128)),
              ("int8", 128, 256, 256, dict(kernel=1, tile_m=128, tile_n=256, tile_k=128, mfma=32)),
              ("bf16", 128, 256, 128, dict(kernel=1, tile_m=128, tile_n=256, tile_k=64, mfma=32)),
              ("bf16", 128, 256, 320, dict(kernel=1, tile_m=128, tile_n=256, tile_k=64, mfma=32, pipeline=3)),
              ("fp8", 128, 256, 640, dict(kernel=1, tile_m=128, tile_n=256, tile_k=128, pipeline=3)),
              ("mxfp4", 128, 256, 512, dict(kernel=1, tile_m=128, tile_n=256, tile_k=256, mfma=32)),
              ("fp8", 128, 512, 384, dict(kernel=1, tile_m=64, tile_n=256, tile_k=128)),
              ("fp8", 16, 256, 1024, dict(kernel=2)),
              ("bf16", 256, 256, 128, dict(kernel=1, tile_m=128, tile_n=256, tile_k=64)),
              ("mxfp4", 128, 256, 512, dict(kernel=1, tile_m=64, tile_n=256, tile_k=256)),
              ("mxfp4", 16, 128, 1024, dict(kernel=2)),
              ("fp16", 128, 256, 320, dict(kernel=1, tile_m=128, tile_n=256, tile_k=64, pipeline=3)),
              ("fp16", 128, 256, 128, dict(kernel=1, tile_m=128, tile_n=256, tile_k=64, mfma=32, pipeline=3)),
              ("w4a8", 16, 256, 2048, dict(kernel=2)),
              ("w4a8", 32, 512, 1024, dict(kernel=2, tile_n=16, tile_k=128)),
              ("w4a8", 128, 256, 768, dict(kernel=1, tile_m=64, tile_n=128, tile_k=256)),
              ("w4a8", 128, 512, 512, dict(kernel=1, tile_m=128, tile_n=256, tile_k=128))]


@pytest.mark.parametrize("case", PERM_CASES, ids=lambda c: f"{c[0]}-{c[1]}x{c[2]}x{c[3]}-k{c[4].get('kernel', 0)}")
def test_permutation_b_bit_exact(case):
    dtype, M, N, K, opts = case
    say(f"perm {dtype} {M}x{N}x{K}")
    rng = np.random.default_rng(3)
    host = workloads.make_inputs(dtype, M, N, K, seed=5)
    perm = rng.integers(0, K, size=N)
    host.update(_one_hot_b(dtype, N, K, perm))
    if dtype in ("fp8", "w4a8"):
        host["scale_a"] = np.exp2(rng.integers(-3, 4, size=M)).astype(np.float32)
    out = gpu_run(dtype, host, opts)
    ref = oracle.gemm(dtype, host)
    if dtype == "int8":
        assert np.array_equal(out, ref)
    else:
        dec = oracle.decode_f16 if dtype == "fp16" else oracle.decode_bf16
        assert np.array_equal(dec(out), ref), "one-hot B must select columns exactly"


def test_fp8_exhaustive_code_pairs_bit_exact():
    say("fp8 exhaustive codes")
    M = N = 256
    K = 128
    codes = np.arange(256, dtype=np.uint8)
    codes[[0x7F, 0xFF]] = 0
    a = np.zeros((M, K), np.uint8)
    b = np.zeros((N, K), np.uint8)
    a[:, 0] = codes
    b[:, 0] = codes
    host = {"a": a, "b": b, "scale_a": np.ones(M, np.float32), "scale_b": np.ones(N, np.float32)}
    for opts in (dict(kernel=1, tile_m=64, tile_n=256, tile_k=128), dict(kernel=1, tile_m=128, tile_n=128, tile_k=128, epilogue=2)):
        out = gpu_run("fp8", host, opts)
        assert np.array_equal(oracle.decode_bf16(out), oracle.gemm("fp8", host)), opts


def test_bf16_single_products_round_to_nearest_even():
    say("bf16 single products")
    rng = np.random.default_rng(9)
    M, N, K = 128, 256, 64
    a = np.zeros((M, K), np.uint16)
    b = np.zeros((N, K), np.uint16)
    a[:, 5] = (rng.integers(0, 2 ** 16, M).astype(np.uint16) & 0x3FFF) | 0x3C00
    b[:, 5] = (rng.integers(0, 2 ** 16, N).astype(np.uint16) & 0xBFFF) | 0x3800
    host = {"a": a, "b": b}
    for opts in (dict(kernel=1, tile_m=128, tile_n=256, tile_k=32, mfma=16),
                 dict(kernel=1, tile_m=128, tile_n=256, tile_k=32, mfma=32)):
        out = gpu_run("bf16", host, opts)
        assert np.array_equal(oracle.decode_bf16(out), oracle.bf16_rne(oracle.gemm("bf16", host))), opts


def test_fp4_exhaustive_codes_and_scales_bit_exact():
    say("fp4 exhaustive codes")
    M = N = 16
    K = 512
    ca = np.zeros((M, K), np.uint8)
    cb = np.zeros((N, K), np.uint8)
    ca[:, 0] = np.arange(16)
    cb[:, 0] = np.arange(16)
    sa = np.full((M, K // 32), 127, np.uint8)
    sb = np.full((N, K // 32), 127, np.uint8)
    sa[:, 0] = 127 + (np.arange(M) % 5) - 2
    sb[:, 0] = 127 + (np.arange(N) % 3) - 1
    host = {"a": ca[:, 0::2] | (ca[:, 1::2] << 4), "scale_a": sa,
            "b": cb[:, 0::2] | (cb[:, 1::2] << 4), "scale_b": sb}
    out = gpu_run("mxfp4", host, dict(kernel=2))
    assert np.array_equal(oracle.decode_bf16(out), oracle.gemm("mxfp4", host))


FP4_PLACEMENT_OPTS = [dict(kernel=1, tile_m=64, tile_n=256, tile_k=256, mfma=16),
                      dict(kernel=1, tile_m=32, tile_n=256, tile_k=256, mfma=16),
                      dict(kernel=1, tile_m=128, tile_n=256, tile_k=256, mfma=32),
                      dict(kernel=1, tile_m=64, tile_n=128, tile_k=256, mfma=32),
                      dict(kernel=1, tile_m=128, tile_n=256, tile_k=256, mfma=32, pipeline=2),
                      dict(kernel=2)]


@pytest.mark.parametrize("opts", FP4_PLACEMENT_OPTS, ids=["t64", "t32", "t128m32", "t64x128m32", "t128m32dma", "splitk"])
def test_fp4_block_scale_placement_bit_exact(opts):
    say(f"fp4 scale placement {opts}")
    rng = np.random.default_rng(4)
    # tile kernel: 16 K tiles, so the marked blocks spread over two or four scale groups
    M, N, K = (128, 256, 4096) if opts["kernel"] == 1 else (16, 64, 1024)
    nblk = K // 32
    blk = rng.integers(0, nblk, size=M)                  # row m is 1.0 on block blk[m] only
    ca = np.zeros((M, K), np.uint8)
    for m in range(M):
        ca[m, blk[m] * 32:(blk[m] + 1) * 32] = 2
    sa = rng.integers(120, 134, size=(M, nblk)).astype(np.uint8)
    cb = np.full((N, K), 2, np.uint8)                     # B all ones
    sb = np.full((N, nblk), 127, np.uint8)
    sb[:, :] = 127 + (np.arange(N)[:, None] % 3)          # per-row power of two
    host = {"a": ca[:, 0::2] | (ca[:, 1::2] << 4), "scale_a": sa,
            "b": cb[:, 0::2] | (cb[:, 1::2] << 4), "scale_b": sb}
    out = gpu_run("mxfp4", host, opts)
    ref = oracle.gemm("mxfp4", host)
    assert np.array_equal(oracle.decode_bf16(out), ref)


def test_fp16_single_products_round_to_nearest_even():
    say("fp16 single products")
    rng = np.random.default_rng(10)
    M, N, K = 128, 256, 64
    a = np.zeros((M, K), np.uint16)
    b = np.zeros((N, K), np.uint16)
    a[:, 9] = (rng.integers(0, 2 ** 16, M).astype(np.uint16) & 0x83FF) | 0x3800     # [0.5, 1) and negatives
    b[:, 9] = (rng.integers(0, 2 ** 16, N).astype(np.uint16) & 0x83FF) | 0x3C00     # [1, 2)
    host = {"a": a, "b": b}
    for opts in (dict(kernel=1, tile_m=128, tile_n=256, tile_k=64, mfma=16),
                 dict(kernel=1, tile_m=128, tile_n=256, tile_k=64, mfma=32, pipeline=3), dict(kernel=3)):
        if opts.get("kernel") == 3:
            host3 = {"a": np.zeros((256, K), np.uint16), "b": np.zeros((256, K), np.uint16)}
            host3["a"][:128] = a
            host3["b"][:] = b
            out = gpu_run("fp16", host3, opts)
            ref = oracle.gemm("fp16", host3)
        else:
            out = gpu_run("fp16", host, opts)
            ref = oracle.gemm("fp16", host)
        assert np.array_equal(oracle.decode_f16(out), oracle.f16_rne(ref)), opts


# ---------------------------------------------------------------- determinism
def test_bitwise_repeatable():
    say("repeatability")
    host = workloads.make_inputs("fp8", 16, 1024, 2048, seed=21)
    o1, o2 = gpu_run("fp8", host, None, repeat=2)
    assert np.array_equal(o1, o2)
    host = workloads.make_inputs("bf16", 256, 512, 512, seed=22)
    o1, o2 = gpu_run("bf16", host, None, repeat=2)
    assert np.array_equal(o1, o2)


@pytest.mark.parametrize("dtype,M,N,K,act", [("fp8", 16, 7168, 2048, None), ("w4a8", 16, 7168, 2048, "gelu"),
                                            ("bf16", 512, 512, 1024, None), ("mxfp4", 256, 512, 4096, None),
                                            ("fp8", 512, 1024, 1024, "silu"), ("fp16", 300, 272, 512, None),
                                            ("w4a8", 512, 1024, 1024, "relu"), ("int8", 512, 1024, 1024, None),
                                            ("bf16", 1000, 16, 64, None)])
def test_bitwise_repeatable_20_runs(dtype, M, N, K, act):
    """Twenty launches on the same inputs give bitwise-identical outputs: no
    atomics, a fixed reduction order in every kernel."""
    import torch

    from dense_gemm_preshuffle_amd import workload

    say(f"repeat x20 {dtype} {M}x{N}x{K} {act}")
    host = workloads.make_inputs(dtype, M, N, K, seed=51, bias=act is not None)
    p = workload.prepare(dtype, workload.to_device(dtype, host))
    outs = [workload.run(dtype, p, act=act) for _ in range(20)]
    torch.cuda.synchronize()
    first = workload.to_host(outs[0])
    for o in outs[1:]:
        assert np.array_equal(workload.to_host(o), first)


# ---------------------------------------------------------------- HIP graph replay
def test_graph_replay_matches_eager():
    """Launches captured in a HIP graph give the eager result on every replay,
    with eager work and synchronizations between the replays."""
    import torch

    from dense_gemm_preshuffle_amd import workload

    say("graph replay")
    for dtype, M, N, K in [("fp8", 16, 7168, 2048), ("bf16", 256, 512, 256), ("mxfp4", 128, 256, 4608),
                           ("w4a8", 256, 512, 1024), ("int8", 16, 16, 64)]:
        host = workloads.make_inputs(dtype, M, N, K, seed=31)
        p = workload.prepare(dtype, workload.to_device(dtype, host))
        eager = workload.to_host(workload.run(dtype, p))
        outs = [workload.run(dtype, p) for _ in range(3)]
        torch.cuda.synchronize()
        for o in outs:
            o.zero_()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for o in outs:
                workload.run(dtype, p, c=o)
        for rep in range(3):
            for o in outs:
                o.zero_()
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for o in outs:
                assert np.array_equal(workload.to_host(o), eager), (dtype, rep)
            workload.run(dtype, p)          # eager work between replays
            torch.cuda.synchronize()
