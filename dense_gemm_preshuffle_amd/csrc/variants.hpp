// Compiled kernel variants. The host planner and the launch tables both read
// these lists, so a tile the planner may pick is always instantiated.
//
// Tile kernel: X(dtype, mfma, tile_m, tile_n, tile_k_bytes, pipe): mfma = 16 or
// 32 (the MFMA block); pipe 0 = A staged through VGPRs (2 stages), 2 / 3 = A
// by LDS DMA with 2 / 3 stages. Each is built with the direct and the
// CShuffle epilogue. tile_n = 512 runs on 8 waves (64 columns each).
// Small-M (split-K) kernel: Y(dtype, n_blocks_of_16, waves,
// chunk_bytes_per_wave, m_blocks_of_16); W4A8 chunk bytes count bytes of B.
// Wide kernel (256x256 tiles, 8 waves): W(dtype, mfma, tile_k_bytes, pipe),
// pipe = LDS DMA stages of A and B.
#pragma once

#define GP_TILE_I8(X)                                                                              \
  X(DT_I8, 16, 16, 64, 256, 0) X(DT_I8, 16, 32, 64, 128, 0) X(DT_I8, 16, 64, 64, 128, 0)                     \
  X(DT_I8, 16, 64, 128, 128, 0) X(DT_I8, 16, 64, 256, 128, 0) X(DT_I8, 16, 128, 128, 128, 0)                 \
  X(DT_I8, 16, 128, 256, 128, 0) X(DT_I8, 32, 128, 256, 128, 0) X(DT_I8, 32, 64, 256, 128, 0)              \
  X(DT_I8, 16, 64, 128, 256, 3) X(DT_I8, 16, 64, 256, 128, 3) X(DT_I8, 16, 128, 256, 128, 3)              \
  X(DT_I8, 16, 64, 128, 64, 3) X(DT_I8, 16, 128, 256, 64, 3) X(DT_I8, 16, 128, 128, 128, 3) X(DT_I8, 16, 64, 128, 128, 3)

#define GP_TILE_FP8(X)                                                                             \
  X(DT_FP8, 16, 16, 64, 512, 0) X(DT_FP8, 16, 32, 256, 128, 0) X(DT_FP8, 16, 64, 128, 128, 0)               \
  X(DT_FP8, 16, 64, 256, 128, 0) X(DT_FP8, 16, 128, 128, 128, 0) X(DT_FP8, 16, 128, 256, 128, 0)            \
  X(DT_FP8, 16, 64, 256, 256, 0) X(DT_FP8, 16, 128, 256, 128, 2) X(DT_FP8, 16, 128, 256, 128, 3)  \
  X(DT_FP8, 16, 64, 256, 128, 3) X(DT_FP8, 16, 32, 256, 128, 3)  \
  X(DT_FP8, 16, 32, 128, 128, 3) X(DT_FP8, 16, 32, 128, 256, 3) X(DT_FP8, 16, 32, 256, 256, 3)  \
  X(DT_FP8, 16, 32, 256, 128, 4) X(DT_FP8, 16, 32, 256, 128, 6)   \
  X(DT_FP8, 16, 32, 128, 256, 4) X(DT_FP8, 16, 32, 128, 256, 6) X(DT_FP8, 16, 64, 256, 128, 4)   \
  X(DT_FP8, 16, 64, 128, 256, 3) X(DT_FP8, 16, 128, 128, 128, 3) X(DT_FP8, 16, 128, 128, 256, 3)   \
  X(DT_FP8, 16, 128, 512, 128, 3) X(DT_FP8, 16, 64, 128, 512, 3) X(DT_FP8, 16, 64, 128, 512, 2)

#define GP_TILE_BF16(X) X(DT_BF16, 16, 16, 64, 256, 0) \
  X(DT_BF16, 16, 32, 128, 128, 0) X(DT_BF16, 16, 64, 128, 128, 0) X(DT_BF16, 16, 128, 256, 128, 0) X(DT_BF16, 16, 128, 256, 64, 0)          \
  X(DT_BF16, 32, 64, 128, 128, 0) X(DT_BF16, 32, 64, 256, 128, 0) X(DT_BF16, 32, 128, 128, 128, 0)          \
  X(DT_BF16, 32, 128, 256, 128, 0) X(DT_BF16, 32, 128, 256, 64, 0)                                \
  X(DT_BF16, 32, 128, 256, 128, 2) X(DT_BF16, 32, 128, 256, 128, 3) X(DT_BF16, 16, 128, 256, 128, 3) \
  X(DT_BF16, 32, 256, 256, 128, 3) X(DT_BF16, 32, 256, 256, 128, 2) \
  X(DT_BF16, 32, 256, 256, 64, 3) X(DT_BF16, 16, 256, 256, 64, 3) X(DT_BF16, 16, 256, 256, 64, 4) \
  X(DT_BF16, 16, 128, 512, 128, 3) X(DT_BF16, 32, 128, 512, 128, 3) X(DT_BF16, 16, 128, 512, 128, 2) \
  X(DT_BF16, 16, 256, 256, 128, 3) X(DT_BF16, 16, 256, 256, 128, 2) X(DT_BF16, 16, 256, 256, 128, 4) \
  X(DT_BF16, 16, 64, 128, 128, 3) X(DT_BF16, 16, 64, 256, 128, 3) X(DT_BF16, 16, 128, 128, 128, 3)

#define GP_TILE_F16(X) X(DT_F16, 16, 16, 64, 256, 0) \
  X(DT_F16, 16, 32, 128, 128, 0) X(DT_F16, 16, 64, 128, 128, 0) X(DT_F16, 16, 64, 256, 128, 0)             \
  X(DT_F16, 16, 128, 128, 128, 0) X(DT_F16, 16, 128, 256, 128, 0) X(DT_F16, 16, 128, 256, 128, 3)          \
  X(DT_F16, 32, 128, 256, 128, 3) X(DT_F16, 32, 64, 128, 128, 0)                                  \
  X(DT_F16, 16, 128, 256, 64, 0) X(DT_F16, 16, 64, 128, 64, 0) X(DT_F16, 16, 128, 512, 128, 3)           \
  X(DT_F16, 32, 128, 512, 128, 3) X(DT_F16, 16, 256, 256, 128, 3) X(DT_F16, 16, 256, 256, 128, 4) \
  X(DT_F16, 16, 64, 128, 128, 3) X(DT_F16, 16, 64, 256, 128, 3) X(DT_F16, 16, 128, 128, 128, 3)

#define GP_TILE_FP4(X)                                                                             \
  X(DT_FP4, 16, 32, 256, 128, 0) X(DT_FP4, 16, 64, 128, 128, 0) X(DT_FP4, 16, 64, 256, 128, 0)              \
  X(DT_FP4, 32, 64, 128, 128, 0) X(DT_FP4, 32, 64, 256, 128, 0)                                    \
  X(DT_FP4, 32, 128, 128, 128, 0) X(DT_FP4, 32, 128, 256, 128, 0) X(DT_FP4, 32, 128, 256, 128, 2) \
  X(DT_FP4, 16, 128, 256, 64, 2) X(DT_FP4, 16, 64, 128, 64, 0)                                  \
  X(DT_FP4, 32, 256, 256, 128, 2) X(DT_FP4, 32, 256, 256, 128, 0) X(DT_FP4, 32, 128, 512, 128, 2)          \
  X(DT_FP4, 32, 128, 512, 128, 0) X(DT_FP4, 32, 64, 256, 128, 2) X(DT_FP4, 16, 32, 256, 128, 2) X(DT_FP4, 32, 64, 128, 128, 2) X(DT_FP4, 32, 128, 128, 128, 2)
// (No FP4 128 x 256 tile with 16 x 16 blocks, nor with a 3-stage pipeline:
// the first put its accumulators in scratch memory, the second spilled.)
// (No 256 x 256 tile for FP4 or FP8, nor for BF16 with 16 x 16 blocks and
// 128-byte K tiles: beside 256 accumulator registers per lane, their B stages
// do not fit the remaining registers and the compiler moved values, or the
// whole accumulator array, to scratch memory, at 50x the run time.)

#define GP_SPLITK_I8(Y) Y(DT_I8, 1, 4, 64, 1) Y(DT_I8, 1, 4, 256, 1) Y(DT_I8, 2, 4, 256, 1) Y(DT_I8, 1, 1, 64, 1) \
  Y(DT_I8, 2, 4, 256, 2) Y(DT_I8, 2, 8, 256, 4) Y(DT_I8, 1, 4, 128, 1) Y(DT_I8, 2, 4, 128, 1) Y(DT_I8, 2, 4, 128, 2)
#define GP_SPLITK_FP8(Y)                                                                           \
  Y(DT_FP8, 1, 4, 128, 1) Y(DT_FP8, 1, 4, 256, 1) Y(DT_FP8, 1, 4, 512, 1) Y(DT_FP8, 2, 4, 256, 1)             \
  Y(DT_FP8, 2, 4, 512, 1) Y(DT_FP8, 1, 8, 256, 1) Y(DT_FP8, 4, 4, 256, 1) Y(DT_FP8, 2, 8, 256, 1) Y(DT_FP8, 4, 8, 256, 1) \
  Y(DT_FP8, 1, 1, 128, 1) \
  Y(DT_FP8, 2, 4, 256, 2) Y(DT_FP8, 2, 8, 128, 4)
#define GP_SPLITK_BF16(Y) Y(DT_BF16, 1, 4, 64, 1) Y(DT_BF16, 1, 4, 256, 1) Y(DT_BF16, 2, 4, 256, 1) Y(DT_BF16, 1, 1, 64, 1) \
  Y(DT_BF16, 2, 4, 256, 2) Y(DT_BF16, 2, 8, 256, 4) Y(DT_BF16, 1, 4, 128, 1) Y(DT_BF16, 2, 4, 128, 1) Y(DT_BF16, 2, 4, 128, 2)
#define GP_SPLITK_FP4(Y) Y(DT_FP4, 1, 4, 64, 1) Y(DT_FP4, 1, 4, 256, 1) Y(DT_FP4, 2, 4, 256, 1) Y(DT_FP4, 1, 1, 64, 1) \
  Y(DT_FP4, 2, 4, 256, 2) Y(DT_FP4, 2, 8, 64, 4) \
  Y(DT_FP4, 1, 4, 128, 1) Y(DT_FP4, 2, 4, 128, 1) Y(DT_FP4, 2, 4, 128, 2)
#define GP_SPLITK_F16(Y) Y(DT_F16, 1, 4, 64, 1) Y(DT_F16, 1, 4, 256, 1) Y(DT_F16, 2, 4, 256, 1) Y(DT_F16, 1, 1, 64, 1) \
  Y(DT_F16, 2, 4, 256, 2) Y(DT_F16, 2, 8, 256, 4) Y(DT_F16, 1, 4, 128, 1) Y(DT_F16, 2, 4, 128, 1) Y(DT_F16, 2, 4, 128, 2)
// W4A8: chunk bytes are bytes of B (the int8 A chunk is twice as long)
#define GP_SPLITK_I4(Y)                                                                            \
  Y(DT_I4, 1, 4, 64, 1) Y(DT_I4, 1, 4, 128, 1) Y(DT_I4, 1, 4, 256, 1) Y(DT_I4, 2, 4, 64, 1) Y(DT_I4, 2, 4, 128, 1)  \
  Y(DT_I4, 2, 4, 256, 1) Y(DT_I4, 2, 8, 128, 1) Y(DT_I4, 1, 1, 64, 1) \
  Y(DT_I4, 2, 4, 128, 2) Y(DT_I4, 2, 8, 128, 4)

#define GP_WIDE_I8(W) W(DT_I8, 16, 128, 2) W(DT_I8, 32, 128, 2)
#define GP_WIDE_FP8(W) W(DT_FP8, 16, 128, 2)
#define GP_WIDE_BF16(W) W(DT_BF16, 16, 128, 2) W(DT_BF16, 32, 128, 2) W(DT_BF16, 16, 64, 3) W(DT_BF16, 32, 64, 3) \
  W(DT_BF16, 16, 64, 4) W(DT_BF16, 32, 64, 4)
#define GP_WIDE_F16(W) W(DT_F16, 16, 128, 2) W(DT_F16, 16, 64, 4)
#define GP_WIDE_FP4(W)  /* FP4 runs on the 4-wave kernel */

// Tile kernel with two K groups (8 waves, 512 threads): X2(dtype, mfma,
// tile_m, tile_n, tile_k_bytes, pipe), for grids of about one tile per CU.
#define GP_TILE_KG2_I8(X) X(DT_I8, 16, 64, 128, 128, 0)
#define GP_TILE_KG2_FP8(X) X(DT_FP8, 16, 64, 128, 256, 3) X(DT_FP8, 16, 32, 256, 256, 3) X(DT_FP8, 16, 64, 256, 128, 3)
#define GP_TILE_KG2_BF16(X) X(DT_BF16, 16, 128, 256, 128, 3) X(DT_BF16, 16, 64, 128, 128, 0)
#define GP_TILE_KG2_F16(X)
#define GP_TILE_KG2_FP4(X)

// W4A8 on the tile kernel (tile_k in bytes of B; A tiles are twice as long)
#define GP_TILE_I4(X) X(DT_I4, 16, 16, 64, 128, 0) \
  X(DT_I4, 16, 128, 256, 64, 3) X(DT_I4, 16, 64, 256, 64, 3) X(DT_I4, 16, 64, 128, 128, 3)         \
  X(DT_I4, 16, 64, 128, 64, 3) X(DT_I4, 16, 32, 128, 64, 3) X(DT_I4, 16, 32, 64, 64, 0)
#define GP_TILE_KG2_I4(X)
#define GP_WIDE_I4(W)

// Tiles that also have a variant with the compiler's own hot-loop order
// (gemm_opts.scheduler = 2): the planner's default tiles of the benchmark
// workloads, plain epilogue only.
#define GP_TILE_NOSCHED_I8(X) X(DT_I8, 16, 16, 64, 256, 0) X(DT_I8, 16, 64, 128, 256, 3)
#define GP_TILE_NOSCHED_FP8(X) X(DT_FP8, 16, 64, 128, 256, 3) X(DT_FP8, 16, 64, 256, 128, 3) \
  X(DT_FP8, 16, 128, 256, 128, 3) X(DT_FP8, 16, 128, 128, 256, 3)
#define GP_TILE_NOSCHED_BF16(X) X(DT_BF16, 16, 128, 256, 128, 3) X(DT_BF16, 16, 128, 512, 128, 3) \
  X(DT_BF16, 16, 256, 256, 128, 3)
#define GP_TILE_NOSCHED_F16(X) X(DT_F16, 16, 128, 256, 128, 3) X(DT_F16, 16, 128, 512, 128, 3) \
  X(DT_F16, 16, 256, 256, 128, 3)
#define GP_TILE_NOSCHED_FP4(X) X(DT_FP4, 32, 128, 256, 128, 2) X(DT_FP4, 32, 128, 512, 128, 2)
#define GP_TILE_NOSCHED_I4(X) X(DT_I4, 16, 64, 128, 128, 3)
#define GP_TILE_NOSCHED_ALL(X) GP_TILE_NOSCHED_I8(X) GP_TILE_NOSCHED_FP8(X) GP_TILE_NOSCHED_BF16(X) \
  GP_TILE_NOSCHED_F16(X) GP_TILE_NOSCHED_FP4(X) GP_TILE_NOSCHED_I4(X)

// Tiles that also have a variant able to split K across workgroups
// (gemm_ex_ws, gemm_opts.ksplit > 1), plain epilogue only, in the order the
// planner prefers them for an automatic split (measured on long-K shapes:
// FP8 64 x 128 beat 128 x 128, FP4 128 x 128 beat 128 x 256).
#define GP_TILE_KSPLIT_I8(X) X(DT_I8, 16, 64, 128, 256, 3) X(DT_I8, 16, 128, 128, 128, 0) X(DT_I8, 16, 16, 64, 256, 0)
#define GP_TILE_KSPLIT_FP8(X) X(DT_FP8, 16, 64, 128, 256, 3) X(DT_FP8, 16, 64, 256, 128, 3) X(DT_FP8, 16, 16, 64, 512, 0) \
  X(DT_FP8, 16, 32, 256, 256, 3) X(DT_FP8, 16, 128, 128, 128, 3) X(DT_FP8, 16, 128, 128, 256, 3)
#define GP_TILE_KSPLIT_BF16(X) X(DT_BF16, 16, 128, 256, 128, 3) X(DT_BF16, 16, 64, 128, 128, 0) X(DT_BF16, 16, 16, 64, 256, 0)
#define GP_TILE_KSPLIT_F16(X) X(DT_F16, 16, 128, 256, 128, 3) X(DT_F16, 16, 64, 128, 128, 0) X(DT_F16, 16, 16, 64, 256, 0)
#define GP_TILE_KSPLIT_FP4(X) X(DT_FP4, 32, 128, 128, 128, 0) X(DT_FP4, 32, 128, 256, 128, 2)
#define GP_TILE_KSPLIT_I4(X) X(DT_I4, 16, 64, 128, 128, 3) X(DT_I4, 16, 64, 256, 64, 3) X(DT_I4, 16, 16, 64, 128, 0)
#define GP_TILE_KSPLIT_ALL(X) GP_TILE_KSPLIT_I8(X) GP_TILE_KSPLIT_FP8(X) GP_TILE_KSPLIT_BF16(X) \
  GP_TILE_KSPLIT_F16(X) GP_TILE_KSPLIT_FP4(X) GP_TILE_KSPLIT_I4(X)

#define GP_TILE_ALL(X) GP_TILE_I8(X) GP_TILE_FP8(X) GP_TILE_BF16(X) GP_TILE_FP4(X) GP_TILE_F16(X) GP_TILE_I4(X)
#define GP_TILE_KG2_ALL(X) GP_TILE_KG2_I8(X) GP_TILE_KG2_FP8(X) GP_TILE_KG2_BF16(X) GP_TILE_KG2_F16(X) GP_TILE_KG2_FP4(X) \
  GP_TILE_KG2_I4(X)
#define GP_SPLITK_ALL(Y) \
  GP_SPLITK_I8(Y) GP_SPLITK_FP8(Y) GP_SPLITK_BF16(Y) GP_SPLITK_FP4(Y) GP_SPLITK_F16(Y) GP_SPLITK_I4(Y)
#define GP_WIDE_ALL(W) GP_WIDE_I8(W) GP_WIDE_FP8(W) GP_WIDE_BF16(W) GP_WIDE_FP4(W) GP_WIDE_F16(W)
