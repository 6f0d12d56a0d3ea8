// Compiled kernel variants. The host planner and the launch tables both read
// these lists, so a tile the planner may pick is always instantiated.
//
// Tile kernel: X(dtype, tile_m, tile_n, tile_k_bytes); each is built with the
// direct and the CShuffle epilogue.
// Split-K kernel: Y(dtype, n_blocks_of_16, waves, chunk_bytes_per_wave).
#pragma once

#define GP_TILE_I8(X)                                                                   \
  X(DT_I8, 16, 64, 256) X(DT_I8, 32, 64, 128) X(DT_I8, 64, 64, 128)                    \
  X(DT_I8, 64, 128, 128) X(DT_I8, 64, 256, 128) X(DT_I8, 128, 128, 128)                \
  X(DT_I8, 128, 256, 128)

#define GP_TILE_FP8(X)                                                                  \
  X(DT_FP8, 16, 64, 512) X(DT_FP8, 32, 256, 128) X(DT_FP8, 64, 128, 128)               \
  X(DT_FP8, 64, 256, 128) X(DT_FP8, 128, 128, 128) X(DT_FP8, 128, 256, 128)            \
  X(DT_FP8, 64, 256, 256)

#define GP_TILE_BF16(X)                                                                 \
  X(DT_BF16, 64, 128, 128) X(DT_BF16, 64, 256, 128) X(DT_BF16, 128, 128, 128)          \
  X(DT_BF16, 128, 256, 128) X(DT_BF16, 128, 256, 64)

#define GP_TILE_FP4(X)                                                                  \
  X(DT_FP4, 32, 256, 128) X(DT_FP4, 64, 128, 128) X(DT_FP4, 64, 256, 128)              \
  X(DT_FP4, 128, 128, 128) X(DT_FP4, 128, 256, 128)

#define GP_SPLITK_I8(Y) Y(DT_I8, 1, 4, 64) Y(DT_I8, 1, 4, 256) Y(DT_I8, 2, 4, 256)
#define GP_SPLITK_FP8(Y)                                                                \
  Y(DT_FP8, 1, 4, 128) Y(DT_FP8, 1, 4, 256) Y(DT_FP8, 1, 4, 512) Y(DT_FP8, 2, 4, 256)  \
  Y(DT_FP8, 2, 4, 512) Y(DT_FP8, 1, 8, 256) Y(DT_FP8, 4, 4, 256)
#define GP_SPLITK_BF16(Y) Y(DT_BF16, 1, 4, 64) Y(DT_BF16, 1, 4, 256) Y(DT_BF16, 2, 4, 256)
#define GP_SPLITK_FP4(Y) Y(DT_FP4, 1, 4, 64) Y(DT_FP4, 1, 4, 256) Y(DT_FP4, 2, 4, 256)

#define GP_TILE_ALL(X) GP_TILE_I8(X) GP_TILE_FP8(X) GP_TILE_BF16(X) GP_TILE_FP4(X)
#define GP_SPLITK_ALL(Y) GP_SPLITK_I8(Y) GP_SPLITK_FP8(Y) GP_SPLITK_BF16(Y) GP_SPLITK_FP4(Y)
