// Launch-table interface between the host API and the per-dtype kernel
// translation units.
#pragma once

#include <hip/hip_runtime.h>

#include "gemm_splitk.hpp"
#include "gemm_tile.hpp"
#include "gemm_wide.hpp"

namespace gp {

// Each returns hipErrorInvalidValue if the variant is not compiled.
hipError_t launch_tile_i8(int ms, int tm, int tn, int tkb, int pipe, int epi, const TileArgs& a, hipStream_t s);
hipError_t launch_tile_fp8(int ms, int tm, int tn, int tkb, int pipe, int epi, const TileArgs& a, hipStream_t s);
hipError_t launch_tile_bf16(int ms, int tm, int tn, int tkb, int pipe, int epi, const TileArgs& a, hipStream_t s);
hipError_t launch_tile_fp4(int ms, int tm, int tn, int tkb, int pipe, int epi, const TileArgs& a, hipStream_t s);
hipError_t launch_splitk_i8(int nb, int waves, int kch, const SplitArgs& a, hipStream_t s);
hipError_t launch_splitk_fp8(int nb, int waves, int kch, const SplitArgs& a, hipStream_t s);
hipError_t launch_splitk_bf16(int nb, int waves, int kch, const SplitArgs& a, hipStream_t s);
hipError_t launch_splitk_fp4(int nb, int waves, int kch, const SplitArgs& a, hipStream_t s);
hipError_t launch_wide_i8(int ms, int tkb, int pipe, const TileArgs& a, hipStream_t s);
hipError_t launch_wide_fp8(int ms, int tkb, int pipe, const TileArgs& a, hipStream_t s);
hipError_t launch_wide_bf16(int ms, int tkb, int pipe, const TileArgs& a, hipStream_t s);

}  // namespace gp

// Body of one dtype's launch tables.
#define GP_TILE_CASE(DT, MS, TM, TN, TKB, PIPE)                                            \
  if (ms == MS && tm == TM && tn == TN && tkb == TKB && pipe == PIPE) {                    \
    const dim3 grid(a.tiles_m * a.tiles_n);                                                \
    if (epi == EPI_CSHUFFLE)                                                               \
      hipLaunchKernelGGL((gemm_tile_kernel<DT, MS, TM, TN, TKB, EPI_CSHUFFLE, PIPE>), grid, dim3(256), 0, s, a); \
    else                                                                                   \
      hipLaunchKernelGGL((gemm_tile_kernel<DT, MS, TM, TN, TKB, EPI_DIRECT, PIPE>), grid, dim3(256), 0, s, a);   \
    return hipGetLastError();                                                              \
  }
#define GP_SPLITK_CASE(DT, NB, W, KCH)                                                     \
  if (nb == NB && waves == W && kch == KCH) {                                              \
    const dim3 grid(a.N / (16 * NB), a.M / 16);                                            \
    hipLaunchKernelGGL((gemm_splitk_kernel<DT, NB, W, KCH>), grid, dim3(W * 64), 0, s, a); \
    return hipGetLastError();                                                              \
  }
#define GP_WIDE_CASE(DT, MS, TKB, PIPE)                                                     \
  if (ms == MS && tkb == TKB && pipe == PIPE) {                                            \
    hipLaunchKernelGGL((gemm_wide_kernel<DT, MS, TKB, PIPE>), dim3(a.tiles_m * a.tiles_n), dim3(512), 0, s, a); \
    return hipGetLastError();                                                              \
  }
