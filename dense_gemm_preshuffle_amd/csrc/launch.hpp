// Launch-table interface between the host API and the per-dtype kernel
// translation units. Every tile and wide variant is built twice: plain, and
// with the fused bias / activation epilogue (its own translation unit, so
// the two halves compile in parallel).
#pragma once

#include <hip/hip_runtime.h>

#include "gemm_splitk.hpp"
#include "gemm_tile.hpp"
#include "gemm_wide.hpp"

namespace gp {

// Each returns hipErrorInvalidValue if the variant is not compiled.
#define GP_DECLARE_TILE(NAME)                                                                       \
  hipError_t launch_tile_##NAME(int ms, int tm, int tn, int tkb, int pipe, int epi, int kg, bool fused, \
                                bool sched, const TileArgs& a, hipStream_t s);                      \
  hipError_t launch_tile_##NAME##_fused(int ms, int tm, int tn, int tkb, int pipe, int epi, int kg, \
                                        const TileArgs& a, hipStream_t s);
#define GP_DECLARE_WIDE(NAME)                                                                       \
  hipError_t launch_wide_##NAME(int ms, int tkb, int pipe, bool fused, const TileArgs& a, hipStream_t s); \
  hipError_t launch_wide_##NAME##_fused(int ms, int tkb, int pipe, const TileArgs& a, hipStream_t s);
GP_DECLARE_TILE(i8) GP_DECLARE_TILE(fp8) GP_DECLARE_TILE(bf16) GP_DECLARE_TILE(fp4) GP_DECLARE_TILE(f16)
GP_DECLARE_TILE(i4)
GP_DECLARE_WIDE(i8) GP_DECLARE_WIDE(fp8) GP_DECLARE_WIDE(bf16) GP_DECLARE_WIDE(f16) GP_DECLARE_WIDE(fp4)
GP_DECLARE_WIDE(i4)
hipError_t launch_splitk_i8(int nb, int waves, int kch, int mb, const SplitArgs& a, hipStream_t s);
hipError_t launch_splitk_fp8(int nb, int waves, int kch, int mb, const SplitArgs& a, hipStream_t s);
hipError_t launch_splitk_bf16(int nb, int waves, int kch, int mb, const SplitArgs& a, hipStream_t s);
hipError_t launch_splitk_fp4(int nb, int waves, int kch, int mb, const SplitArgs& a, hipStream_t s);
hipError_t launch_splitk_f16(int nb, int waves, int kch, int mb, const SplitArgs& a, hipStream_t s);
hipError_t launch_splitk_i4(int nb, int waves, int kch, int mb, const SplitArgs& a, hipStream_t s);

}  // namespace gp

// Bodies of one dtype's launch tables.
// (the grid has one workgroup per tile and K split)
#define GP_TILE_CASE_IMPL(DT, MS, TM, TN, TKB, PIPE, FU, KGV, SCHV, KSV)                           \
  if (ms == MS && tm == TM && tn == TN && tkb == TKB && pipe == PIPE && kg == KGV && sched == SCHV && \
      (a.ksplit > 1) == KSV) {                                                                     \
    const dim3 grid(a.tiles_m * a.tiles_n * a.ksplit);                                             \
    if (epi == EPI_CSHUFFLE)                                                                       \
      hipLaunchKernelGGL((gemm_tile_kernel<DT, MS, TM, TN, TKB, EPI_CSHUFFLE, PIPE, FU, KGV, SCHV, KSV>), grid, dim3(64 * tile_waves(TM, TN) * KGV), 0, s, a); \
    else                                                                                           \
      hipLaunchKernelGGL((gemm_tile_kernel<DT, MS, TM, TN, TKB, EPI_DIRECT, PIPE, FU, KGV, SCHV, KSV>), grid, dim3(64 * tile_waves(TM, TN) * KGV), 0, s, a);   \
    return hipGetLastError();                                                                      \
  }
#define GP_TILE_CASE(DT, MS, TM, TN, TKB, PIPE) GP_TILE_CASE_IMPL(DT, MS, TM, TN, TKB, PIPE, false, 1, true, false)
#define GP_TILE_CASE_FUSED(DT, MS, TM, TN, TKB, PIPE) GP_TILE_CASE_IMPL(DT, MS, TM, TN, TKB, PIPE, true, 1, true, false)
#define GP_TILE_CASE_KG2(DT, MS, TM, TN, TKB, PIPE) GP_TILE_CASE_IMPL(DT, MS, TM, TN, TKB, PIPE, false, 2, true, false)
#define GP_TILE_CASE_KG2_FUSED(DT, MS, TM, TN, TKB, PIPE) GP_TILE_CASE_IMPL(DT, MS, TM, TN, TKB, PIPE, true, 2, true, false)
#define GP_TILE_CASE_NOSCHED(DT, MS, TM, TN, TKB, PIPE) GP_TILE_CASE_IMPL(DT, MS, TM, TN, TKB, PIPE, false, 1, false, false)
#define GP_TILE_CASE_KSPLIT(DT, MS, TM, TN, TKB, PIPE) GP_TILE_CASE_IMPL(DT, MS, TM, TN, TKB, PIPE, false, 1, true, true)
#define GP_TILE_CASE_KSPLIT_FUSED(DT, MS, TM, TN, TKB, PIPE) GP_TILE_CASE_IMPL(DT, MS, TM, TN, TKB, PIPE, true, 1, true, true)
#define GP_SPLITK_CASE(DT, NB, W, KCH, MB)                                                     \
  if (nb == NB && waves == W && kch == KCH && mb == MB) {                                      \
    const dim3 grid(a.N / (16 * NB), (a.M + 16 * MB - 1) / (16 * MB));                         \
    hipLaunchKernelGGL((gemm_splitk_kernel<DT, NB, W, KCH, MB>), grid, dim3(W * 64), 0, s, a); \
    return hipGetLastError();                                                                  \
  }
#define GP_WIDE_CASE_IMPL(DT, MS, TKB, PIPE, FU)                                                  \
  if (ms == MS && tkb == TKB && pipe == PIPE) {                                                   \
    hipLaunchKernelGGL((gemm_wide_kernel<DT, MS, TKB, PIPE, FU>), dim3(a.tiles_m * a.tiles_n), dim3(512), 0, s, a); \
    return hipGetLastError();                                                                     \
  }
#define GP_WIDE_CASE(DT, MS, TKB, PIPE) GP_WIDE_CASE_IMPL(DT, MS, TKB, PIPE, false)
#define GP_WIDE_CASE_FUSED(DT, MS, TKB, PIPE) GP_WIDE_CASE_IMPL(DT, MS, TKB, PIPE, true)

// Plain launch tables of one dtype (the fused ones are in inst_<name>_fused.hip).
#define GP_DEFINE_PLAIN(NAME, TILES, KG2TILES, WIDES, NOSCHED, KSPLIT)                              \
  hipError_t launch_tile_##NAME(int ms, int tm, int tn, int tkb, int pipe, int epi, int kg, bool fused, \
                                bool sched, const TileArgs& a, hipStream_t s) {                     \
    if (fused) return sched ? launch_tile_##NAME##_fused(ms, tm, tn, tkb, pipe, epi, kg, a, s)     \
                            : hipErrorInvalidValue;                                                 \
    TILES(GP_TILE_CASE)                                                                             \
    KG2TILES(GP_TILE_CASE_KG2)                                                                      \
    NOSCHED(GP_TILE_CASE_NOSCHED)                                                                   \
    KSPLIT(GP_TILE_CASE_KSPLIT)                                                                     \
    return hipErrorInvalidValue;                                                                    \
  }                                                                                                 \
  hipError_t launch_wide_##NAME(int ms, int tkb, int pipe, bool fused, const TileArgs& a, hipStream_t s) { \
    if (fused) return launch_wide_##NAME##_fused(ms, tkb, pipe, a, s);                              \
    WIDES(GP_WIDE_CASE)                                                                             \
    return hipErrorInvalidValue;                                                                    \
  }
#define GP_DEFINE_FUSED(NAME, TILES, KG2TILES, WIDES, KSPLIT)                                       \
  hipError_t launch_tile_##NAME##_fused(int ms, int tm, int tn, int tkb, int pipe, int epi, int kg, \
                                        const TileArgs& a, hipStream_t s) {                         \
    constexpr bool sched = true; /* fused variants keep the pinned schedule */                       \
    TILES(GP_TILE_CASE_FUSED)                                                                       \
    KG2TILES(GP_TILE_CASE_KG2_FUSED)                                                                \
    KSPLIT(GP_TILE_CASE_KSPLIT_FUSED)                                                               \
    return hipErrorInvalidValue;                                                                    \
  }                                                                                                 \
  hipError_t launch_wide_##NAME##_fused(int ms, int tkb, int pipe, const TileArgs& a, hipStream_t s) { \
    WIDES(GP_WIDE_CASE_FUSED)                                                                       \
    return hipErrorInvalidValue;                                                                    \
  }
