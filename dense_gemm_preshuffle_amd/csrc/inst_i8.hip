// Kernel instantiations and launch tables for INT8 (exact int32 output: no
// fused epilogue, so no fused variants).
#include "launch.hpp"
#include "variants.hpp"

namespace gp {

hipError_t launch_tile_i8_fused(int, int, int, int, int, int, int, const TileArgs&, hipStream_t) {
  return hipErrorInvalidValue;
}
hipError_t launch_wide_i8_fused(int, int, int, const TileArgs&, hipStream_t) { return hipErrorInvalidValue; }

GP_DEFINE_PLAIN(i8, GP_TILE_I8, GP_TILE_KG2_I8, GP_WIDE_I8, GP_TILE_NOSCHED_I8, GP_TILE_KSPLIT_I8)

hipError_t launch_splitk_i8(int nb, int waves, int kch, int mb, const SplitArgs& a, hipStream_t s) {
  GP_SPLITK_I8(GP_SPLITK_CASE)
  return hipErrorInvalidValue;
}

}  // namespace gp
