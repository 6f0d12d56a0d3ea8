// Kernel instantiations and launch tables for one input type.
#include "launch.hpp"
#include "variants.hpp"

namespace gp {

hipError_t launch_tile_i8(int ms, int tm, int tn, int tkb, int pipe, int epi, const TileArgs& a, hipStream_t s) {
  GP_TILE_I8(GP_TILE_CASE)
  return hipErrorInvalidValue;
}

hipError_t launch_splitk_i8(int nb, int waves, int kch, const SplitArgs& a, hipStream_t s) {
  GP_SPLITK_I8(GP_SPLITK_CASE)
  return hipErrorInvalidValue;
}

hipError_t launch_wide_i8(int ms, int tkb, int pipe, const TileArgs& a, hipStream_t s) {
  GP_WIDE_I8(GP_WIDE_CASE)
  return hipErrorInvalidValue;
}

}  // namespace gp
