// Kernel instantiations and launch tables for one input type (plain epilogue).
#include "launch.hpp"
#include "variants.hpp"

namespace gp {

GP_DEFINE_PLAIN(f16, GP_TILE_F16, GP_TILE_KG2_F16, GP_WIDE_F16, GP_TILE_NOSCHED_F16, GP_TILE_KSPLIT_F16)

hipError_t launch_splitk_f16(int nb, int waves, int kch, int mb, const SplitArgs& a, hipStream_t s) {
  GP_SPLITK_F16(GP_SPLITK_CASE)
  return hipErrorInvalidValue;
}

}  // namespace gp
