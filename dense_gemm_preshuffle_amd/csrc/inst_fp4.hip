// Kernel instantiations and launch tables for one input type (plain epilogue).
#include "launch.hpp"
#include "variants.hpp"

namespace gp {

GP_DEFINE_PLAIN(fp4, GP_TILE_FP4, GP_TILE_KG2_FP4, GP_WIDE_FP4, GP_TILE_NOSCHED_FP4, GP_TILE_KSPLIT_FP4)

hipError_t launch_splitk_fp4(int nb, int waves, int kch, int mb, const SplitArgs& a, hipStream_t s) {
  GP_SPLITK_FP4(GP_SPLITK_CASE)
  return hipErrorInvalidValue;
}

}  // namespace gp
