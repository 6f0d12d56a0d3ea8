// Kernel instantiations and launch tables for one input type (plain epilogue).
#include "launch.hpp"
#include "variants.hpp"

namespace gp {

GP_DEFINE_PLAIN(fp8, GP_TILE_FP8, GP_TILE_KG2_FP8, GP_WIDE_FP8, GP_TILE_NOSCHED_FP8, GP_TILE_KSPLIT_FP8)

hipError_t launch_splitk_fp8(int nb, int waves, int kch, int mb, const SplitArgs& a, hipStream_t s) {
  GP_SPLITK_FP8(GP_SPLITK_CASE)
  return hipErrorInvalidValue;
}

}  // namespace gp
