// Kernel instantiations and launch tables for one input type (plain epilogue).
#include "launch.hpp"
#include "variants.hpp"

namespace gp {

GP_DEFINE_PLAIN(bf16, GP_TILE_BF16, GP_TILE_KG2_BF16, GP_WIDE_BF16, GP_TILE_NOSCHED_BF16, GP_TILE_KSPLIT_BF16)

hipError_t launch_splitk_bf16(int nb, int waves, int kch, int mb, const SplitArgs& a, hipStream_t s) {
  GP_SPLITK_BF16(GP_SPLITK_CASE)
  return hipErrorInvalidValue;
}

}  // namespace gp
