// Kernel instantiations and launch tables of the W4A8 type (plain epilogue).
#include "launch.hpp"
#include "variants.hpp"

namespace gp {

GP_DEFINE_PLAIN(i4, GP_TILE_I4, GP_TILE_KG2_I4, GP_WIDE_I4, GP_TILE_NOSCHED_I4, GP_TILE_KSPLIT_I4)

hipError_t launch_splitk_i4(int nb, int waves, int kch, int mb, const SplitArgs& a, hipStream_t s) {
  GP_SPLITK_I4(GP_SPLITK_CASE)
  return hipErrorInvalidValue;
}

}  // namespace gp
