// W4A8 tile-kernel instantiations with the fused bias / activation epilogue
// (Kernel Tuning Guide §6).
#include "launch.hpp"
#include "variants.hpp"

namespace gp {

GP_DEFINE_FUSED(i4, GP_TILE_I4, GP_TILE_KG2_I4, GP_WIDE_I4, GP_TILE_KSPLIT_I4)

}  // namespace gp
