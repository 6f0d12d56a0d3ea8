// Kernel instantiations with the fused bias / activation epilogue for one
// input type (Kernel Tuning Guide §6).
#include "launch.hpp"
#include "variants.hpp"

namespace gp {

GP_DEFINE_FUSED(fp4, GP_TILE_FP4, GP_TILE_KG2_FP4, GP_WIDE_FP4, GP_TILE_KSPLIT_FP4)

}  // namespace gp
