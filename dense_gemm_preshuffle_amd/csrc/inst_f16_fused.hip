// Kernel instantiations with the fused bias / activation epilogue for one
// input type (Kernel Tuning Guide §6).
#include "launch.hpp"
#include "variants.hpp"

namespace gp {

GP_DEFINE_FUSED(f16, GP_TILE_F16, GP_TILE_KG2_F16, GP_WIDE_F16, GP_TILE_KSPLIT_F16)

}  // namespace gp
