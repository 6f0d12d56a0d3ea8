// Kernel instantiations with the fused bias / activation epilogue for one
// input type (Kernel Tuning Guide §6).
#include "launch.hpp"
#include "variants.hpp"

namespace gp {

GP_DEFINE_FUSED(bf16, GP_TILE_BF16, GP_TILE_KG2_BF16, GP_WIDE_BF16, GP_TILE_KSPLIT_BF16)

}  // namespace gp
