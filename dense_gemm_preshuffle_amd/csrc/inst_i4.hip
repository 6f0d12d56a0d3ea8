// Kernel instantiations and launch table of the W4A8 type (small-M kernel only).
#include "launch.hpp"
#include "variants.hpp"

namespace gp {

hipError_t launch_splitk_i4(int nb, int waves, int kch, const SplitArgs& a, hipStream_t s) {
  GP_SPLITK_I4(GP_SPLITK_CASE)
  return hipErrorInvalidValue;
}

}  // namespace gp
