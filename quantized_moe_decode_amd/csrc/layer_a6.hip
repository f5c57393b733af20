// Instantiations of the fused layer kernel with 6-bit gate/up weights.
#include "layer_kernel.hpp"

namespace moe {
LayerFn layer_kernel_a6(int bb, int sb, int xt) { return layer_kernel_pick<6, kLayerNRA>(bb, sb, xt); }
}  // namespace moe
