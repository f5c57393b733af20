// Instantiations of the fused layer kernel with 4-bit gate/up weights.
#include "layer_kernel.hpp"

namespace moe {
LayerFn layer_kernel_a4(int bb, int sb, int xt) { return layer_kernel_pick<4, kLayerNRA>(bb, sb, xt); }
}  // namespace moe
