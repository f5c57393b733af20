// Instantiations of the fused layer kernel with 8-bit gate/up weights.
#include "layer_kernel.hpp"

namespace moe {
LayerFn layer_kernel_a8(int bb, int sb, int xt) { return layer_kernel_pick<8, kLayerNRA>(bb, sb, xt); }
}  // namespace moe
