// Instantiations of the fused layer kernel (pipelined kernel-A units) with 6-bit gate/up weights.
#include "layer_kernel.hpp"

namespace moe {
LayerFn layer_kernel_a6p(int bb, int sb, int xt) { return layer_kernel_pick<6, kLayerNRA2>(bb, sb, xt); }
}  // namespace moe
