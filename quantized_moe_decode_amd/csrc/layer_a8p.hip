// Instantiations of the fused layer kernel (pipelined kernel-A units) with 8-bit gate/up weights.
#include "layer_kernel.hpp"

namespace moe {
LayerFn layer_kernel_a8p(int bb, int sb, int xt) { return layer_kernel_pick<8, kLayerNRA2>(bb, sb, xt); }
}  // namespace moe
