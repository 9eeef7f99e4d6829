// k_tiled_small.hip -- register-staged kernels of configuration CfgSmall, plain
// and fused epilogue.
#include "kernels.hpp"
#include "k_tiled.inc"

namespace tgemm {
KernelFn tiled_kernel_small(int in, int out, bool fast, bool epi) {
    return epi ? tiled_pick_half<CfgSmall, true>(in, out, fast) : tiled_pick_half<CfgSmall, false>(in, out, fast);
}
}  // namespace tgemm
