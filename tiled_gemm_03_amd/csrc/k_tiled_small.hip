// k_tiled_small.hip -- register-staged kernels of configuration CfgSmall.
#include "kernels.hpp"
#include "k_tiled.inc"

namespace tgemm {
KernelFn tiled_kernel_small(int in, int out, bool fast) { return tiled_pick_half<CfgSmall>(in, out, fast); }
}  // namespace tgemm
