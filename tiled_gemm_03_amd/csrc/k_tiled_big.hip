// k_tiled_big.hip -- register-staged kernels of configuration CfgBig.
#include "kernels.hpp"
#include "k_tiled.inc"

namespace tgemm {
KernelFn tiled_kernel_big(int in, int out, bool fast) { return tiled_pick_half<CfgBig>(in, out, fast); }
}  // namespace tgemm
