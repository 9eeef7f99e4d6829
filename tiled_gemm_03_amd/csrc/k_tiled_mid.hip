// k_tiled_mid.hip -- register-staged kernels of configuration CfgMid.
#include "kernels.hpp"
#include "k_tiled.inc"

namespace tgemm {
KernelFn tiled_kernel_mid(int in, int out, bool fast) { return tiled_pick_half<CfgMid>(in, out, fast); }
}  // namespace tgemm
