// k_tiled_tiny.hip -- register-staged kernels of configuration CfgTiny.
#include "kernels.hpp"
#include "k_tiled.inc"

namespace tgemm {
KernelFn tiled_kernel_tiny(int in, int out, bool fast) { return tiled_pick_half<CfgTiny>(in, out, fast); }
}  // namespace tgemm
