// k_tiled_big_fused.hip -- register-staged kernels of configuration CfgBig
// with the fused epilogue.
#include "kernels.hpp"
#include "k_tiled.inc"

namespace tgemm {
KernelFn tiled_kernel_big_fused(int in, int out, bool fast) { return tiled_pick_half<CfgBig, true>(in, out, fast); }
}  // namespace tgemm
