// k_tiled_mid.hip -- register-staged kernels of configuration CfgMid, plain
// and fused epilogue.
#include "kernels.hpp"
#include "k_tiled.inc"

namespace tgemm {
KernelFn tiled_kernel_mid(int in, int out, bool fast, bool epi) {
    return epi ? tiled_pick_half<CfgMid, true>(in, out, fast) : tiled_pick_half<CfgMid, false>(in, out, fast);
}
}  // namespace tgemm
