// k_tiled_tiny.hip -- register-staged kernels of configuration CfgTiny, plain
// and fused epilogue.
#include "kernels.hpp"
#include "k_tiled.inc"

namespace tgemm {
KernelFn tiled_kernel_tiny(int in, int out, bool fast, bool epi) {
    return epi ? tiled_pick_half<CfgTiny, true>(in, out, fast) : tiled_pick_half<CfgTiny, false>(in, out, fast);
}
}  // namespace tgemm
