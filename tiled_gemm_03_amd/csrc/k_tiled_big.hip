// k_tiled_big.hip -- register-staged kernels of configuration CfgBig, plain
// epilogue (the fused ones: k_tiled_big_fused.hip).
#include "kernels.hpp"
#include "k_tiled.inc"

namespace tgemm {
KernelFn tiled_kernel_big(int in, int out, bool fast, bool epi) {
    return epi ? tiled_kernel_big_fused(in, out, fast) : tiled_pick_half<CfgBig, false>(in, out, fast);
}
}  // namespace tgemm
