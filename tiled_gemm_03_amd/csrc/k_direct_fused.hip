// k_direct_fused.hip -- the direct kernels with the fused epilogue.
#include "gemm_kernel_direct.hpp"
#include "kernels.hpp"
#include "k_direct.inc"

namespace tgemm {
KernelFn direct_kernel_fused(int in, int out, int la, int lb, bool va, bool vb) {
    return direct_pick<true>(in, out, la, lb, va, vb);
}
}  // namespace tgemm
