// k_direct.hip -- the direct kernels (operands straight to registers) for
// every type pair, operand layout and load width, plain epilogue (the fused
// ones: k_direct_fused.hip).
#include "gemm_kernel_direct.hpp"
#include "kernels.hpp"
#include "k_direct.inc"

namespace tgemm {
KernelFn direct_kernel(int in, int out, int la, int lb, bool va, bool vb, bool epi) {
    if (out == DT_FP8) return direct_kernel_fp8(in, la, lb, va, vb);
    return epi ? direct_kernel_fused(in, out, la, lb, va, vb) : direct_pick<false>(in, out, la, lb, va, vb);
}
}  // namespace tgemm
