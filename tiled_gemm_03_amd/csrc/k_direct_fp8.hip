// k_direct_fp8.hip -- the direct kernels with an 8-bit float output (fused
// epilogue; format chosen at run time).
#include "gemm_kernel_direct.hpp"
#include "kernels.hpp"
#include "k_direct.inc"

namespace tgemm {
KernelFn direct_kernel_fp8(int in, int la, int lb, bool va, bool vb) {
    if (in == DT_F16) return direct_pick_layout<DT_F16, DT_FP8, true>(la, lb, va, vb);
    if (in == DT_BF16) return direct_pick_layout<DT_BF16, DT_FP8, true>(la, lb, va, vb);
    return nullptr;
}
}  // namespace tgemm
