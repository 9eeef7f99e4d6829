// k_tiled_f32.hip -- register-staged kernels of the fp32 configurations.
#include "kernels.hpp"

namespace tgemm {
KernelFn tiled_kernel_f32(int cfg, int in, int out, bool fast) {
    if (in != DT_F32 || out != DT_F32) return nullptr;
    if (cfg == CFG_F32_MID)
        return fast ? gemm_kernel<CfgF32Mid, DT_F32, DT_F32, true> : gemm_kernel<CfgF32Mid, DT_F32, DT_F32, false>;
    if (cfg == CFG_F32_TINY)
        return fast ? gemm_kernel<CfgF32Tiny, DT_F32, DT_F32, true> : gemm_kernel<CfgF32Tiny, DT_F32, DT_F32, false>;
    return nullptr;
}
}  // namespace tgemm
