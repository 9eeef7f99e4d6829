// k_tiled_f32.hip -- register-staged kernels of the fp32 configurations,
// plain and fused epilogue.
#include "kernels.hpp"

namespace tgemm {
namespace {
template <class T, bool EPI>
KernelFn f32_pick(bool fast) {
    return fast ? gemm_kernel<T, DT_F32, DT_F32, true, EPI> : gemm_kernel<T, DT_F32, DT_F32, false, EPI>;
}
}  // namespace

KernelFn tiled_kernel_f32(int cfg, int in, int out, bool fast, bool epi) {
    if (in != DT_F32 || out != DT_F32) return nullptr;
    if (cfg == CFG_F32_MID) return epi ? f32_pick<CfgF32Mid, true>(fast) : f32_pick<CfgF32Mid, false>(fast);
    if (cfg == CFG_F32_BIG) return epi ? f32_pick<CfgF32Big, true>(fast) : f32_pick<CfgF32Big, false>(fast);
    if (cfg == CFG_F32_TINY) return epi ? f32_pick<CfgF32Tiny, true>(fast) : f32_pick<CfgF32Tiny, false>(fast);
    return nullptr;
}
}  // namespace tgemm
