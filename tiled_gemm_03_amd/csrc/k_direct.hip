// k_direct.hip -- the direct kernels (operands straight to registers) for
// every type pair, operand layout and load width.
#include "gemm_kernel_direct.hpp"
#include "kernels.hpp"

namespace tgemm {
namespace {
template <int IN, int OUT, int LA, int LB>
KernelFn direct_pick_vec(bool va, bool vb) {
    // 16-byte loads only for a k-contiguous 16-bit operand
    constexpr bool CA = IN != DT_F32 && LA == LAYOUT_ROW, CB = IN != DT_F32 && LB == LAYOUT_COL;
    if constexpr (CA && CB) {
        if (va && vb) return gemm_kernel_direct<IN, OUT, LA, LB, true, true>;
        if (va) return gemm_kernel_direct<IN, OUT, LA, LB, true, false>;
        if (vb) return gemm_kernel_direct<IN, OUT, LA, LB, false, true>;
    } else if constexpr (CA) {
        if (va) return gemm_kernel_direct<IN, OUT, LA, LB, true, false>;
    } else if constexpr (CB) {
        if (vb) return gemm_kernel_direct<IN, OUT, LA, LB, false, true>;
    }
    return gemm_kernel_direct<IN, OUT, LA, LB, false, false>;
}
template <int IN, int OUT>
KernelFn direct_pick_layout(int la, int lb, bool va, bool vb) {
    if (la == LAYOUT_ROW && lb == LAYOUT_ROW) return direct_pick_vec<IN, OUT, LAYOUT_ROW, LAYOUT_ROW>(va, vb);
    if (la == LAYOUT_ROW && lb == LAYOUT_COL) return direct_pick_vec<IN, OUT, LAYOUT_ROW, LAYOUT_COL>(va, vb);
    if (la == LAYOUT_COL && lb == LAYOUT_ROW) return direct_pick_vec<IN, OUT, LAYOUT_COL, LAYOUT_ROW>(va, vb);
    if (la == LAYOUT_COL && lb == LAYOUT_COL) return direct_pick_vec<IN, OUT, LAYOUT_COL, LAYOUT_COL>(va, vb);
    return nullptr;
}
}  // namespace

KernelFn direct_kernel(int in, int out, int la, int lb, bool va, bool vb) {
    if (in == DT_F32 && out == DT_F32) return direct_pick_layout<DT_F32, DT_F32>(la, lb, false, false);
    if (in == DT_F16 && out == DT_F16) return direct_pick_layout<DT_F16, DT_F16>(la, lb, va, vb);
    if (in == DT_F16 && out == DT_F32) return direct_pick_layout<DT_F16, DT_F32>(la, lb, va, vb);
    if (in == DT_BF16 && out == DT_BF16) return direct_pick_layout<DT_BF16, DT_BF16>(la, lb, va, vb);
    if (in == DT_BF16 && out == DT_F32) return direct_pick_layout<DT_BF16, DT_F32>(la, lb, va, vb);
    return nullptr;
}
}  // namespace tgemm
