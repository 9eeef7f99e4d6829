// k_ring_small.hip -- direct-to-LDS ring kernels of configuration RingSmall
// (64 x 128 tiles, row-major A), plain epilogue with and without the K tail
// (the fused ones: k_ring_small_fused.hip).
#include "kernels.hpp"
#include "k_ring.inc"

namespace tgemm {
KernelFn ring_kernel_small(int in, int out, int la, int lb, bool epi, bool kt) {
    if (out == DT_FP8) return ring_kernel_small_fp8(in, la, lb, kt);
    if (epi) return ring_kernel_small_fused(in, out, la, lb, kt);
    if (kt) return ring_pick<RingSmall, false, true>(in, out, la, lb);
    return ring_pick<RingSmall, false, false>(in, out, la, lb);
}
}  // namespace tgemm
