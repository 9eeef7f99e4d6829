// k_ring_small_fused.hip -- direct-to-LDS ring kernels of configuration
// RingSmall (64 x 128 tiles, row-major A) with the fused epilogue, with and
// without the K tail.
#include "kernels.hpp"
#include "k_ring.inc"

namespace tgemm {
KernelFn ring_kernel_small_fused(int in, int out, int la, int lb, bool kt) {
    if (kt) return ring_pick<RingSmall, true, true>(in, out, la, lb);
    return ring_pick<RingSmall, true, false>(in, out, la, lb);
}
}  // namespace tgemm
