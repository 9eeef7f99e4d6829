// k_ring_mid.hip -- direct-to-LDS ring kernels of configuration RingMid, plain
// epilogue (the fused ones: k_ring_mid_fused.hip).
#include "kernels.hpp"
#include "k_ring.inc"

namespace tgemm {
KernelFn ring_kernel_mid(int in, int out, int la, int lb, bool epi) {
    return epi ? ring_kernel_mid_fused(in, out, la, lb) : ring_pick<RingMid, false>(in, out, la, lb);
}
}  // namespace tgemm
