// k_ring_big.hip -- direct-to-LDS ring kernels of configuration RingBig, plain
// epilogue (the fused ones: k_ring_big_fused.hip).
#include "kernels.hpp"
#include "k_ring.inc"

namespace tgemm {
KernelFn ring_kernel_big(int in, int out, int la, int lb, bool epi) {
    return epi ? ring_kernel_big_fused(in, out, la, lb) : ring_pick<RingBig, false>(in, out, la, lb);
}
}  // namespace tgemm
