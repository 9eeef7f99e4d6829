// k_ring_mid_fused.hip -- direct-to-LDS ring kernels of configuration RingMid
// with the fused epilogue (with the K tail: k_ring_mid_fused_kt.hip).
#include "kernels.hpp"
#include "k_ring.inc"

namespace tgemm {
KernelFn ring_kernel_mid_fused(int in, int out, int la, int lb, bool kt) {
    return kt ? ring_kernel_mid_fused_kt(in, out, la, lb) : ring_pick<RingMid, true, false>(in, out, la, lb);
}
}  // namespace tgemm
