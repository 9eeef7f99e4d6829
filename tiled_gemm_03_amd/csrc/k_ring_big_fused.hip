// k_ring_big_fused.hip -- direct-to-LDS ring kernels of configuration RingBig
// with the fused epilogue (with the K tail: k_ring_big_fused_kt.hip).
#include "kernels.hpp"
#include "k_ring.inc"

namespace tgemm {
KernelFn ring_kernel_big_fused(int in, int out, int la, int lb, bool kt) {
    return kt ? ring_kernel_big_fused_kt(in, out, la, lb) : ring_pick<RingBig, true, false>(in, out, la, lb);
}
}  // namespace tgemm
