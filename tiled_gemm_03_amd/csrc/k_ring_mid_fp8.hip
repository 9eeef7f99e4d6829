// k_ring_mid_fp8.hip -- direct-to-LDS ring kernels of configuration RingMid (128 x 128 tiles)
// with an 8-bit float output (fused epilogue), with and without the K tail.
#include "kernels.hpp"
#include "k_ring.inc"

namespace tgemm {
KernelFn ring_kernel_mid_fp8(int in, int la, int lb, bool kt) {
    return kt ? ring_pick_fp8<RingMid, true>(in, la, lb) : ring_pick_fp8<RingMid, false>(in, la, lb);
}
}  // namespace tgemm
