// k_ring_small_fp8.hip -- direct-to-LDS ring kernels of configuration RingSmall (64 x 128 tiles)
// with an 8-bit float output (fused epilogue), with and without the K tail.
#include "kernels.hpp"
#include "k_ring.inc"

namespace tgemm {
KernelFn ring_kernel_small_fp8(int in, int la, int lb, bool kt) {
    return kt ? ring_pick_fp8<RingSmall, true>(in, la, lb) : ring_pick_fp8<RingSmall, false>(in, la, lb);
}
}  // namespace tgemm
