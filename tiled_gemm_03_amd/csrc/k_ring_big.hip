// k_ring_big.hip -- direct-to-LDS ring kernels of configuration RingBig, plain
// epilogue (the fused ones: k_ring_big_fused.hip; with the K tail:
// k_ring_big_kt.hip).
#include "kernels.hpp"
#include "k_ring.inc"

namespace tgemm {
KernelFn ring_kernel_big(int in, int out, int la, int lb, bool epi, bool kt) {
    if (out == DT_FP8) return kt ? ring_kernel_big_fp8_kt(in, la, lb) : ring_kernel_big_fp8(in, la, lb);
    if (epi) return ring_kernel_big_fused(in, out, la, lb, kt);
    if (kt) return ring_kernel_big_kt(in, out, la, lb);
    return ring_pick<RingBig, false, false>(in, out, la, lb);
}
}  // namespace tgemm
