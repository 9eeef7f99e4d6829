// k_ring_mid.hip -- direct-to-LDS ring kernels of configuration RingMid, plain
// epilogue (the fused ones: k_ring_mid_fused.hip; with the K tail:
// k_ring_mid_kt.hip).
#include "kernels.hpp"
#include "k_ring.inc"

namespace tgemm {
KernelFn ring_kernel_mid(int in, int out, int la, int lb, bool epi, bool kt) {
    if (out == DT_FP8) return ring_kernel_mid_fp8(in, la, lb, kt);
    if (epi) return ring_kernel_mid_fused(in, out, la, lb, kt);
    if (kt) return ring_kernel_mid_kt(in, out, la, lb);
    return ring_pick<RingMid, false, false>(in, out, la, lb);
}
}  // namespace tgemm
