// k_ring_mid_fused.hip -- direct-to-LDS ring kernels of configuration RingMid
// with the fused epilogue.
#include "kernels.hpp"
#include "k_ring.inc"

namespace tgemm {
KernelFn ring_kernel_mid_fused(int in, int out, int la, int lb) { return ring_pick<RingMid, true>(in, out, la, lb); }
}  // namespace tgemm
