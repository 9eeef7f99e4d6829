// k_ring_big_fused.hip -- direct-to-LDS ring kernels of configuration RingBig
// with the fused epilogue.
#include "kernels.hpp"
#include "k_ring.inc"

namespace tgemm {
KernelFn ring_kernel_big_fused(int in, int out, int la, int lb) { return ring_pick<RingBig, true>(in, out, la, lb); }
}  // namespace tgemm
