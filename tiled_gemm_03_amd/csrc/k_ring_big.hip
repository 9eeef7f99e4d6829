// k_ring_big.hip -- direct-to-LDS ring kernels of configuration RingBig.
#include "kernels.hpp"
#include "k_ring.inc"

namespace tgemm {
KernelFn ring_kernel_big(int in, int out, int la, int lb) { return ring_pick<RingBig>(in, out, la, lb); }
}  // namespace tgemm
