// k_ring_mid.hip -- direct-to-LDS ring kernels of configuration RingMid.
#include "kernels.hpp"
#include "k_ring.inc"

namespace tgemm {
KernelFn ring_kernel_mid(int in, int out, int la, int lb) { return ring_pick<RingMid>(in, out, la, lb); }
}  // namespace tgemm
