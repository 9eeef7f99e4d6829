// k_ring_mid_kt.hip -- direct-to-LDS ring kernels of configuration RingMid with
// the K tail (K not a multiple of 128), plain epilogue.
#include "kernels.hpp"
#include "k_ring.inc"

namespace tgemm {
KernelFn ring_kernel_mid_kt(int in, int out, int la, int lb) { return ring_pick<RingMid, false, true>(in, out, la, lb); }
}  // namespace tgemm
