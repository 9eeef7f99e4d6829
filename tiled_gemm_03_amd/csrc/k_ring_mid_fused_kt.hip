// k_ring_mid_fused_kt.hip -- direct-to-LDS ring kernels of configuration
// RingMid with the K tail (K not a multiple of 128) and the fused epilogue.
#include "kernels.hpp"
#include "k_ring.inc"

namespace tgemm {
KernelFn ring_kernel_mid_fused_kt(int in, int out, int la, int lb) { return ring_pick<RingMid, true, true>(in, out, la, lb); }
}  // namespace tgemm
