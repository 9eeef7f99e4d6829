// k_ring_big_fused_kt.hip -- direct-to-LDS ring kernels of configuration
// RingBig with the K tail (K not a multiple of 128) and the fused epilogue.
#include "kernels.hpp"
#include "k_ring.inc"

namespace tgemm {
KernelFn ring_kernel_big_fused_kt(int in, int out, int la, int lb) { return ring_pick<RingBig, true, true>(in, out, la, lb); }
}  // namespace tgemm
