// k_ring_big_fp8_kt.hip -- direct-to-LDS ring kernels of configuration RingBig (256 x 256 tiles)
// with an 8-bit float output (fused epilogue), with the K tail.
#include "kernels.hpp"
#include "k_ring.inc"

namespace tgemm {
KernelFn ring_kernel_big_fp8_kt(int in, int la, int lb) { return ring_pick_fp8<RingBig, true>(in, la, lb); }
}  // namespace tgemm
