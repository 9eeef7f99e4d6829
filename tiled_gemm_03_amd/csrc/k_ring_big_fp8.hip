// k_ring_big_fp8.hip -- direct-to-LDS ring kernels of configuration RingBig (256 x 256 tiles)
// with an 8-bit float output (fused epilogue), without the K tail.
#include "kernels.hpp"
#include "k_ring.inc"

namespace tgemm {
KernelFn ring_kernel_big_fp8(int in, int la, int lb) { return ring_pick_fp8<RingBig, false>(in, la, lb); }
}  // namespace tgemm
