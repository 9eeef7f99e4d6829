// kernels.hpp -- the tile configurations of the table and the kernel
// selectors.  Each kernel family is compiled in translation units of its own
// (k_*.hip, built in parallel); the host code (tgemm.hip) only sees these
// selectors, which return the launchable kernel of a configuration, type pair
// and operand layout.
#pragma once
#include "gemm_kernel.hpp"
#include "gemm_kernel_ring.hpp"

namespace tgemm {

// Tile-config tuples (block_M, block_N, block_K, waves, occupancy) in the
// spirit of the tuning tables of page "企业官网建设流程全解析", §3.3 / §4.4, and
// of the DeepSeek/Ascend TileLang toolkit page, §4.3, sized for gfx950:
// 160 KiB LDS per CU, 512 registers per lane at one wave per SIMD.
using CfgBig = TileCfg<256, 256, 64, 2, 2, 2, 1>;    // 4 waves, 128x128 per wave
using CfgMid = TileCfg<128, 128, 64, 2, 2, 2, 2>;    // 4 waves, 64x64 per wave
using CfgSmall = TileCfg<64, 64, 64, 2, 2, 2, 2>;    // 4 waves, 32x32 per wave
using CfgTiny = TileCfg<32, 32, 64, 1, 1, 2, 4>;     // 1 wave
using CfgF32Mid = TileCfg<64, 64, 32, 2, 2, 4, 2>;   // fp32 inputs
using CfgF32Tiny = TileCfg<32, 32, 32, 1, 1, 4, 4>;  // fp32 inputs, 1 wave
using CfgF32Big = TileCfg<128, 128, 32, 2, 2, 4, 2>; // fp32 inputs, 64x64 per wave
// direct-to-LDS ring kernels of the two largest tiles
using RingBig = RingCfg<256, 256, 2, 2, 1>;
using RingMid = RingCfg<128, 128, 2, 2, 2>;
// a ring-only configuration of 64 x 128 tiles (4 waves of 32 x 64): twice the
// workgroups of RingMid for products that leave CUs idle at 128 x 128
// (row-major A only)
using RingSmall = RingCfg<64, 128, 2, 2, 2>;

enum { CFG_BIG = 0, CFG_MID = 1, CFG_SMALL = 2, CFG_TINY = 3, CFG_F32_MID = 4, CFG_F32_TINY = 5,
       CFG_DIRECT = 6, CFG_F32_DIRECT = 7, CFG_RING_SMALL = 8, CFG_F32_BIG = 9, NUM_CONFIGS = 10 };

typedef void (*KernelFn)(GemmArgs);

// Register-staged kernel of configuration cfg (CFG_BIG .. CFG_F32_TINY, CFG_F32_BIG) for
// (in, out) (DT_* values); fast: the unchecked whole-tile path; epi: the
// fused epilogue (GemmArgs::epi ... act).  nullptr if the pair is not served.
// One definition per configuration (k_tiled_<cfg>.hip).
KernelFn tiled_kernel_big(int in, int out, bool fast, bool epi);
KernelFn tiled_kernel_mid(int in, int out, bool fast, bool epi);
KernelFn tiled_kernel_small(int in, int out, bool fast, bool epi);
KernelFn tiled_kernel_tiny(int in, int out, bool fast, bool epi);
KernelFn tiled_kernel_f32(int cfg, int in, int out, bool fast, bool epi);

// Ring kernel of CFG_BIG or CFG_MID for (in, out) and the layouts of A and B
// (LAYOUT_ROW / LAYOUT_COL); kt: the variant with the K tail (K not a
// multiple of 128).  k_ring_big.hip, k_ring_mid.hip.
KernelFn ring_kernel_big(int in, int out, int la, int lb, bool epi, bool kt);
KernelFn ring_kernel_mid(int in, int out, int la, int lb, bool epi, bool kt);
// RingSmall (k_ring_small.hip, k_ring_small_fused.hip): every variant
KernelFn ring_kernel_small(int in, int out, int la, int lb, bool epi, bool kt);
KernelFn ring_kernel_small_fused(int in, int out, int la, int lb, bool kt);

// The sum of the split-K slices with the call's epilogue, for output type
// out (DT_*): k_splitk.hip.  Arguments: the call's GemmArgs (C, ldc and the
// epilogue of the call), the workspace, its row stride in floats (a multiple
// of 4), floats per slice, and the number of slices.
typedef void (*SplitkReduceFn)(GemmArgs, const float*, int64_t, int64_t, int);
SplitkReduceFn splitk_reduce_kernel_for(int out);
// Threads per workgroup of that kernel, one group of 4 outputs each.
constexpr int kSplitkReduceThreads = 64;

// Direct kernel for (in, out), the layouts of A and B, and whether each
// operand takes 16-byte loads.  k_direct.hip.
KernelFn direct_kernel(int in, int out, int la, int lb, bool va, bool vb, bool epi);

// The fused-epilogue halves of the largest families, compiled in units of
// their own (k_*_fused.hip) so that the build runs them in parallel.
KernelFn tiled_kernel_big_fused(int in, int out, bool fast);
KernelFn ring_kernel_big_fused(int in, int out, int la, int lb, bool kt);
KernelFn ring_kernel_mid_fused(int in, int out, int la, int lb, bool kt);
KernelFn ring_kernel_big_kt(int in, int out, int la, int lb);
KernelFn ring_kernel_mid_kt(int in, int out, int la, int lb);
KernelFn ring_kernel_big_fused_kt(int in, int out, int la, int lb);
KernelFn ring_kernel_mid_fused_kt(int in, int out, int la, int lb);
KernelFn direct_kernel_fused(int in, int out, int la, int lb, bool va, bool vb);
// 8-bit float output (out == DT_FP8; always the fused epilogue's kernels):
// k_ring_big_fp8(_kt).hip, k_ring_mid_fp8.hip, k_ring_small_fp8.hip,
// k_direct_fp8.hip.  The selectors above forward to these.
KernelFn ring_kernel_big_fp8(int in, int la, int lb);
KernelFn ring_kernel_big_fp8_kt(int in, int la, int lb);
KernelFn ring_kernel_mid_fp8(int in, int la, int lb, bool kt);
KernelFn ring_kernel_small_fp8(int in, int la, int lb, bool kt);
KernelFn direct_kernel_fp8(int in, int la, int lb, bool va, bool vb);

}  // namespace tgemm
