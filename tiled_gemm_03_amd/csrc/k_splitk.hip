// k_splitk.hip -- the sum of the split-K slices.  For a product with too few
// output tiles to occupy the CUs and a long K, the ring kernel runs S slices
// of K as S times the workgroups, each writing its fp32 partial tile to a
// slice of a workspace (the product is a sum over k, so partial sums over
// disjoint ranges of k add up to it; page "企业官网建设流程全解析" §3.3
// defines C as that sum).  This kernel adds the S partials of each group of 4
// outputs in slice order (the same order on every run) and applies the
// epilogue of the call: the fused one (alpha, beta C, bias, activation) or
// the identity, and the output rounding, with the stores of any C alignment.
#include "kernels.hpp"

namespace tgemm {

// One wave per workgroup: a skinny product's few output groups still spread
// over every CU.  The loads of eight slices are issued together and added in
// slice order afterwards, so the memory latency is paid once per eight
// slices and the sum is the same as slice by slice.
template <int OUT>
__global__ __launch_bounds__(kSplitkReduceThreads) void splitk_reduce_kernel(GemmArgs p, const float* w, int64_t ldw,
                                                                             int64_t slice, int splits) {
    const int64_t groups = ((int64_t)p.N + 3) / 4;  // of each row
    const int64_t gid = (int64_t)blockIdx.x * kSplitkReduceThreads + threadIdx.x;
    if (gid >= (int64_t)p.M * groups) return;
    const int row = (int)(gid / groups), col = (int)(gid - (int64_t)row * groups) * 4;
    const float* src = w + (int64_t)row * ldw + col;  // ldw % 4 == 0: 16-byte aligned groups
    f32x4 acc = *(const f32x4*)src;
    for (int s = 1; s < splits; s += 8) {
        f32x4 v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (s + j < splits) v[j] = *(const f32x4*)(src + (s + j) * slice);
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (s + j < splits) acc += v[j];
    }
    const int n = p.N - col < 4 ? p.N - col : 4;
    store4_fused<OUT>(p, row, col, n, p.vec_c != 0 && n == 4, acc);
}

SplitkReduceFn splitk_reduce_kernel_for(int out) {
    switch (out) {
        case DT_F16: return splitk_reduce_kernel<DT_F16>;
        case DT_BF16: return splitk_reduce_kernel<DT_BF16>;
        case DT_F32: return splitk_reduce_kernel<DT_F32>;
        case DT_FP8: return splitk_reduce_kernel<DT_FP8>;
        default: return nullptr;
    }
}

}  // namespace tgemm
