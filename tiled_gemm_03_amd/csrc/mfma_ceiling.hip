// mfma_ceiling.hip -- measures what the matrix cores of one MI355X sustain
// for the two fp16 MFMA shapes the kernels use, with no memory traffic:
// every SIMD runs independent v_mfma_f32_32x32x16_f16 or
// v_mfma_f32_16x16x32_f16 chains whose operands change every instruction,
// taken from N(0,1) or all-ones fp16 data.  The shader clock is read inside
// the kernel (s_memtime against the 100 MHz s_memrealtime).
//
// It is the practical ceiling that a matrix-product kernel on this part is
// measured against besides the published peak: at the board's power cap the
// clock, and so the ceiling, depends on the MFMA shape and on the data.
// Output: one JSON object per line.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <vector>

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

#define CHECK(x)                                                                         \
    do {                                                                                 \
        hipError_t e_ = (x);                                                             \
        if (e_ != hipSuccess) {                                                          \
            fprintf(stderr, "mfma_ceiling: %s at line %d\n", hipGetErrorString(e_), __LINE__); \
            exit(1);                                                                     \
        }                                                                                \
    } while (0)

namespace {

constexpr int kWavesPerBlock = 4;
constexpr int kBlocks = 1024;         // 4 rounds of one workgroup per CU on 256 CUs
constexpr int kOperandSets = 64;      // distinct operand sets (per wave slot)

__device__ uint32_t mix(uint32_t x) {
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    x ^= x >> 16;
    return x;
}

// N(0,1) by Box-Muller over a counter hash, or all ones
__global__ void fill(_Float16* p, int n, int ones) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const float u1 = (mix(2u * i + 1u) + 1.0f) * 2.3283064e-10f;
    const float u2 = mix(2u * i + 2u) * 2.3283064e-10f;
    p[i] = ones ? (_Float16)1.0f : (_Float16)(sqrtf(-2.0f * logf(u1)) * cosf(6.2831853f * u2));
}

// SHAPE 0: 32x32x16 (16 accumulators of 16), SHAPE 1: 16x16x32 (64 of 4).
// Each iteration of the outer loop issues 8 x NA MFMAs; both shapes do the
// same FLOP per iteration of `iters` (16x16x32 runs iters / 2).
template <int SHAPE>
__global__ __launch_bounds__(256) void mfma_loop(const f16x8* ops, float* out, int iters, uint64_t* clk) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    f16x8 a[8], b[8];
    const f16x8* src = ops + ((blockIdx.x * kWavesPerBlock + wave) % kOperandSets) * 1024;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = src[i * 64 + lane];
        b[i] = src[512 + i * 64 + lane];
    }
    float s = 0.f;
    if constexpr (SHAPE == 0) {
        f32x16 acc[16];
#pragma unroll
        for (int i = 0; i < 16; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
        for (int it = 0; it < iters; it += 8) {
#pragma unroll
            for (int u = 0; u < 8; ++u)
#pragma unroll
                for (int m = 0; m < 16; ++m)
                    acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_f16(b[m % 8], a[(m / 4 + u) % 8], acc[m], 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) s += acc[i][r];
    } else {
        f32x4 acc[64];
#pragma unroll
        for (int i = 0; i < 64; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[i][r] = 0.f;
        for (int it = 0; it < iters; it += 8) {
#pragma unroll
            for (int u = 0; u < 8; ++u)
#pragma unroll
                for (int m = 0; m < 64; ++m)
                    acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(b[m % 8], a[(m / 8 + u) % 8], acc[m], 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 64; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) s += acc[i][r];
    }
    out[blockIdx.x * 256 + threadIdx.x] = s;
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    if (threadIdx.x == 0) {
        clk[blockIdx.x * 4 + 0] = t0;
        clk[blockIdx.x * 4 + 1] = t1;
        clk[blockIdx.x * 4 + 2] = r0;
        clk[blockIdx.x * 4 + 3] = r1;
    }
}

}  // namespace

int main(int argc, char** argv) {
    const int iters = argc > 1 ? atoi(argv[1]) : 4000;  // a multiple of 16
    if (iters <= 0 || iters % 16 != 0) {
        fprintf(stderr, "mfma_ceiling: iterations must be a positive multiple of 16\n");
        return 2;
    }
    const int n_ops = kOperandSets * 1024 * 8;  // halves: 64 sets x 1024 vectors of 8
    _Float16 *ops_randn, *ops_ones;
    float* out;
    uint64_t* clk;
    CHECK(hipMalloc(&ops_randn, n_ops * sizeof(_Float16)));
    CHECK(hipMalloc(&ops_ones, n_ops * sizeof(_Float16)));
    CHECK(hipMalloc(&out, kBlocks * 256 * sizeof(float)));
    CHECK(hipMalloc(&clk, kBlocks * 4 * sizeof(uint64_t)));
    fill<<<n_ops / 256, 256>>>(ops_randn, n_ops, 0);
    fill<<<n_ops / 256, 256>>>(ops_ones, n_ops, 1);
    CHECK(hipGetLastError());
    CHECK(hipDeviceSynchronize());
    hipEvent_t e0, e1;
    CHECK(hipEventCreate(&e0));
    CHECK(hipEventCreate(&e1));
    const double flop = (double)kBlocks * kWavesPerBlock * iters * 16 * 32768.0;
    for (int shape = 0; shape < 2; ++shape)
        for (int ones = 0; ones < 2; ++ones) {
            const f16x8* o = (const f16x8*)(ones ? ops_ones : ops_randn);
            auto launch = [&]() {
                if (shape == 0) mfma_loop<0><<<kBlocks, 256>>>(o, out, iters, clk);
                else mfma_loop<1><<<kBlocks, 256>>>(o, out, iters / 2, clk);
            };
            launch();
            launch();
            CHECK(hipGetLastError());
            CHECK(hipDeviceSynchronize());
            const int reps = 5;
            CHECK(hipEventRecord(e0));
            for (int r = 0; r < reps; ++r) launch();
            CHECK(hipEventRecord(e1));
            CHECK(hipEventSynchronize(e1));
            float ms = 0.f;
            CHECK(hipEventElapsedTime(&ms, e0, e1));
            ms /= reps;
            std::vector<uint64_t> h(kBlocks * 4);
            CHECK(hipMemcpy(h.data(), clk, h.size() * sizeof(uint64_t), hipMemcpyDeviceToHost));
            double ghz = 0.0;
            for (int b = 0; b < kBlocks; ++b)
                ghz += (double)(h[b * 4 + 1] - h[b * 4]) / (double)(h[b * 4 + 3] - h[b * 4 + 2]) * 0.1;
            ghz /= kBlocks;
            const double tflops = flop / (ms * 1e-3) / 1e12;
            // dense fp16 rate at that clock: 1024 SIMDs x 1024 FLOP per cycle
            const double ceiling = 1024.0 * 1024.0 * ghz * 1e9 / 1e12;
            printf("{\"mfma\": \"%s\", \"data\": \"%s\", \"ms\": %.4f, \"tflops\": %.1f, \"sclk_ghz\": %.3f, "
                   "\"dense_rate_at_sclk_tflops\": %.1f, \"issue_efficiency\": %.3f}\n",
                   shape == 0 ? "v_mfma_f32_32x32x16_f16" : "v_mfma_f32_16x16x32_f16", ones ? "ones" : "N(0,1)", ms,
                   tflops, ghz, ceiling, tflops / ceiling);
            fflush(stdout);
        }
    return 0;
}
