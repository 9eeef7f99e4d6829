// gemm_kernel_direct.hpp -- the latency path of the tiled matrix product:
// small, ragged or unaligned products, every input type.
//
// For a product of a few tiles the time goes into memory round trips, not
// MFMA work: a workgroup that walks K through a few LDS stages pays one
// latency per stage.  Here each wave owns one 16 x 16 block of C (the output
// tile of page "企业官网建设流程全解析" §3.3 shrunk to one MFMA block; a
// workgroup is 2 x 2 waves, 32 x 32) and reads the MFMA operands straight
// from global memory into registers, with no LDS and no barrier, through a
// ring of D register slots: the loads of step s + D (steps of 32 of K) are
// issued when step s is computed.
//
// Operands (v_mfma_f32_16x16x32_{f16,bf16}; lane l, q = l / 16):
//   A: row l % 16, k = 8q .. 8q+7 of the step: one 16-byte load when rows
//      are whole 16-byte chunks (AVEC), else eight 16-bit loads;
//   B: column l % 16, k = 8q .. 8q+7: eight 16-bit loads, each coalesced
//      with the 15 neighbouring lanes (32 contiguous bytes of one row).
// fp32 inputs use v_mfma_f32_16x16x4f32 (lane l: row / column l % 16,
// k = q of each group of 4), 4-byte loads, chunks of 4 steps.
//
// Ragged edges need no branches in the loop: buffer resources end at the
// operand's last element, so loads past it return zero (rows of A beyond M,
// rows of B beyond K); columns of B beyond N and rows of A beyond M only feed
// outputs that are never stored; the elements of A with k >= K (inside the
// matrix: padding or the next row) are zeroed in the last step, so that no
// Inf or NaN stored there can meet a zero of B.  The epilogue masks rows and
// columns.
//
// The MFMA takes B as its first operand and A as its second, so the
// accumulator holds C transposed: lane l owns row l % 16 and columns
// 4 q .. 4 q + 3 of the block.

#pragma once
#include <type_traits>

#include "gemm_kernel.hpp"

namespace tgemm {

typedef short s16x8 __attribute__((ext_vector_type(8)));

// Preconditions (checked by the host): 32 lda + K + 320 elements and
// (K + 320) ldb elements below 2^31 bytes (buffer offsets, including the
// loads of the ring past K); with AVEC, A 16-byte aligned, lda % 8 == 0 and
// K % 8 == 0.
template <int IN, int OUT, bool AVEC>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256))) void gemm_kernel_direct(GemmArgs p) {
    constexpr int EB = IN == DT_F32 ? 4 : 2;
    // register ring depth (steps of 32 in flight); shallower when A takes
    // eight loads per step, to stay within the 63 loads vmcnt can count
    constexpr int D = (IN != DT_F32 && !AVEC) ? 4 : 8;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int q = lane >> 4, l16 = lane & 15;

    int tm, tn;
    tile_of(blockIdx.x, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
    const int m0 = tm * 32 + 16 * (wave >> 1), n0 = tn * 32 + 16 * (wave & 1);
    const int M = p.M, N = p.N, K = p.K;
    const int64_t lda = p.lda, ldb = p.ldb;

    auto rsrc = [&](const char* base, int64_t bytes) __attribute__((always_inline)) {
        const int n = bytes <= 0 ? 0 : bytes > 0x7fffffffLL ? 0x7fffffff : (int)bytes;
        return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, n, 0x00020000);
    };
    // A from this wave's first row, B from its first column; both end at the
    // operand's last element.  With K = 0 the operands hold no element (and
    // may be no allocation at all): empty ranges, and no load is issued.
    const auto rs_a = rsrc(p.A + (int64_t)m0 * lda * EB, K > 0 ? ((int64_t)(M - 1 - m0) * lda + K) * EB : 0);
    const auto rs_b = rsrc(p.B + (int64_t)n0 * EB, K > 0 ? ((int64_t)(K - 1) * ldb + N - n0) * EB : 0);
    const int a_row = (int)((int64_t)l16 * lda * EB);   // this lane's A row
    const int b_col = l16 * EB;                         // this lane's B column
    const int b_rstep = (int)(ldb * EB);                // one row of B

    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};

    // One step = 32 of K.  Operand registers of one step (lane l, q = l/16):
    //  16-bit: A 8 consecutive k of row l%16 (k = 8q ..), B the same k of
    //          column l%16; one v_mfma_f32_16x16x32;
    //  fp32:   8 MFMAs of k = 4; A and B hold k = 4u + q for u = 0..7.
    struct Frag {
        // 16-bit: a (8 k of one row of A), b (8 k of one column of B);
        // fp32: fa, fb (k = 4u + q, u = 0..7)
        s16x8 a, b;
        float fa[8], fb[8];
    };
    auto load_step = [&](Frag& f, int s) __attribute__((always_inline)) {
        if constexpr (IN == DT_F32) {
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int k = s * 32 + 4 * u + q;
                f.fa[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs_a, a_row + k * 4, 0, 0));
                f.fb[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs_b, b_col + k * b_rstep, 0, 0));
            }
        } else {
            const int k0 = s * 32 + 8 * q;
            if constexpr (AVEC) {
                f.a = __builtin_bit_cast(s16x8, __builtin_amdgcn_raw_buffer_load_b128(rs_a, a_row + k0 * EB, 0, 0));
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    f.a[e] = (short)__builtin_amdgcn_raw_buffer_load_b16(rs_a, a_row + (k0 + e) * EB, 0, 0);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e)
                f.b[e] = (short)__builtin_amdgcn_raw_buffer_load_b16(rs_b, b_col + (k0 + e) * b_rstep, 0, 0);
        }
    };
    // MASK: elements of A with k >= K are taken as zero (the partial last step)
    auto mma_step = [&](auto mask_t, const Frag& f, int s) __attribute__((always_inline)) {
        constexpr bool MASK = decltype(mask_t)::value;
        if constexpr (IN == DT_F32) {
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                float a = f.fa[u];
                if constexpr (MASK) a = s * 32 + 4 * u + q < K ? a : 0.f;
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(f.fb[u], a, acc, 0, 0, 0);
            }
        } else {
            s16x8 a = f.a;
            if constexpr (MASK) {
#pragma unroll
                for (int e = 0; e < 8; ++e) a[e] = s * 32 + 8 * q + e < K ? a[e] : (short)0;
            }
            if constexpr (IN == DT_F16)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, f.b), __builtin_bit_cast(f16x8, a),
                                                             acc, 0, 0, 0);
            else
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, f.b),
                                                              __builtin_bit_cast(bf16x8, a), acc, 0, 0, 0);
        }
    };
    constexpr BoolTag<false> nomask{};
    constexpr BoolTag<true> mask{};

    // Full steps through a ring of D register slots: the loads of step s + D
    // are issued when step s is computed.  Loads past the last full step read
    // zeros or in-bounds data that is never used.
    const int nfull = K / 32;
    if (K > 0) {
        Frag ring[D];
#pragma unroll
        for (int t = 0; t < D; ++t) load_step(ring[t], t);
        int s = 0;
        for (; s + D <= nfull; s += D) {
#pragma unroll
            for (int t = 0; t < D; ++t) {
                mma_step(nomask, ring[t], s + t);
                load_step(ring[t], s + D + t);
            }
        }
        // the remaining full steps are already in the ring
#pragma unroll
        for (int t = 0; t < D; ++t)
            if (s + t < nfull) mma_step(nomask, ring[t], s + t);
        // the partial last step: elements of A past K are zeroed (B reads
        // zeros there, outside its range)
        if (K % 32 != 0) {
            Frag f;
            load_step(f, nfull);
            mma_step(mask, f, nfull);
        }
    }

    // epilogue: row m0 + l%16, columns n0 + 4q .. +3; fp32 -> fp16 / bf16
    // rounds to nearest even
    constexpr int OB = OUT == DT_F32 ? 4 : 2;
    const int row = m0 + l16, col = n0 + 4 * q;
    if (row < M) {
        char* dst = p.C + ((int64_t)row * p.ldc + col) * OB;
        if (p.vec_c && col + 4 <= N) {
            store4<OUT>(dst, acc[0], acc[1], acc[2], acc[3], true);
        } else {
            if (col + 0 < N) store_elem<OUT>(dst + 0 * OB, acc[0]);
            if (col + 1 < N) store_elem<OUT>(dst + 1 * OB, acc[1]);
            if (col + 2 < N) store_elem<OUT>(dst + 2 * OB, acc[2]);
            if (col + 3 < N) store_elem<OUT>(dst + 3 * OB, acc[3]);
        }
    }
}

}  // namespace tgemm
