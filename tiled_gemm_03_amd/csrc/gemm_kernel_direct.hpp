// gemm_kernel_direct.hpp -- the latency path of the tiled matrix product:
// small, ragged or unaligned products, every input type.
//
// For a product of a few tiles the time goes into memory round trips, not
// MFMA work: a workgroup that walks K through a few LDS stages pays one
// latency per stage.  Here each wave owns one 16 x 16 block of C (the output
// tile of page "企业官网建设流程全解析" §3.3 shrunk to one MFMA block; a
// workgroup is 2 x 2 waves, 32 x 32) and reads the MFMA operands straight
// from global memory into registers, with no LDS stage and no barrier in the
// K loop, through a
// ring of D register slots (2 to 8, as many as keep the loads in flight within
// what vmcnt counts): the loads of step s + D (steps of 32 of K) are issued
// when step s is computed.
//
// Operands (v_mfma_f32_16x16x32_{f16,bf16}; lane l, q = l / 16): row
// l % 16 of A and column l % 16 of B, k = 8q .. 8q+7 of the step.  An
// operand whose k is contiguous in memory (A row-major, B column-major; page
// "TileLang实战：用Python DSL自动生成高性能GPU计算内核" §5.1 for the two
// layouts) takes one 16-byte load when its rows are whole 16-byte chunks
// (VA / VB), else eight 16-bit loads; one whose k is strided takes eight
// 16-bit loads, each coalesced with the 15 neighbouring lanes (32 contiguous
// bytes).  fp32 inputs use v_mfma_f32_16x16x4f32 (lane l: row / column
// l % 16, k = q of each group of 4) and 4-byte loads.
//
// Ragged edges need no branches in the loop: buffer resources end at the
// operand's last element, so loads past it return zero; columns of B beyond
// N and rows of A beyond M only feed outputs that are never stored; elements
// with k >= K that lie inside an operand (padding, or the next row of a
// k-contiguous operand) are zeroed in the one partial step, so that no Inf or
// NaN stored there can meet a zero of the other operand.  The epilogue masks
// rows and columns of C (row-major).
//
// The MFMA takes B as its first operand and A as its second, so the
// accumulator holds C transposed: lane l owns row l % 16 and columns
// 4 q .. 4 q + 3 of the block.
//
// K split over the waves (p.splits == 4; else 1): when the steps of K are
// more than one ring holds but a quarter of them fits one, a workgroup
// computes one 16 x 16 block and its four waves take a quarter of the steps
// each (the partial last step to the fourth), all loads issued at once:
// one memory round trip instead of several.  The four partial blocks meet in
// LDS and the first wave adds them in wave order (the same order on every
// run) before the epilogue.  The sum is that of the unsplit kernel up to
// the order of the fp32 additions.

#pragma once
#include <type_traits>

#include "gemm_kernel.hpp"
#include "gemm_kernel_ring.hpp"  // LAYOUT_ROW / LAYOUT_COL

namespace tgemm {

typedef short s16x8 __attribute__((ext_vector_type(8)));

// Preconditions (checked by the host): for a k-contiguous operand
// (32 ld + K + 320) elements, for a k-strided one ((K + 320) ld + 32)
// elements below 2^31 bytes (buffer offsets, including the loads of the ring
// past K); VA / VB only for a k-contiguous 16-bit operand that is 16-byte
// aligned with ld % 8 == 0 and K % 8 == 0.  LA / LB: LAYOUT_ROW or LAYOUT_COL.
template <int IN, int OUT, int LA, int LB, bool VA, bool VB, bool EPI = false>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256))) void gemm_kernel_direct(GemmArgs p) {
    constexpr int EB = IN == DT_F32 ? 4 : 2;
    constexpr bool KCA = LA == LAYOUT_ROW, KCB = LB == LAYOUT_COL;  // k contiguous
    static_assert((!VA || (KCA && IN != DT_F32)) && (!VB || (KCB && IN != DT_F32)), "");
    // register ring depth (steps of 32 in flight): as many steps as keep the
    // outstanding loads within the 63 that vmcnt counts
    constexpr int LPS = IN == DT_F32 ? 16 : (VA ? 1 : 8) + (VB ? 1 : 8);  // loads per step
    constexpr int D = 63 / LPS < 2 ? 2 : 63 / LPS > 8 ? 8 : 63 / LPS;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int q = lane >> 4, l16 = lane & 15;

    const bool ks = p.splits == 4;  // K split over the waves, 16 x 16 tiles
    int tm, tn;
    tile_of(blockIdx.x, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
    const int m0 = ks ? tm * 16 : tm * 32 + 16 * (wave >> 1), n0 = ks ? tn * 16 : tn * 32 + 16 * (wave & 1);
    const int M = p.M, N = p.N, K = p.K;
    const int64_t lda = p.lda, ldb = p.ldb;

    auto rsrc = [&](const char* base, int64_t bytes) __attribute__((always_inline)) {
        const int n = bytes <= 0 ? 0 : bytes > 0x7fffffffLL ? 0x7fffffff : (int)bytes;
        return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, n, 0x00020000);
    };
    // Each operand from this wave's first row (A) / column (B), ending at the
    // operand's last element.  With K = 0 the operands hold no element (and
    // may be no allocation at all): empty ranges, and no load is issued.
    auto operand = [&](auto kc_t, const char* X, int64_t ld, int o0, int outer) __attribute__((always_inline)) {
        if (K <= 0) return rsrc(X, 0);
        if constexpr (decltype(kc_t)::value)   // element (o, k) at o * ld + k
            return rsrc(X + (int64_t)o0 * ld * EB, ((int64_t)(outer - 1 - o0) * ld + K) * EB);
        else                                    // element (o, k) at k * ld + o
            return rsrc(X + (int64_t)o0 * EB, ((int64_t)(K - 1) * ld + outer - o0) * EB);
    };
    const auto rs_a = operand(BoolTag<KCA>{}, p.A, lda, m0, M);
    const auto rs_b = operand(BoolTag<KCB>{}, p.B, ldb, n0, N);
    // byte offset of this lane's element (its row of A / column of B, k):
    // lane part + k * kstride
    const int a_lane = KCA ? (int)((int64_t)l16 * lda * EB) : l16 * EB;
    const int a_kstr = KCA ? EB : (int)(lda * EB);
    const int b_lane = KCB ? (int)((int64_t)l16 * ldb * EB) : l16 * EB;
    const int b_kstr = KCB ? EB : (int)(ldb * EB);
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
    auto load8 = [&](auto vec_t, const auto& rs, int lane_off, int kstr, int k0) __attribute__((always_inline)) {
        s16x8 v;
        if constexpr (decltype(vec_t)::value) {
            v = __builtin_bit_cast(s16x8, __builtin_amdgcn_raw_buffer_load_b128(rs, lane_off + k0 * EB, 0, 0));
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                v[e] = (short)__builtin_amdgcn_raw_buffer_load_b16(rs, lane_off + (k0 + e) * kstr, 0, 0);
        }
        return v;
    };
    auto load_step = [&](Frag& f, int s) __attribute__((always_inline)) {
        if constexpr (IN == DT_F32) {
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int k = s * 32 + 4 * u + q;
                f.fa[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs_a, a_lane + k * a_kstr, 0, 0));
                f.fb[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs_b, b_lane + k * b_kstr, 0, 0));
            }
        } else {
            const int k0 = s * 32 + 8 * q;
            f.a = load8(BoolTag<VA>{}, rs_a, a_lane, a_kstr, k0);
            f.b = load8(BoolTag<VB>{}, rs_b, b_lane, b_kstr, k0);
        }
    };
    // MASK: elements with k >= K are taken as zero (the partial last step)
    auto mma_step = [&](auto mask_t, const Frag& f, int s) __attribute__((always_inline)) {
        constexpr bool MASK = decltype(mask_t)::value;
        if constexpr (IN == DT_F32) {
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                float a = f.fa[u], b = f.fb[u];
                if constexpr (MASK) {
                    const bool in = s * 32 + 4 * u + q < K;
                    a = in ? a : 0.f;
                    b = in ? b : 0.f;
                }
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(b, a, acc, 0, 0, 0);
            }
        } else {
            s16x8 a = f.a, b = f.b;
            if constexpr (MASK) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const bool in = s * 32 + 8 * q + e < K;
                    a[e] = in ? a[e] : (short)0;
                    b[e] = in ? b[e] : (short)0;
                }
            }
            if constexpr (IN == DT_F16)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, b), __builtin_bit_cast(f16x8, a),
                                                             acc, 0, 0, 0);
            else
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, b),
                                                              __builtin_bit_cast(bf16x8, a), acc, 0, 0, 0);
        }
    };
    constexpr BoolTag<false> nomask{};
    constexpr BoolTag<true> mask{};

    // Full steps through a ring of D register slots: the loads of step s + D
    // are issued when step s is computed.  Loads past the last full step read
    // zeros or in-bounds data that is never used.
    const int nfull = K / 32;
    if (K > 0 && ks) {
        // this wave's steps [s0, s1), at most D (the host's condition), and
        // the fourth wave's partial step: every load issued before the first
        // MFMA
        const int quarter = (nfull + 3) / 4;
        const int s0 = wave * quarter < nfull ? wave * quarter : nfull;
        const int s1 = s0 + quarter < nfull ? s0 + quarter : nfull;
        const bool tail = K % 32 != 0 && wave == 3;
        Frag ring[D], f;
#pragma unroll
        for (int t = 0; t < D; ++t)
            if (s0 + t < s1) load_step(ring[t], s0 + t);
        if (tail) load_step(f, nfull);
#pragma unroll
        for (int t = 0; t < D; ++t)
            if (s0 + t < s1) mma_step(nomask, ring[t], s0 + t);
        if (tail) mma_step(mask, f, nfull);
    } else if (K > 0) {
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
        // the partial last step: elements past K are zeroed
        if (K % 32 != 0) {
            Frag f;
            load_step(f, nfull);
            mma_step(mask, f, nfull);
        }
    }

    if (ks) {  // the waves' partial blocks, added by the first wave
        __shared__ f32x4 part[3][64];
        if (wave > 0) part[wave - 1][lane] = acc;
        __syncthreads();
        if (wave > 0) return;
        acc += part[0][lane];
        acc += part[1][lane];
        acc += part[2][lane];
    }

    // epilogue: row m0 + l%16, columns n0 + 4q .. +3; fp32 -> fp16 / bf16
    // rounds to nearest even
    constexpr int OB = out_bytes<OUT>();
    const int row = m0 + l16, col = n0 + 4 * q;
    if constexpr (EPI) {
        // fused epilogue (one block per wave: no staging needed)
        const int n = row < M ? (N - col >= 4 ? 4 : N - col > 0 ? N - col : 0) : 0;
        if (n > 0) store4_fused<OUT>(p, row, col, n, p.vec_c != 0, acc);
        return;
    }
    if (row < M) {
        char* dst = p.C + ((int64_t)row * p.ldc + col) * OB;
        if (col + 4 <= N) {
            store4<OUT>(dst, acc[0], acc[1], acc[2], acc[3], p.vec_c != 0);
        } else {
            if (col + 0 < N) store_elem<OUT>(dst + 0 * OB, acc[0]);
            if (col + 1 < N) store_elem<OUT>(dst + 1 * OB, acc[1]);
            if (col + 2 < N) store_elem<OUT>(dst + 2 * OB, acc[2]);
            if (col + 3 < N) store_elem<OUT>(dst + 3 * OB, acc[3]);
        }
    }
}

}  // namespace tgemm
