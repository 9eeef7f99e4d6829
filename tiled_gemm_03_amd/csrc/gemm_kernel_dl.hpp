// gemm_kernel_dl.hpp -- the gfx950 direct-to-LDS variant of the tiled
// matrix-product kernel, for 16-bit inputs (fp16 / bf16) on whole tiles.
//
// Same method as gemm_kernel.hpp (one workgroup per BM x BN tile of C, K
// walked in BK steps through a two-stage LDS pipeline, fp32 MFMA
// accumulators), with the two data paths gfx950 adds:
//
//  * global -> LDS without registers: buffer_load_dwordx4 ... lds writes the
//    16 bytes of lane l of a wave at LDS byte M0 + 16 l, so one instruction
//    fills a 1 KiB block.  The XOR swizzle of the LDS layout is obtained by
//    choosing, per lane, which global 16-byte chunk lands in which slot.
//    No staging registers, no ds_write, no register transpose.
//  * B stays k-major in LDS (rows of BN elements) and its MFMA operand is
//    read with ds_read_b64_tr_b16: in each group of 16 lanes, lane i points
//    at 4 consecutive columns of row i/4 and receives element i%4 of the
//    loads of lanes i/4, i/4+4, i/4+8, i/4+12, i.e. one column of a 4-row
//    block.  Two such reads give the 8 k-consecutive values of one column
//    that v_mfma_f32_32x32x16_{f16,bf16} takes per lane.
//
// LDS layouts (per stage):
//   A: BM rows x BK (128-byte rows), 16-byte chunk c of row r stored at
//      chunk c ^ (r%8 ^ (r/8)%2)        -- as in gemm_kernel.hpp
//   B: BK rows x BN (2*BN-byte rows), 16-byte chunk c of k-row r stored at
//      chunk c ^ 4*(r%4): the 16 lanes of one transposing read (4 rows x 2
//      chunks) and the 32 lanes of a half wave (4 rows x 4 chunks) then
//      touch 16 different 16-byte bank groups.
//
// Schedule of one K step s (k-groups of 16 K, NKG = BK/16 of them): the
// MFMAs of group g run while the fragments of group g+1 are read; group 0
// also issues the B loads of step s+1; then the wave waits for its
// outstanding global->LDS loads, all waves meet at the barrier, and the MFMAs
// of the last group overlap the reads of the next step's first fragments and
// the A loads of step s+2 into the stage just released.

#pragma once
#include "gemm_kernel.hpp"

namespace tgemm {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt that limits only the vector-memory counter, to N outstanding
// (gfx9 encoding: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[15:14]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Tile configuration of the direct-to-LDS kernel: BM x BN x BK, WM x WN
// waves, 16-bit inputs.
template <int BM_, int BN_, int BK_, int WM_, int WN_>
struct DlCfg {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_;
    static constexpr int THREADS = 64 * WM * WN, WAVES = WM * WN;
    static constexpr int EB = 2;
    static constexpr int RA = BK * 2;               // bytes per A row in LDS
    static constexpr int RBB = BN * 2;              // bytes per B k-row in LDS
    static constexpr int CA = RA / 16, CB = RBB / 16;   // 16-byte chunks per row
    static constexpr int A_BYTES = BM * RA, B_BYTES = BK * RBB;
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    static constexpr int LDS_BYTES = 2 * STAGE_BYTES;
    static constexpr int A_BLOCKS = A_BYTES / 1024, B_BLOCKS = B_BYTES / 1024;  // 1 KiB loads
    static constexpr int A_LOADS = A_BLOCKS / WAVES, B_LOADS = B_BLOCKS / WAVES;  // per wave
    static constexpr int A_ROWS_PER_BLOCK = 1024 / RA, B_ROWS_PER_BLOCK = 1024 / RBB;
    static constexpr int WTM = BM / WM, WTN = BN / WN;
    static constexpr int FM = WTM / 32, FN = WTN / 32;
    static constexpr int NKG = BK / 16;
    static_assert(CA == 8, "A rows of 128 bytes (BK = 64)");
    static_assert(CB >= 16 && 1024 % RBB == 0, "B rows of 256 or 512 bytes");
    static_assert(A_BLOCKS % WAVES == 0 && B_BLOCKS % WAVES == 0, "");
    static_assert(LDS_BYTES <= 160 * 1024, "");
    static_assert(WTM % 32 == 0 && WTN % 32 == 0 && NKG >= 2, "");
};

// Preconditions (checked by the host): 16-bit inputs, M % BM == 0,
// N % BN == 0, K % BK == 0, A and B 16-byte aligned, lda and ldb multiples of
// 8, the buffer offsets of one tile (BM rows of A, BK rows of B) below 2^31,
// C aligned for 4-element stores (ldc % 4 == 0).
template <class T, int IN, int OUT>
__global__ __attribute__((amdgpu_flat_work_group_size(T::THREADS, T::THREADS), amdgpu_waves_per_eu(1)))
void gemm_kernel_dl(GemmArgs p) {
    __shared__ __attribute__((aligned(1024))) char smem[T::LDS_BYTES];
    // LDS byte address of smem (the M0 value of direct-to-LDS loads)
    const int smem_base = (int)(uintptr_t)(lds_void*)smem;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / T::WN, wn = wave % T::WN;

    int tm, tn;
    tile_of(blockIdx.x, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
    const int m0 = tm * T::BM, n0 = tn * T::BN;
    const int K = p.K;
    const int64_t lda = p.lda, ldb = p.ldb;
    const int swz = p.swz_mask != 0;  // 1: swizzled layouts, 0: plain (A/B runs)

    // ---------------------------------------------------------- a2: loads
    // A block b (rows b*8 .. b*8+7): lane l fills slot l = (row l/8, chunk
    // l%8) with logical chunk (l%8) ^ (l/8) ^ (b%2).
    // B block b (rows b*RPB ..): lane l fills slot (row l/CB, chunk l%CB)
    // with logical chunk (l%CB) ^ 4*(row%4).
    int a_voff[2], b_voff[2];
#pragma unroll
    for (int par = 0; par < 2; ++par) {
        const int ar = lane / 8;
        const int ac = swz ? ((lane % 8) ^ ar ^ par) : (lane % 8);
        a_voff[par] = (int)(((int64_t)ar * lda + ac * 8) * 2);
        const int br = lane / T::CB;
        const int krow = par * T::B_ROWS_PER_BLOCK + br;  // block parity decides row%4 for 2-row blocks
        const int bc = swz ? ((lane % T::CB) ^ (4 * (krow % 4))) : (lane % T::CB);
        b_voff[par] = (int)(((int64_t)br * ldb + bc * 8) * 2);
    }
    // load x of this wave for the K step at k0 into `stage`: x < A_LOADS is
    // A block wave*A_LOADS + x, otherwise B block wave*B_LOADS + x - A_LOADS.
    // Issued through inline asm (M0 = LDS destination, then the load): the
    // compiler then does not guard later LDS reads with a wait for these
    // loads; the kernel waits for them itself (vmcnt) before the barrier that
    // publishes the stage.
    auto rsrc = [&](const char* base) {
        const uint64_t a = (uint64_t)base;
        return i32x4{__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
                     __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32)), -1, 0x00020000};
    };
    auto issue_load = [&](int k0, int stage, int x) {
        const int st_off = stage * T::STAGE_BYTES;
        int lds_addr, voff, soff;
        i32x4 rs;
        if (x < T::A_LOADS) {
            const int blk = wave * T::A_LOADS + x;
            rs = rsrc(p.A + ((int64_t)m0 * lda + k0) * 2);
            soff = (int)((int64_t)blk * T::A_ROWS_PER_BLOCK * lda * 2);
            voff = a_voff[blk & 1];
            lds_addr = smem_base + st_off + blk * 1024;
        } else {
            const int blk = wave * T::B_LOADS + (x - T::A_LOADS);
            rs = rsrc(p.B + ((int64_t)k0 * ldb + n0) * 2);
            soff = (int)((int64_t)blk * T::B_ROWS_PER_BLOCK * ldb * 2);
            voff = b_voff[T::B_ROWS_PER_BLOCK == 2 ? (blk & 1) : 0];
            lds_addr = smem_base + st_off + T::A_BYTES + blk * 1024;
        }
        asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                     :
                     : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(voff), "s"(rs),
                       "s"(__builtin_amdgcn_readfirstlane(soff))
                     : "memory");
    };
    auto issue_loads = [&](int k0, int stage) {
        static_for<0, T::A_LOADS + T::B_LOADS>([&](auto x) { issue_load(k0, stage, decltype(x)::value); });
    };

    // ---------------------------------------------------------- a5: fragments
    const int l32 = lane & 31, h = lane >> 5;
    // A: row wm*WTM + 32 i + l32, chunk 2g + h, stored at chunk (2g + h) ^ key
    const int a_row = wm * T::WTM + l32;
    const int a_key = swz ? ((a_row % 8) ^ ((a_row / 8) % 2)) : 0;
    const int a_base = a_row * T::RA;
    // B: group q = lane/16, i = lane%16: k-row 16g + 8h + 4r + i/4, columns
    // n = wn*WTN + 32 j + 16 (q%2) + 4 (i%4) .. +3
    const int q = lane >> 4, i16 = lane & 15;
    const int bx = i16 >> 2;                      // row within the 4-row block; swizzle key bx*4
    const int b_rowoff = (8 * h + bx) * T::RBB;
    const int b_sub = 2 * (q & 1) + ((i16 & 3) >> 1);  // chunk within the 32-column block
    const int b_half = 8 * (i16 & 1);                  // byte offset within the chunk
    int b_coloff[T::FN];
#pragma unroll
    for (int j = 0; j < T::FN; ++j) {
        const int c = (wn * T::WTN + 32 * j) / 8 + b_sub;
        b_coloff[j] = b_rowoff + (swz ? (c ^ (4 * bx)) : c) * 16 + b_half;
    }

    i16x4 fb[2][T::FN][2];
    u32x4 fa[2][T::FM];
    constexpr int NREAD = T::FM + 2 * T::FN;

    auto read_frag = [&](int stage, int g, int buf, int r) {
        const char* As = smem + stage * T::STAGE_BYTES;
        const char* Bs = As + T::A_BYTES;
        if (r < T::FM) {
            const int chunk = swz ? ((2 * g + h) ^ a_key) : (2 * g + h);
            fa[buf][r] = *(const u32x4*)(As + a_base + 32 * r * T::RA + chunk * 16);
        } else {
            const int j = (r - T::FM) / 2, half = (r - T::FM) % 2;
            fb[buf][j][half] =
                __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(Bs + b_coloff[j] + (16 * g + 4 * half) * T::RBB));
        }
    };

    f32x16 acc[T::FM][T::FN];
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int j = 0; j < T::FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    constexpr int NMF = T::FM * T::FN;
    auto mfma_one = [&](int buf, int m) {
        const int i = m / T::FN, j = m % T::FN;
        typedef short i16x8 __attribute__((ext_vector_type(8)));
        const i16x8 bop = __builtin_shufflevector(fb[buf][j][0], fb[buf][j][1], 0, 1, 2, 3, 4, 5, 6, 7);
        if constexpr (IN == DT_F16) {
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, bop),
                                                                __builtin_bit_cast(f16x8, fa[buf][i]), acc[i][j], 0, 0, 0);
        } else {
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, bop),
                                                                 __builtin_bit_cast(bf16x8, fa[buf][i]), acc[i][j], 0, 0, 0);
        }
    };

    // One K step on LDS stage `cur`.  LOAD_A: after the barrier, issue the A
    // loads of step s+2 (k0 = k_a) into `cur`, just released.  LOAD_B: in
    // k-group 0, issue the B loads of step s+1 (k0 = k_b) into the other
    // stage (released at the previous barrier); splitting the loads of a step
    // over two k-groups keeps the wave's memory queue from filling up.
    // NEXT: read the next step's first fragments after the barrier.
    auto kstep = [&](auto loada_tag, auto loadb_tag, auto next_tag, int cur, int k_a, int k_b) {
        constexpr bool LOAD_A = decltype(loada_tag)::value;
        constexpr bool LOAD_B = decltype(loadb_tag)::value;
        constexpr bool NEXT = decltype(next_tag)::value;
        constexpr int NKG = T::NKG;
        const int nxt = cur ^ 1;
        static_for<0, NKG>([&](auto gt) {
            constexpr int g = decltype(gt)::value;
            constexpr bool last = g == NKG - 1;
            if constexpr (last) {
                wait_vmcnt<0>();
                __syncthreads();
            }
            constexpr int n_read = last ? (NEXT ? NREAD : 0) : NREAD;
            constexpr int n_load = (last && LOAD_A) ? T::A_LOADS : ((g == 0 && LOAD_B) ? T::B_LOADS : 0);
            constexpr int n_work = n_read + n_load;
            static_for<0, NMF>([&](auto mt) {
                constexpr int m = decltype(mt)::value;
                mfma_one(g & 1, m);
                constexpr int wb = (m * n_work + NMF - 1) / NMF;
                constexpr int we = ((m + 1) * n_work + NMF - 1) / NMF;
                static_for<wb, we>([&](auto wt) {
                    constexpr int w = decltype(wt)::value;
                    if constexpr (w < n_read) {
                        if constexpr (last) read_frag(nxt, 0, 0, w);
                        else read_frag(cur, g + 1, (g + 1) & 1, w);
                    } else if constexpr (last) {
                        issue_load(k_a, cur, w - n_read);
                    } else {
                        issue_load(k_b, nxt, T::A_LOADS + (w - n_read));
                    }
                });
                __builtin_amdgcn_sched_barrier(0);
            });
        });
    };

    const int nk = K / T::BK;
    if (nk > 0) {
        constexpr BoolTag<true> yes{};
        constexpr BoolTag<false> no{};
        // step 0 whole, A of step 1; B of step 1 goes out in step 0's group 0
        issue_loads(0, 0);
        if (nk > 1) {
            static_for<0, T::A_LOADS>([&](auto x) { issue_load(T::BK, 1, decltype(x)::value); });
            wait_vmcnt<T::A_LOADS>();
        } else {
            wait_vmcnt<0>();
        }
        __syncthreads();
        static_for<0, NREAD>([&](auto r) { read_frag(0, 0, 0, decltype(r)::value); });
        int s = 0;
        for (; s + 2 < nk; ++s) kstep(yes, yes, yes, s & 1, (s + 2) * T::BK, (s + 1) * T::BK);
        if (s + 1 < nk) {
            kstep(no, yes, yes, s & 1, 0, (s + 1) * T::BK);
            ++s;
        }
        kstep(no, no, no, s & 1, 0, 0);
    }

    // a7: epilogue (accumulator holds C transposed: lane owns 4 consecutive
    // columns of one row per 4 registers)
    constexpr int OB = OUT == DT_F32 ? 4 : 2;
    const int64_t ldc = p.ldc;
    static_for<0, T::FM * T::FN>([&](auto bt) {
        constexpr int i = decltype(bt)::value / T::FN, j = decltype(bt)::value % T::FN;
        const int row = m0 + wm * T::WTM + 32 * i + l32;
        static_for<0, 4>([&](auto qt) {
            constexpr int qq = decltype(qt)::value;
            const int col = n0 + wn * T::WTN + 32 * j + 8 * qq + 4 * h;
            char* dst = p.C + ((int64_t)row * ldc + col) * OB;
            store4<OUT>(dst, acc[i][j][4 * qq + 0], acc[i][j][4 * qq + 1], acc[i][j][4 * qq + 2],
                        acc[i][j][4 * qq + 3], true);
        });
        __builtin_amdgcn_sched_barrier(0);
    });
}

}  // namespace tgemm
