// gemm_kernel_ring.hpp -- the gfx950 fast path of the tiled matrix product
// for 16-bit inputs (fp16 / bf16) on whole tiles: direct-to-LDS loads into
// S-stage LDS rings and v_mfma_f32_16x16x32_{f16,bf16}.
//
// The method is the tiled kernel of page "企业官网建设流程全解析" §3.3 (one
// workgroup per BM x BN tile of C, K walked in steps, A and B tiles staged in
// shared memory by a software pipeline of num_stages buffers, fp32 register
// accumulators), laid out for CDNA4:
//
//  * a2  global -> LDS without registers.  buffer_load_dwordx4 ... lds writes
//        the 16 bytes of lane l at LDS byte M0 + 16 l, so one instruction
//        fills a 1 KiB block; the XOR swizzle (a3) is obtained by choosing
//        which global 16-byte chunk each lane fetches.  The buffer resources
//        start at the tile's corner and end at the operand's last element;
//        the K position is the scalar offset, one add per operand and step.
//        Loads issued past the end of K read zeros (or in-bounds data that
//        is never used), so every step of the loop has the same shape.
//  * a4  pipeline.  BK = 32 per step; A and B each have a ring of S = 4 LDS
//        stages.  The loads of step s + S are issued during step s, so a
//        load has S - 1 steps (about 3 x 1000 cycles) to arrive.  One
//        barrier per step: after it, the stage read during the previous step
//        is free and is refilled.
//  * a5  MFMA.  v_mfma_f32_16x16x32: lane l holds 8 consecutive k of row /
//        column l % 16 of each operand (k = 8 (l / 16) ..).  At the power
//        limit that random fp16 data sets on MI355X, this shape keeps a
//        higher clock than the 32x32x16 one (about 1.9 vs 1.6 GHz for MFMA
//        issue alone), which more than pays for its lower issue rate.
//        B is the first operand and A the second, so the accumulator holds C
//        transposed: lane l owns row l % 16 and the 4 consecutive columns
//        4 (l / 16) .. of each 16 x 16 block, stored with one write.
//  * A k-strided operand is read with ds_read_b64_tr_b16: in each group of
//        16 lanes, lane i points at
//        4 consecutive columns of k-row i / 4 and receives element i % 4 of
//        the loads of lanes i / 4, i / 4 + 4, i / 4 + 8, i / 4 + 12, i.e.
//        one column of a 4-row block.  Two such reads give the 8 k-values of
//        one column.
//  * The loop is unrolled over the ring, so every LDS read is a base
//        register plus an immediate offset and the loop body holds no vector
//        address arithmetic: with one wave per SIMD, every instruction between
//        two MFMAs takes issue slots that the MFMA pipe would otherwise use.
//
// Operand layouts (the row-major default and the column-major option of page
// "TileLang实战：用Python DSL自动生成高性能GPU计算内核" §5.1): an operand
// whose k is contiguous in memory (A row-major, B column-major) is staged as
// rows of 32 k (64 bytes) per row / column and read with ds_read_b128; one
// whose k is strided (A column-major, B row-major) is staged as 32 k-rows of
// the tile's width and read with ds_read_b64_tr_b16.
//
// LDS: the A ring (S stages), then the B ring (S stages), each stage
// width x 32 x 2 bytes.
//   k contiguous: 16-byte chunk c of row r stored at chunk c ^ ((r / 4) % 4):
//      the 16 rows read by one quarter wave (one ds_read_b128 cycle) land in
//      16 different bank groups.
//   k strided: chunk c of k-row r stored at chunk c ^ (4 (r % 4) ^ 2 ((r/8)
//      % 2)): the rows r .. r+3 and r+8 .. r+11 read by one half wave of a
//      transposing read land in 16 different bank groups.

#pragma once
#include "gemm_kernel.hpp"

namespace tgemm {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

// operand layouts (gemm_t): element (i, j) of a row-major matrix at
// X[i * ld + j], of a column-major one at X[j * ld + i]
enum { LAYOUT_ROW = 0, LAYOUT_COL = 1 };

// s_waitcnt that limits only the vector-memory counter, to N outstanding
// (gfx9 encoding: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[15:14]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// One operand's tile in the ring: EXT rows / columns (BM for A, BN for B) by
// 32 of K; KC: k contiguous in memory.
template <int EXT, bool KC_>
struct RingOperand {
    static constexpr bool KC = KC_;
    static constexpr int STAGE = EXT * 64;               // bytes per stage
    static constexpr int ROW = KC ? 64 : EXT * 2;        // bytes per LDS row
    static constexpr int CHUNKS = ROW / 16;              // 16-byte chunks per row
    static constexpr int RPB = 1024 / ROW;               // LDS rows per 1 KiB load
    static constexpr int BLOCKS = STAGE / 1024;
    static constexpr int READS = KC ? 1 : 2;             // LDS reads per fragment
    static_assert(KC || CHUNKS == 16 || CHUNKS == 32, "k-strided tiles of 128 or 256");
};

__device__ __forceinline__ int ring_key_kc(int r) { return (r >> 2) & 3; }
__device__ __forceinline__ int ring_key_ks(int r) { return 4 * (r & 3) ^ 2 * ((r >> 3) & 1); }

// Tile configuration of the ring kernel: BM x BN output tile, WM x WN waves,
// S ring stages of BK = 32, OCC workgroups per CU the registers are sized for.
template <int BM_, int BN_, int WM_, int WN_, int S_, int OCC_>
struct RingCfg {
    static constexpr int BM = BM_, BN = BN_, BK = 32, WM = WM_, WN = WN_, S = S_, OCC = OCC_;
    static constexpr int THREADS = 64 * WM * WN, WAVES = WM * WN;
    static constexpr int EB = 2;
    static constexpr int A_STAGE = BM * 64, B_STAGE = BN * 64;
    static constexpr int A_RING = S * A_STAGE, B_RING = S * B_STAGE;
    static constexpr int LDS_BYTES = A_RING + B_RING;
    static constexpr int A_BLOCKS = A_STAGE / 1024, B_BLOCKS = B_STAGE / 1024;
    static constexpr int A_LOADS = A_BLOCKS / WAVES, B_LOADS = B_BLOCKS / WAVES;
    static constexpr int L = A_LOADS + B_LOADS;    // loads per wave per step
    static constexpr int WTM = BM / WM, WTN = BN / WN;
    static constexpr int FM = WTM / 16, FN = WTN / 16;
    static constexpr int U = S;                    // steps per loop trip
    static constexpr int K_MULT = BK * U;          // K must be a multiple of this
    static_assert(S % 2 == 0, "fragment buffers alternate per step");
    static_assert(A_BLOCKS % WAVES == 0 && B_BLOCKS % WAVES == 0, "");
    static_assert(LDS_BYTES <= 160 * 1024, "gfx950 LDS is 160 KiB per CU");
    static_assert(S >= 3 && (S - 1) * L < 64, "vmcnt range");
    // every LDS read offset fits the 16-bit immediate of ds_read, in either
    // layout of either operand
    static_assert(A_RING - A_STAGE + (FM - 1) * 16 * 64 < 65536 && A_RING - A_STAGE + 4 * BM * 2 < 65536, "");
    static_assert(B_RING - B_STAGE + (FN - 1) * 16 * 64 < 65536 && B_RING - B_STAGE + 4 * BN * 2 < 65536, "");
    static_assert(WTM % 16 == 0 && WTN % 16 == 0, "");
};

// Preconditions (checked by the host): 16-bit inputs; M % BM == 0,
// N % BN == 0, K % K_MULT == 0; A and B 16-byte aligned with lda and ldb
// multiples of 8; C aligned for 4-element stores with ldc % 4 == 0; the
// buffer offsets (a tile's rows or columns of each operand over K + S*BK of
// K) below 2^31 bytes.  LA / LB: LAYOUT_ROW or LAYOUT_COL; C is row-major.
template <class T, int IN, int OUT, int LA, int LB>
__global__ __attribute__((amdgpu_flat_work_group_size(T::THREADS, T::THREADS),
                          amdgpu_waves_per_eu(T::OCC * T::WAVES / 4 > 0 ? T::OCC * T::WAVES / 4 : 1)))
void gemm_kernel_ring(GemmArgs p) {
    // A is k-contiguous when row-major, B when column-major
    using OA = RingOperand<T::BM, LA == LAYOUT_ROW>;
    using OB_ = RingOperand<T::BN, LB == LAYOUT_COL>;
    __shared__ __attribute__((aligned(1024))) char smem[T::LDS_BYTES];
    const int smem_base = (int)(uintptr_t)(lds_void*)smem;   // LDS byte address (M0 values)
    lds_char* const lds = (lds_char*)smem;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / T::WN, wn = wave % T::WN;

    // a1: which tile
    int tm, tn;
    tile_of(blockIdx.x, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
    const int m0 = tm * T::BM, n0 = tn * T::BN;
    const int K = p.K;
    const int64_t lda = p.lda, ldb = p.ldb;
    // 1: XOR-swizzled LDS layouts; 0: plain LDS rows (kept for measuring
    // bank conflicts against the swizzle)
    const int swz = p.swz_mask != 0 ? 1 : 0;

    // ---------------------------------------------------------- a2: loads
    auto make_rsrc = [&](const char* base, int64_t bytes) __attribute__((always_inline)) {
        const uint64_t a = (uint64_t)base;
        const uint32_t n = bytes <= 0 ? 0u : bytes > 0xffffffffLL ? 0xffffffffu : (uint32_t)bytes;
        return i32x4{__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
                     __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32)),
                     __builtin_amdgcn_readfirstlane((int)n), 0x00020000};
    };
    // Buffer resource of one operand: it starts at the tile's corner and ends
    // at the operand's last element (empty when K = 0: no load is issued
    // then).  outer0: the tile's first row (A) / column (B); outer: M / N.
    auto operand_rsrc = [&](auto op_t, const char* X, int64_t ld, int outer0, int outer) __attribute__((always_inline)) {
        using O = decltype(op_t);
        if (K <= 0) return make_rsrc(X, 0);
        if constexpr (O::KC)  // element (o, k) at o * ld + k
            return make_rsrc(X + (int64_t)outer0 * ld * 2, ((int64_t)(outer - 1 - outer0) * ld + K) * 2);
        else                  // element (o, k) at k * ld + o
            return make_rsrc(X + (int64_t)outer0 * 2, ((int64_t)(K - 1) * ld + outer - outer0) * 2);
    };
    const i32x4 rs_a = operand_rsrc(OA{}, p.A, lda, m0, p.M);
    const i32x4 rs_b = operand_rsrc(OB_{}, p.B, ldb, n0, p.N);
    // per-lane byte offset of load x (block blk of the stage): lane l fills
    // slot l of the 1 KiB block (LDS row l / CHUNKS, chunk l % CHUNKS) with
    // the logical chunk the swizzle puts there
    auto load_voff = [&](auto op_t, int blk, int64_t ld) __attribute__((always_inline)) {
        using O = decltype(op_t);
        const int r = blk * O::RPB + lane / O::CHUNKS;   // LDS row: outer index (KC) or k (KS)
        const int key = O::KC ? ring_key_kc(r) : ring_key_ks(r);
        const int c = (lane % O::CHUNKS) ^ (swz * key);
        return (int)((int64_t)r * ld * 2 + c * 16);
    };
    int voff[T::L];
#pragma unroll
    for (int x = 0; x < T::L; ++x)
        voff[x] = x < T::A_LOADS ? load_voff(OA{}, wave * T::A_LOADS + x, lda)
                                 : load_voff(OB_{}, wave * T::B_LOADS + (x - T::A_LOADS), ldb);
    // K advance per step: 32 elements along a row (KC) or 32 rows (KS)
    const int a_kstep = OA::KC ? 64 : (int)(32 * lda * 2);
    const int b_kstep = OB_::KC ? 64 : (int)(32 * ldb * 2);
    // Issued through inline asm (M0 = LDS destination, then the load): the
    // compiler then does not guard later LDS reads with waits for these
    // loads; the kernel waits for them itself (vmcnt) before the barrier that
    // publishes a stage.
    auto dma = [&](int lds_addr, int vo, i32x4 rs, int so) __attribute__((always_inline)) {
        asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                     :
                     : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(vo), "s"(rs), "s"(so)
                     : "memory");
    };
    // load x of the step whose K byte offsets are (ka, kb) into ring stage st
    auto issue_load = [&](int st, int x, int ka, int kb) __attribute__((always_inline)) {
        if (x < T::A_LOADS)
            dma(smem_base + st * T::A_STAGE + (wave * T::A_LOADS + x) * 1024, voff[x], rs_a, ka);
        else
            dma(smem_base + T::A_RING + st * T::B_STAGE + (wave * T::B_LOADS + x - T::A_LOADS) * 1024, voff[x],
                rs_b, kb);
    };

    // ---------------------------------------------------------- a5: fragments
    // v_mfma_f32_16x16x32: lane l holds 8 consecutive k (8q .., q = l / 16) of
    // row / column l % 16 of each operand.
    const int q = lane >> 4, i16 = lane & 15;
    // per-lane LDS base of fragment f of an operand whose wave block starts
    // at outer index wo (the stage and the second transposing read go in the
    // immediate offset)
    auto frag_base = [&](auto op_t, lds_char* ring, int wo, int f) __attribute__((always_inline)) {
        using O = decltype(op_t);
        if constexpr (O::KC) {
            // row wo + 16 f + l%16, chunk q
            const int r = wo + 16 * f + i16;
            return ring + r * O::ROW + (q ^ (swz * ring_key_kc(r))) * 16;
        } else {
            // lane i of group q: k-row 8q + i/4 (+4 for the second read),
            // columns wo + 16 f + 4 (i%4) .. +3
            const int r = 8 * q + (i16 >> 2);
            const int c = (wo + 16 * f) / 8 + ((i16 & 3) >> 1);
            return ring + r * O::ROW + (c ^ (swz * ring_key_ks(r))) * 16 + 8 * (i16 & 1);
        }
    };
    // k-contiguous operands need one base (the fragments are 1 KiB apart);
    // k-strided ones one per fragment (the swizzle permutes their columns)
    constexpr int NBA = OA::KC ? 1 : T::FM, NBB = OB_::KC ? 1 : T::FN;
    lds_char* a_base[NBA];
    lds_char* b_base[NBB];
#pragma unroll
    for (int f = 0; f < NBA; ++f) a_base[f] = frag_base(OA{}, lds, wm * T::WTM, f);
#pragma unroll
    for (int f = 0; f < NBB; ++f) b_base[f] = frag_base(OB_{}, lds + T::A_RING, wn * T::WTN, f);

    // fragments: h[0] (k 0..3) and h[1] (k 4..7) of a lane's 8 k
    i16x4 fa[2][T::FM][2], fb[2][T::FN][2];
    auto read_one = [&](auto op_t, lds_char* const* base, int stage_bytes, int st, int f, int h,
                        i16x4 (&dst)[2]) __attribute__((always_inline)) {
        using O = decltype(op_t);
        if constexpr (O::KC) {
            const u32x4 v = *(const lds_u32x4*)(base[0] + st * stage_bytes + f * 16 * O::ROW);
            const i16x8 w = __builtin_bit_cast(i16x8, v);
            dst[0] = __builtin_shufflevector(w, w, 0, 1, 2, 3);
            dst[1] = __builtin_shufflevector(w, w, 4, 5, 6, 7);
        } else {
            dst[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base[f] + st * stage_bytes + 4 * h * O::ROW));
        }
    };
    constexpr int NRB = T::FN * OB_::READS, NRA = T::FM * OA::READS;
    constexpr int NREAD = NRA + NRB;
    // read r of stage st into buffer buf: the B fragments first, then the A
    // fragments, the order the MFMAs need them in
    auto read_frag = [&](int st, int buf, int r) __attribute__((always_inline)) {
        if (r < NRB)
            read_one(OB_{}, b_base, T::B_STAGE, st, r / OB_::READS, r % OB_::READS, fb[buf][r / OB_::READS]);
        else
            read_one(OA{}, a_base, T::A_STAGE, st, (r - NRB) / OA::READS, (r - NRB) % OA::READS,
                     fa[buf][(r - NRB) / OA::READS]);
    };

    // a6: accumulators, zeroed (T.clear of §3.3).  The empty asm makes each
    // one opaque, so that every accumulator gets registers of its own and
    // every MFMA accumulates in place (a shared zero register would make the
    // first MFMAs write elsewhere and the loop copy accumulators around).
    f32x4 acc[T::FM][T::FN];
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int j = 0; j < T::FN; ++j) {
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
            asm volatile("" : "+a"(acc[i][j]));
        }

    constexpr int NMF = T::FM * T::FN;
    // B is the first operand and A the second, so the accumulator holds C
    // transposed: lane l owns row l % 16 and the 4 consecutive columns
    // 4 (l / 16) .. of each 16 x 16 block
    auto mfma_one = [&](int buf, int m) __attribute__((always_inline)) {
        // snake order over j: neighbours share one operand
        const int i = m / T::FN, jj = m % T::FN, j = (i & 1) ? T::FN - 1 - jj : jj;
        const i16x8 bop = __builtin_shufflevector(fb[buf][j][0], fb[buf][j][1], 0, 1, 2, 3, 4, 5, 6, 7);
        const i16x8 aop = __builtin_shufflevector(fa[buf][i][0], fa[buf][i][1], 0, 1, 2, 3, 4, 5, 6, 7);
        if constexpr (IN == DT_F16) {
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, bop),
                                                                __builtin_bit_cast(f16x8, aop), acc[i][j], 0, 0, 0);
        } else {
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, bop),
                                                                 __builtin_bit_cast(bf16x8, aop), acc[i][j], 0, 0, 0);
        }
    };

    // One step on ring stage ST, fragments in buffer BUF: wait until this
    // wave's loads of the next stage have landed ((S-2)*L loads of later
    // steps may still be in flight), barrier (every wave has then finished
    // the previous step, so the next stage is complete and stage ST, read
    // during the previous step, is free), then the MFMAs, with the next
    // stage's fragment reads and the loads of step s + S into stage ST
    // interleaved: one load after every NREAD / L reads, spread over the
    // MFMAs so that at most two other instructions sit between two MFMAs.
    auto step = [&](auto st_t, auto buf_t, int ka, int kb) __attribute__((always_inline)) {
        constexpr int ST = decltype(st_t)::value, BUF = decltype(buf_t)::value;
        constexpr int NXT = (ST + 1) % T::S;
        wait_vmcnt<(T::S - 2) * T::L>();
        __syncthreads();
        constexpr int n_work = NREAD + T::L;
        constexpr int per = NREAD / T::L;
        static_assert(NREAD % T::L == 0, "");
        static_for<0, NMF>([&](auto mt) __attribute__((always_inline)) {
            constexpr int m = decltype(mt)::value;
            mfma_one(BUF, m);
            constexpr int wb = (m * n_work + NMF - 1) / NMF;
            constexpr int we = ((m + 1) * n_work + NMF - 1) / NMF;
            static_for<wb, we>([&](auto wt) __attribute__((always_inline)) {
                constexpr int w = decltype(wt)::value;
                constexpr int grp = w / (per + 1);
                if constexpr (w % (per + 1) == per) issue_load(ST, grp, ka, kb);
                else read_frag(NXT, BUF ^ 1, w - grp);
            });
            __builtin_amdgcn_sched_barrier(0);
        });
    };

    const int nk = K / T::BK;  // a multiple of U (host precondition)
    if (nk > 0) {
        // prologue: steps 0 .. S-1 into stages 0 .. S-1, then the fragments
        // of step 0
        static_for<0, T::S>([&](auto s_t) __attribute__((always_inline)) {
            constexpr int s = decltype(s_t)::value;
            static_for<0, T::L>([&](auto x) __attribute__((always_inline)) {
                issue_load(s, decltype(x)::value, s * a_kstep, s * b_kstep);
            });
        });
        wait_vmcnt<(T::S - 1) * T::L>();
        __syncthreads();
        static_for<0, NREAD>([&](auto r) __attribute__((always_inline)) { read_frag(0, 0, decltype(r)::value); });
        int ka = T::S * a_kstep, kb = T::S * b_kstep;  // K offsets of the next step to load
        for (int s = 0; s < nk; s += T::U) {
            static_for<0, T::U>([&](auto u_t) __attribute__((always_inline)) {
                constexpr int u = decltype(u_t)::value;
                step(IntTag<u % T::S>{}, IntTag<u & 1>{}, ka, kb);
                ka += a_kstep;
                kb += b_kstep;
            });
        }
        // no load may still be writing LDS when the workgroup ends
        wait_vmcnt<0>();
    }

    // a7: epilogue.  acc[i][j] of lane l is C[row 16 i + l%16][columns
    // 16 j + 4 (l/16) .. +3] of the wave's block; fp32 -> fp16 / bf16 rounds
    // to nearest even.
    constexpr int OB = OUT == DT_F32 ? 4 : 2;
    const int64_t ldc = p.ldc;
    static_for<0, NMF>([&](auto bt) __attribute__((always_inline)) {
        constexpr int i = decltype(bt)::value / T::FN, j = decltype(bt)::value % T::FN;
        const int row = m0 + wm * T::WTM + 16 * i + i16;
        const int col = n0 + wn * T::WTN + 16 * j + 4 * q;
        store4<OUT>(p.C + ((int64_t)row * ldc + col) * OB, acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3],
                    true);
    });
}

}  // namespace tgemm
