// gemm_kernel_ring.hpp -- the gfx950 fast path of the tiled matrix product
// for 16-bit inputs (fp16 / bf16), aligned operands, any M and N (edge tiles
// store masked): direct-to-LDS loads into multi-stage LDS rings and
// v_mfma_f32_16x16x32_{f16,bf16}.  K a multiple of 128, or
// (variant KT) any K above 128: the rings walk the largest multiple of 128 and
// the rest takes a few steps from registers.
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
//  * a4  pipeline.  Steps of BK = 32.  B has a ring of 4 LDS stages of one
//        step; a row-major A (k contiguous) a ring of 2 stages of two steps,
//        so that each of its loads reads whole 128-byte lines (loads of
//        64-byte half lines run at about 60% of that rate).  A stage is
//        refilled at the step that frees it, with the loads of the stage
//        that starts 4 steps later; they have 2 (A) or 3 (B) steps, about
//        1000 cycles each, to arrive.  One barrier per step: after it, the
//        stages read during the previous step for the last time are free.
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
// 64 bytes (32 k) per row / column and step and read with ds_read_b128; one
// whose k is strided (A column-major, B row-major) is staged as 32 k-rows of
// the tile's width and read with ds_read_b64_tr_b16.
//
// LDS: the A ring, then the B ring, 64 KiB each for a 256 x 256 tile (the
// stage layouts and swizzles are described at RingOperand).

#pragma once
#include "gemm_kernel.hpp"

namespace tgemm {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
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

__device__ __forceinline__ constexpr int ring_key_kc(int r) { return (r >> 1) & 3; }
__device__ __forceinline__ constexpr int ring_key_ks(int r) { return 4 * (r & 3) ^ 2 * ((r >> 3) & 1); }

// The ring of one operand: EXT rows (A) / columns (B) of the tile; KC: k
// contiguous in memory; D steps of 32 k per stage, NS stages.
//
// Layout of a stage, as (r, c) -> byte position, r the LDS row (KC: row of A
// / column of B; KS: k) and c its 16-byte chunk (KC: 8 k; KS: 8 columns):
//   KC, D = 1: rows of 64 bytes, chunk c of row r at c ^ key(r);
//   KC, D = 2: 1 KiB blocks of 8 rows; in a block, the first 64 bytes of
//              each row (the stage's first step), then the second 64 bytes;
//              chunk slots swizzled as for D = 1.  A fragment read of one
//              step then touches 512 bytes of each of two blocks, and a load
//              brings whole 128-byte lines of 8 rows;
//   KS:        rows of EXT * 2 bytes, chunk c of row r at c ^ key_ks(r).
// Loads fill 1 KiB blocks lane by lane (lane l: byte 16 l of the block), so a
// layout is realised by choosing which global chunk each lane fetches (at).
// The keys were chosen by measuring the reads of one wave: key (r / 2) % 4
// makes a k-contiguous fragment read (16 rows, chunk l / 16 for lane l) as
// fast as a contiguous 1 KiB ds_read_b128 (256 bytes per clock, no bank
// conflict cycles), while plain rows and the keys (r / 4) % 4, r % 4,
// 2 ((r / 2) % 2) take twice as long; key_ks puts the 16 k-rows of one
// transposing read in different bank groups.
template <int EXT, bool KC_, int D_, int NS_>
struct RingOperand {
    static constexpr bool KC = KC_;
    static constexpr int D = D_, NS = NS_;
    static constexpr int STAGE = EXT * 64 * D;           // bytes per stage
    static constexpr int RING = NS * STAGE;
    static constexpr int ROW = KC ? 64 : EXT * 2;        // bytes per LDS row (a D = 2 row: two of 64)
    static constexpr int BLOCKS = STAGE / 1024;
    static_assert(KC || D == 1, "k-strided operands take one step per stage");
    static_assert(D == 1 || D == 2, "");
    static_assert(KC || EXT == 128 || EXT == 256, "k-strided tiles of 128 or 256");
    // byte position of chunk c of row r in a stage (swz = 0: no swizzle,
    // kept for measuring bank conflicts against the swizzle)
    static constexpr int pos(int r, int c, int swz = 1) {
        if (KC && D == 2)
            return (r >> 3) * 1024 + (c >> 2) * 512 + (r & 7) * 64 + (((c & 3) ^ (swz * ring_key_kc(r))) * 16);
        if (KC) return r * 64 + ((c ^ (swz * ring_key_kc(r))) * 16);
        return r * ROW + ((c ^ (swz * ring_key_ks(r))) * 16);
    }
    // the (row, chunk) stored at byte position p (p a multiple of 16)
    static constexpr void at(int p, int& r, int& c, int swz = 1) {
        if (KC && D == 2) {
            r = (p >> 10) * 8 + ((p >> 6) & 7);
            c = ((p >> 9) & 1) * 4 + (((p >> 4) & 3) ^ (swz * ring_key_kc(r)));
        } else if (KC) {
            r = p >> 6;
            c = ((p >> 4) & 3) ^ (swz * ring_key_kc(r));
        } else {
            r = p / ROW;
            c = ((p % ROW) >> 4) ^ (swz * ring_key_ks(r));
        }
    }
    // stage of step j and the step's place in it
    static constexpr int stage_of(int j) { return (j / D) % NS; }
    static constexpr int sub_of(int j) { return j % D; }
    // a stage is refilled at the step that frees it (its last step): at step v
    // with v % D == D - 1 the loads of the stage that starts at v - D + 1 + NS D
    static constexpr bool issues_at(int v) { return ((v % D) + D) % D == D - 1; }
    static constexpr int first_loaded_at(int v) { return v - D + 1 + NS * D; }
    // the step at which the stage holding step j was loaded
    static constexpr int loaded_at(int j) { return j - j % D + D - 1 - NS * D; }
    // Reads: fragment f of step j is at a per-lane base plus an immediate
    // offset.  k-contiguous: one base per 64 KiB of ring (stage, fragment
    // and step in the immediate); k-strided: one base per fragment (the
    // swizzle permutes the columns; stage and second read in the immediate).
    static constexpr int kc_off(int f, int j) {
        return stage_of(j) * STAGE + (D == 1 ? f * 1024 : f * 2048 + sub_of(j) * 512);
    }
    static constexpr int bases(int F) { return KC ? ((RING - 1) >> 16) + 1 : F; }
    static constexpr bool imm_ok(int F) {
        return KC ? true : (NS - 1) * STAGE + 4 * ROW < 65536;
    }
};

constexpr int ring_gcd(int a, int b) { return b == 0 ? a : ring_gcd(b, a % b); }
constexpr int ring_lcm(int a, int b) { return a / ring_gcd(a, b) * b; }

// Tile configuration of the ring kernel: BM x BN output tile, WM x WN waves,
// OCC workgroups per CU the registers and LDS are sized for; steps of BK = 32.
// BNS: stages of B's ring (one step each); ANS: stages of a k-contiguous A's
// ring (two steps each; a k-strided A takes 2 ANS stages of one step).
template <int BM_, int BN_, int WM_, int WN_, int OCC_, int BNS_ = 4, int ANS_ = 2>
struct RingCfg {
    static constexpr int BM = BM_, BN = BN_, BK = 32, WM = WM_, WN = WN_, OCC = OCC_;
    static_assert(BNS_ >= 2 && ANS_ >= 2, "a stage is refilled while the other stages are read");
    static constexpr int THREADS = 64 * WM * WN, WAVES = WM * WN;
    static constexpr int WTM = BM / WM, WTN = BN / WN;
    static constexpr int FM = WTM / 16, FN = WTN / 16;
    // the rings walk K in multiples of this (one loop trip)
    static constexpr int K_MULT = ring_lcm(ring_lcm(2 * ANS_, BNS_), 4) * BK;
    // Ring of each operand for the layouts of A and B.  A k-contiguous
    // operand reads 64 bytes of every row per step, half a 128-byte line, and
    // such loads run at about 60% of the rate of whole lines: a k-contiguous
    // A takes two stages of two steps (128 bytes per row) instead of four of
    // one, in the same LDS.  B keeps four stages of one step in every layout:
    // with a two-step B ring beside a k-strided A, the register allocator no
    // longer keeps every accumulator in place.
    template <bool KCA, bool KCB>
    struct Plan {
        static constexpr bool DA = KCA;
        using OA = RingOperand<BM, KCA, DA ? 2 : 1, DA ? ANS_ : 2 * ANS_>;
        using OB = RingOperand<BN, KCB, 1, BNS_>;
        static constexpr int LA = OA::BLOCKS / WAVES, LB = OB::BLOCKS / WAVES;  // loads per wave and stage
        static constexpr int LDS_BYTES = OA::RING + OB::RING;
        // steps per loop trip: both rings and the two fragment buffers return
        // to their first state
        static constexpr int U = ring_lcm(ring_lcm(OA::D * OA::NS, OB::D * OB::NS), 4);
        static constexpr int loads_at(int v) { return (OA::issues_at(v) ? LA : 0) + (OB::issues_at(v) ? LB : 0); }
        // loads issued after those that step j's stages need, counted at the
        // start of step `now` (the wait before step j's fragments are read)
        static constexpr int after(int j, int now) {
            const int t = OA::loaded_at(j) > OB::loaded_at(j) ? OA::loaded_at(j) : OB::loaded_at(j);
            int n = 0;
            for (int v = t + 1; v < now; ++v) n += loads_at(v);
            return n;
        }
        static_assert(OA::BLOCKS % WAVES == 0 && OB::BLOCKS % WAVES == 0, "");
        static_assert(LDS_BYTES * OCC <= 160 * 1024, "gfx950 LDS is 160 KiB per CU");
        static_assert(U % (OA::D * OA::NS) == 0 && U % (OB::D * OB::NS) == 0 && U % 4 == 0, "");
        // every LDS read offset fits the 16-bit immediate of ds_read
        static_assert(OA::imm_ok(FM) && OB::imm_ok(FN), "");
    };
    // LDS per workgroup (the same for every layout: a k-strided A ring of 4
    // one-step stages and a k-contiguous one of 2 two-step stages both hold
    // BM x 128 elements)
    static constexpr int LDS_BYTES = Plan<true, false>::LDS_BYTES;
    // a k-strided A stage needs rows of at least 16 chunks for its swizzle
    // key: tiles narrower than 128 rows take row-major A only
    static constexpr bool A_COL_OK = BM >= 128;
    // how far past K the ring loads (steps of 32)
    static constexpr int LOOKAHEAD = 2 * ANS_ > BNS_ ? 2 * ANS_ : BNS_;
    // the rings of row-major A and B (the default layouts)
    static constexpr int A_BK = 32 * Plan<true, false>::OA::D, A_STAGES = Plan<true, false>::OA::NS;
    static constexpr int B_BK = 32, B_STAGES = Plan<true, false>::OB::NS;
    static_assert(WTM % 16 == 0 && WTN % 16 == 0, "");
};

// Preconditions (checked by the host): 16-bit inputs; K % K_MULT == 0, or
// K > K_MULT with KT; A and B element-aligned, and where their rows are not
// whole 16-byte chunks (16-byte aligned, ld a multiple of 8), range_pad_a /
// range_pad_b 2 for an operand whose last element starts a 4-byte part of its
// load at an address of 2 mod 4 (the 2 bytes after it in its page), else 0; without EPI, N % 4 == 0 and C aligned for 4-element stores with
// ldc % 4 == 0 (the fused epilogue, EPI, takes any N and C alignment; a plain
// product that needs it runs EPI with alpha 1, beta 0, no bias and no
// activation, which store the product unchanged); the buffer offsets (a tile's rows or
// columns of each operand over K + LOOKAHEAD * BK of K) below 2^31 bytes.  LA / LB: LAYOUT_ROW or
// LAYOUT_COL; C is row-major.
//
// KT (K tail): the rings walk the largest multiple of K_MULT below K; the
// remaining K % K_MULT values take steps of 32 whose fragments are loaded
// from global memory straight into registers (no LDS, no barrier), with the
// elements at k >= K zeroed (inside the buffer range they are other elements
// of the operand or row padding, which may hold anything).  The main loop is
// the same code as without KT.
template <class T, int IN, int OUT, int LA, int LB, bool EPI = false, bool KT = false>
__global__ __attribute__((amdgpu_flat_work_group_size(T::THREADS, T::THREADS),
                          amdgpu_waves_per_eu(T::OCC * T::WAVES / 4 > 0 ? T::OCC * T::WAVES / 4 : 1)))
void gemm_kernel_ring(GemmArgs p) {
    // A is k-contiguous when row-major, B when column-major
    using P = typename T::template Plan<LA == LAYOUT_ROW, LB == LAYOUT_COL>;
    using OA = typename P::OA;
    using OB_ = typename P::OB;
    __shared__ __attribute__((aligned(1024))) char smem[P::LDS_BYTES];
    const int smem_base = (int)(uintptr_t)(lds_void*)smem;   // LDS byte address (M0 values)
    lds_char* const lds = (lds_char*)smem;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / T::WN, wn = wave % T::WN;

    // split-K (p.splits > 1, plain epilogue only): workgroup g takes slice
    // s = g / tiles of K, [s k_split, min(K, (s + 1) k_split)), and writes
    // its fp32 partial tile to slice s of the workspace that C points to
    int bid = blockIdx.x;
    int K = p.K;
    const char* A = p.A;
    const char* B = p.B;
    char* C = p.C;
    const int64_t lda = p.lda, ldb = p.ldb;
    if (!EPI && p.splits > 1) {
        const int tiles = p.tiles_m * p.tiles_n;
        const int s = bid / tiles;
        bid -= s * tiles;
        const int k0 = s * p.k_split;
        K = p.K - k0 < p.k_split ? p.K - k0 : p.k_split;
        A += (OA::KC ? (int64_t)k0 : (int64_t)k0 * lda) * 2;
        B += (OB_::KC ? (int64_t)k0 : (int64_t)k0 * ldb) * 2;
        C += (int64_t)s * p.split_stride;
    }
    // a1: which tile
    int tm, tn;
    tile_of(bid, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
    const int m0 = tm * T::BM, n0 = tn * T::BN;
    // 1: XOR-swizzled LDS layouts; 0: plain LDS rows (kept for measuring
    // bank conflicts against the swizzle)
    const int swz = p.swz_mask != 0 ? 1 : 0;

    // ---------------------------------------------------------- a2: loads
    // The range check keeps a 4-byte part of a load only if the part ends
    // inside the range, counted from the load's own offset (measured on
    // gfx950, 16-byte loads at every even offset).  A part that holds the
    // operand's last element and the 2 bytes after it would be dropped with
    // the element, so the range's end is rounded up to a dword boundary of
    // the address space: it then never reaches past the aligned dword that
    // holds the last element (no other page), and the bytes it adds reach
    // only outputs past M or N or positions past K, never stored or zeroed.
    // With rows of whole 16-byte chunks this keeps every element.  Otherwise
    // an element that starts a part at an address of 2 mod 4 is kept only
    // with the 2 bytes after it in range: the host then passes a pad of 2
    // (it checks that those bytes lie in the element's page).
    auto make_rsrc = [&](const char* base, int64_t bytes, int pad) __attribute__((always_inline)) {
        const uint64_t a = (uint64_t)base;
        if (bytes > 0) bytes = (int64_t)(((a + (uint64_t)bytes + 3) & ~(uint64_t)3) - a) + pad;
        const uint32_t n = bytes <= 0 ? 0u : bytes > 0xffffffffLL ? 0xffffffffu : (uint32_t)bytes;
        return i32x4{__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
                     __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32)),
                     __builtin_amdgcn_readfirstlane((int)n), 0x00020000};
    };
    // Buffer resource of one operand: it starts at the tile's corner and ends
    // at the operand's last element (empty when K = 0: no load is issued
    // then).  outer0: the tile's first row (A) / column (B); outer: M / N.
    auto operand_start = [&](auto op_t, const char* X, int64_t ld, int outer0) __attribute__((always_inline)) {
        using O = decltype(op_t);
        return O::KC ? X + (int64_t)outer0 * ld * 2 : X + (int64_t)outer0 * 2;
    };
    auto operand_bytes = [&](auto op_t, int64_t ld, int outer0, int outer) __attribute__((always_inline)) {
        using O = decltype(op_t);
        if (K <= 0) return (int64_t)0;
        if constexpr (O::KC)  // element (o, k) at o * ld + k
            return ((int64_t)(outer - 1 - outer0) * ld + K) * 2;
        else                  // element (o, k) at k * ld + o
            return ((int64_t)(K - 1) * ld + outer - outer0) * 2;
    };
    const char* const a_start = operand_start(OA{}, A, lda, m0);
    const char* const b_start = operand_start(OB_{}, B, ldb, n0);
    const int64_t a_bytes = operand_bytes(OA{}, lda, m0, p.M);
    const int64_t b_bytes = operand_bytes(OB_{}, ldb, n0, p.N);
    const i32x4 rs_a = make_rsrc(a_start, a_bytes, p.range_pad_a);
    const i32x4 rs_b = make_rsrc(b_start, b_bytes, p.range_pad_b);
    // per-lane byte offset of a load (block blk of a stage): lane l fills
    // byte 16 l of the block with the chunk the layout puts there
    auto load_voff = [&](auto op_t, int blk, int64_t ld) __attribute__((always_inline)) {
        using O = decltype(op_t);
        int r, c;
        O::at(blk * 1024 + 16 * lane, r, c, swz);
        return (int)((int64_t)r * ld * 2 + c * 16);
    };
    int voff_a[P::LA], voff_b[P::LB];
#pragma unroll
    for (int x = 0; x < P::LA; ++x) voff_a[x] = load_voff(OA{}, wave * P::LA + x, lda);
#pragma unroll
    for (int x = 0; x < P::LB; ++x) voff_b[x] = load_voff(OB_{}, wave * P::LB + x, ldb);
    // K advance per stage: 32 D elements along a row (KC) or 32 rows (KS)
    const int a_kstep = OA::KC ? 64 * OA::D : (int)(32 * lda * 2);
    const int b_kstep = OB_::KC ? 64 * OB_::D : (int)(32 * ldb * 2);
    // Issued through inline asm: the compiler then does not guard later LDS
    // reads with waits for these loads; the kernel waits for them itself
    // (vmcnt) before the barrier that publishes a stage.  The block writes M0
    // (the LDS destination) and names M0 as its output operand, so the
    // compiler knows M0 is overwritten and keeps nothing of its own there
    // across it.  (An "{m0}" input operand instead made the compiler move
    // accumulators in the 256 x 256 main loop.)
    auto dma = [&](int lds_addr, int vo, i32x4 rs, int so) __attribute__((always_inline)) {
        int m0_written;
        asm volatile("s_mov_b32 m0, %1\n\tbuffer_load_dwordx4 %2, %3, %4 offen lds"
                     : "={m0}"(m0_written)
                     : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(vo), "s"(rs), "s"(so)
                     : "memory");
        (void)m0_written;
    };
    // the loads of one operand's stage st at K byte offset k
    auto load_a = [&](int st, int x, int k) __attribute__((always_inline)) {
        dma(smem_base + st * OA::STAGE + (wave * P::LA + x) * 1024, voff_a[x], rs_a, k);
    };
    auto load_b = [&](int st, int x, int k) __attribute__((always_inline)) {
        dma(smem_base + OA::RING + st * OB_::STAGE + (wave * P::LB + x) * 1024, voff_b[x], rs_b, k);
    };

    // ---------------------------------------------------------- a5: fragments
    // v_mfma_f32_16x16x32: lane l holds 8 consecutive k (8q .., q = l / 16) of
    // row / column l % 16 of each operand.
    const int q = lane >> 4, i16 = lane & 15;
    // per-lane LDS bases of an operand whose wave block starts at outer index
    // wo (RingOperand: reads)
    auto make_bases = [&](auto op_t, lds_char* ring, int wo, lds_char** out, int n) __attribute__((always_inline)) {
        using O = decltype(op_t);
#pragma unroll
        for (int b = 0; b < n; ++b) {
            if constexpr (O::KC) {
                // row wo + l%16, chunk q of the stage's first step
                out[b] = ring + O::pos(wo + i16, q, swz) + b * 65536;
            } else {
                // fragment b: lane i of group q reads k-row 8q + i/4 (+4 for
                // the second read), columns wo + 16 b + 4 (i%4) .. +3
                const int r = 8 * q + (i16 >> 2);
                const int c = (wo + 16 * b) / 8 + ((i16 & 3) >> 1);
                out[b] = ring + O::pos(r, c, swz) + 8 * (i16 & 1);
            }
        }
    };
    constexpr int NBA = OA::bases(T::FM), NBB = OB_::bases(T::FN);
    lds_char* a_base[NBA];
    lds_char* b_base[NBB];
    make_bases(OA{}, lds, wm * T::WTM, a_base, NBA);
    make_bases(OB_{}, lds + OA::RING, wn * T::WTN, b_base, NBB);

    // fragments: a lane's 8 k of one row of A / column of B.  A k-strided
    // fragment takes two transposing reads (k 0..3, then k 4..7, 4 LDS rows
    // further); both are issued together and joined at once: reads of the two
    // halves scattered over the step let the register allocator split the
    // fragments and then copy accumulators around the loop.
    i16x8 fa[2][T::FM], fb[2][T::FN];
    // fragment f of step j (compile-time j: stage and step in the stage)
    auto read_one = [&](auto op_t, lds_char* const* base, auto j_t, int f, i16x8& dst) __attribute__((always_inline)) {
        using O = decltype(op_t);
        constexpr int j = decltype(j_t)::value;
        constexpr int st = O::stage_of(j);
        if constexpr (O::KC) {
            const int off = O::kc_off(f, j);
            dst = __builtin_bit_cast(i16x8, *(const lds_u32x4*)(base[off >> 16] + (off & 0xffff)));
        } else {
            lds_char* at = base[f] + st * O::STAGE;
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)at);
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(at + 4 * O::ROW));
            dst = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
    };
    // one unit of read work per fragment
    constexpr int NRB = T::FN, NRA = T::FM;
    constexpr int NREAD = NRA + NRB;
    // read r of step j into buffer buf: the B fragments first, then the A
    // fragments, the order the MFMAs need them in
    auto read_frag = [&](auto j_t, int buf, int r) __attribute__((always_inline)) {
        if (r < NRB)
            read_one(OB_{}, b_base, j_t, r, fb[buf][r]);
        else
            read_one(OA{}, a_base, j_t, r - NRB, fa[buf][r - NRB]);
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
        const i16x8 bop = fb[buf][j], aop = fa[buf][i];
        if constexpr (IN == DT_F16) {
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, bop),
                                                                __builtin_bit_cast(f16x8, aop), acc[i][j], 0, 0, 0);
        } else {
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, bop),
                                                                 __builtin_bit_cast(bf16x8, aop), acc[i][j], 0, 0, 0);
        }
    };

    // The loads of (virtual) step v: each operand refills the stage that step
    // v frees (B loads first, then A), the x-th load of the step.
    int ka = 0, kb = 0;  // K byte offsets of the next stage to load
    auto issue = [&](auto v_t, int x) __attribute__((always_inline)) {
        constexpr int v = decltype(v_t)::value;
        constexpr int nb = OB_::issues_at(v) ? P::LB : 0;
        if (x < nb) {
            load_b(OB_::stage_of(OB_::first_loaded_at(v)), x, kb);
            if (x == nb - 1) kb += b_kstep;
        } else {
            load_a(OA::stage_of(OA::first_loaded_at(v)), x - nb, ka);
            if (x == P::loads_at(v) - 1) ka += a_kstep;
        }
    };

    // One step u of the loop trip (compile-time; the ring state repeats every
    // U steps): wait until this wave's loads of the stages of step u + 1 have
    // landed, barrier (every wave has then finished step u - 1, so those
    // stages are complete and the stages step u frees, read for the last time
    // during step u - 1, can be refilled), then the MFMAs of step u with the
    // fragment reads of step u + 1 and this step's loads interleaved: one
    // load after every few reads, spread over the MFMAs so that at most two
    // other instructions sit between two MFMAs.
    auto step = [&](auto u_t) __attribute__((always_inline)) {
        constexpr int u = decltype(u_t)::value;
        constexpr int BUF = u & 1;
        constexpr int NL = P::loads_at(u);
        wait_vmcnt<P::after(u + 1, u)>();
        __syncthreads();
        constexpr int n_work = NREAD + NL;
        static_for<0, NMF>([&](auto mt) __attribute__((always_inline)) {
            constexpr int m = decltype(mt)::value;
            mfma_one(BUF, m);
            constexpr int wb = (m * n_work + NMF - 1) / NMF;
            constexpr int we = ((m + 1) * n_work + NMF - 1) / NMF;
            static_for<wb, we>([&](auto wt) __attribute__((always_inline)) {
                constexpr int w = decltype(wt)::value;
                // work item w: a load when w * NL / n_work steps up, else a read
                constexpr int lo = w * NL / n_work, hi = (w + 1) * NL / n_work;
                if constexpr (hi > lo) issue(IntTag<u>{}, lo);
                else read_frag(IntTag<(u + 1) % P::U>{}, BUF ^ 1, w - lo);
            });
            __builtin_amdgcn_sched_barrier(0);
        });
    };

    // steps of the rings: a multiple of U (without KT, K % K_MULT == 0)
    // (KT with a k-strided operand's last element loaded on its own: the
    // rings stop before the last k-row, which the tail's element loads keep)
    const bool ks_fix = (!OA::KC && (p.last_fix & 1)) || (!OB_::KC && (p.last_fix & 2));
    const int nk = ((KT && ks_fix) ? K - 1 : K) / (T::BK * P::U) * P::U;
    if (nk > 0) {
        // prologue: the loads of the virtual steps before step 0, then the
        // fragments of step 0
        constexpr int V0 = -(OA::NS * OA::D > OB_::NS * OB_::D ? OA::NS * OA::D : OB_::NS * OB_::D);
        static_for<V0, 0>([&](auto v_t) __attribute__((always_inline)) {
            constexpr int v = decltype(v_t)::value;
            if constexpr (OB_::issues_at(v) && OB_::first_loaded_at(v) >= 0)
                static_for<0, P::LB>([&](auto x) __attribute__((always_inline)) {
                    load_b(OB_::stage_of(OB_::first_loaded_at(v)), decltype(x)::value, kb);
                });
            if constexpr (OB_::issues_at(v) && OB_::first_loaded_at(v) >= 0) kb += b_kstep;
            if constexpr (OA::issues_at(v) && OA::first_loaded_at(v) >= 0)
                static_for<0, P::LA>([&](auto x) __attribute__((always_inline)) {
                    load_a(OA::stage_of(OA::first_loaded_at(v)), decltype(x)::value, ka);
                });
            if constexpr (OA::issues_at(v) && OA::first_loaded_at(v) >= 0) ka += a_kstep;
        });
        wait_vmcnt<P::after(0, 0)>();
        __syncthreads();
        static_for<0, NREAD>([&](auto r) __attribute__((always_inline)) { read_frag(IntTag<0>{}, 0, decltype(r)::value); });
        for (int s = 0; s < nk; s += P::U) static_for<0, P::U>([&](auto u) __attribute__((always_inline)) { step(u); });
        // no load may still be writing LDS when the workgroup ends
        wait_vmcnt<0>();
    }
    if constexpr (KT) {
        // the K tail: steps of 32 from k = 32 nk, fragments from global
        // memory through buffer loads over the same ranges as the rings'
        auto tail_rsrc = [&](const char* base, int64_t bytes, int pad) __attribute__((always_inline)) {
            const uint64_t a = (uint64_t)base;
            if (bytes > 0) bytes = (int64_t)(((a + (uint64_t)bytes + 3) & ~(uint64_t)3) - a) + pad;
            const int n = bytes <= 0 ? 0 : bytes > 0x7fffffffLL ? 0x7fffffff : (int)bytes;
            return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, n, 0x00020000);
        };
        const auto ta = tail_rsrc(a_start, a_bytes, p.range_pad_a);
        const auto tb = tail_rsrc(b_start, b_bytes, p.range_pad_b);
        // lane's 8 k (k ..) of row / column o (from the tile's corner)
        auto tail_frag = [&](auto op_t, const auto& rs, int o, int64_t ld, int k, bool fix) __attribute__((always_inline)) {
            using O = decltype(op_t);
            i16x8 v;
            if constexpr (O::KC) {
                v = __builtin_bit_cast(i16x8, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(((int64_t)o * ld + k) * 2), 0, 0));
                // element K - 1 of the row on its own (a 2-byte load ends
                // inside the range where the 4-byte part of the 16-byte one
                // would not): the operand's last element at 2 mod 4
                const int kk = K - 1 - k;
                if (fix && kk >= 0 && kk < 8) {
                    const short e = (short)__builtin_amdgcn_raw_buffer_load_b16(rs, (int)(((int64_t)o * ld + K - 1) * 2), 0, 0);
#pragma unroll
                    for (int t = 0; t < 8; ++t) v[t] = t == kk ? e : v[t];
                }
            } else {
#pragma unroll
                for (int t = 0; t < 8; ++t)
                    v[t] = (short)__builtin_amdgcn_raw_buffer_load_b16(rs, (int)(((int64_t)(k + t) * ld + o) * 2), 0, 0);
            }
            const int kv = K - k;  // elements of the 8 below K
#pragma unroll
            for (int t = 0; t < 8; ++t) v[t] = t < kv ? v[t] : (short)0;
            return v;
        };
        for (int k0 = nk * T::BK; k0 < K; k0 += T::BK) {
            const int k = k0 + 8 * q;
            static_for<0, T::FN>([&](auto j_t) __attribute__((always_inline)) {
                constexpr int j = decltype(j_t)::value;
                fb[0][j] = tail_frag(OB_{}, tb, wn * T::WTN + 16 * j + i16, ldb, k, (p.last_fix & 2) != 0);
            });
            static_for<0, T::FM>([&](auto i_t) __attribute__((always_inline)) {
                constexpr int i = decltype(i_t)::value;
                fa[0][i] = tail_frag(OA{}, ta, wm * T::WTM + 16 * i + i16, lda, k, (p.last_fix & 1) != 0);
            });
            static_for<0, NMF>([&](auto mt) __attribute__((always_inline)) { mfma_one(0, decltype(mt)::value); });
        }
    }

    // a7: epilogue.  acc[i][j] of lane l is C[row 16 i + l%16][columns
    // 16 j + 4 (l/16) .. +3] of the wave's block; fp32 -> fp16 / bf16 rounds
    // to nearest even.
    if constexpr (EPI) {
        // fused epilogue through the rings' LDS, once no wave reads it; the
        // tile's bias in an LDS array of its own
        __shared__ __attribute__((aligned(16))) float ebias_[T::BM + T::BN];
        lds_float* const ebias = (lds_float*)(lds_void*)ebias_;
        stage_bias<T::THREADS, T::BM, T::BN>(p, ebias, ebias + T::BN, m0, n0);
        __syncthreads();
        constexpr int REGION = P::LDS_BYTES / T::WAVES;  // bytes per wave
        constexpr int PB = REGION / 1024 < NMF ? REGION / 1024 : NMF;
        static_assert(PB >= 1 && NMF % PB == 0, "");
        lds_f32x4* region = (lds_f32x4*)(lds_void*)smem + wave * (REGION / 16);
        // Every block passes through VGPRs (free once the loop is done; an
        // empty asm): the blocks of the later passes, kept in the
        // accumulator registers across the first pass's loop, and the first
        // pass's, written to LDS straight from them, made the register
        // allocator move accumulators around inside the main loop (the
        // latter with column-major A and row-major B: 870 instructions and
        // 348 moves per loop trip against 469 and none).
        f32x4 held[NMF];
        static_for<0, NMF>([&](auto b_t) __attribute__((always_inline)) {
            constexpr int b = decltype(b_t)::value;
            held[b] = acc[b / T::FN][b % T::FN];
            asm volatile("" : "+v"(held[b]));
        });
        // any N and C alignment: the last group of a row may be partial
        // (element stores, in the run-time loop of values read back from
        // LDS, away from the accumulators) and C rows need not be aligned
        // for 4-element stores (p.vec_c)
        fused_epilogue<OUT, NMF, 4, PB, false>(
            p, region, ebias, ebias + T::BN, m0, n0,
            [&](auto b_t) { constexpr int b = decltype(b_t)::value; return held[b]; },
            [&](int b, int, int& row, int& col, int& n, bool& vec) {
                row = m0 + wm * T::WTM + 16 * (b / T::FN) + i16;
                col = n0 + wn * T::WTN + 16 * (b % T::FN) + 4 * q;
                n = row < p.M && col < p.N ? (p.N - col < 4 ? p.N - col : 4) : 0;
                vec = p.vec_c;
            });
        return;
    }
    constexpr int OB = out_bytes<OUT>();
    const int64_t ldc = p.ldc;
    // a tile on the bottom or right edge of C (M or N not a multiple of the
    // tile) stores only its groups inside C (N % 4 == 0: a group of four
    // columns is wholly inside or outside); its other rows and columns hold
    // products of zeros or of elements outside the tile's operand rows and
    // columns, never mixed into the stored ones.  (Element stores for a
    // partial group make the compiler move every accumulator to VGPRs ahead
    // of the stores, and spill.)  fp32 outputs pass through VGPRs (an empty
    // asm) as the converted 16-bit ones do: stored straight from the
    // accumulator registers, they made the register allocator move
    // accumulators around the main loop of the 256 x 256 kernel with
    // column-major A and row-major B (1049 instructions and 484 moves per
    // loop trip against 469 and none).
    static_for<0, NMF>([&](auto bt) __attribute__((always_inline)) {
        constexpr int i = decltype(bt)::value / T::FN, j = decltype(bt)::value % T::FN;
        const int row = m0 + wm * T::WTM + 16 * i + i16;
        const int col = n0 + wn * T::WTN + 16 * j + 4 * q;
        f32x4 v = acc[i][j];
        if constexpr (OUT == DT_F32) asm volatile("" : "+v"(v));
        if (row < p.M && col < p.N) store4<OUT>(C + ((int64_t)row * ldc + col) * OB, v[0], v[1], v[2], v[3], true);
    });
}

}  // namespace tgemm
