// attention_kernel.hpp -- attention forward on the matrix-product pipeline
// of this library: O = softmax(scale Q K^T) V per (batch, head), computed
// blockwise with an online softmax (page "TileLang实战：用Python DSL自动生成
// 高性能GPU计算内核", §4.1 for the definition, §4.2 for the blockwise
// algorithm: walk K and V in blocks, keep per query the running maximum M,
// the normaliser L and the output, so that the Nq x Nk score matrix never
// exists in memory).
//
// One workgroup of NW waves per 32 NW query rows of one (batch, head); wave w
// owns rows 32 w .. 32 w + 31 of the tile as two sets of 16 (every fragment
// read from LDS feeds two MFMAs).  Per block of 64 keys:
//   S = Q K^T      v_mfma_f32_16x16x32 with K (first operand) and Q (second):
//                  lane l holds S[row l % 16][keys 4 (l/16) .. +3] of each
//                  16-key group (Q stays in registers for the whole loop);
//   online softmax in fp32 with exp2 (c = |scale| log2 e; a negative scale
//                  flips the signs of Q, which is exact): p = 2^(c s - m).
//                  The reference point m of a row moves only when a score
//                  passes it by more than 2^8 (then m := the row maximum and
//                  O, L are scaled by 2^(m_old - m), in a branch of its own);
//                  in between p <= 2^8 and O, L keep accumulating against the
//                  old m (O / L does not depend on m).  L is the sum of the
//                  probabilities as rounded for the product with V (so the
//                  weights sum to 1 exactly), accumulated on the MFMA
//                  against a fragment of ones;
//   O += P V       the same MFMA with V (first operand) and P (second).  The
//                  8 k-values a lane feeds per 32 keys are the keys it holds
//                  in S, 4 (l/16) .. +3 and 16 + 4 (l/16) .. +3, so P goes
//                  from the S registers straight into the MFMA; V is read in
//                  that key order with two transposing LDS reads (4 key rows
//                  each).
// K and V blocks go global -> LDS directly (no registers) into rings of two
// LDS slots each, K two blocks ahead and V one (S of the next block is
// computed during this block's softmax), one barrier per block.  LDS layouts
// (XOR swizzles, as the matrix-product kernels): K as [d / 32][64 keys][64
// bytes] with chunk c ^ ((key / 2) % 4) (a K fragment read is the
// conflict-free read of the k-contiguous ring stage); V as [64 keys][d] with
// its 32-byte groups of row r at group g ^ f(r), f spreading the 8 rows of a
// half-wave's transposing read over the 8 bank groups.
//
// Masks (only in the blocks after those that every row of the tile sees
// whole: a separate loop): keys >= Nk, and keys > query when causal, get
// p = 0.  Rows >= Nq are computed on zero queries and not written.  Every row
// sees key 0, so the first block sets every row's reference point.
#pragma once
#include "gemm_kernel.hpp"
#include "gemm_kernel_ring.hpp"

namespace tgemm {

struct AttnArgs {
    const char* Q;
    const char* K;
    const char* V;
    char* O;
    int64_t q_sb, q_sh, q_sn;  // element strides: batch, head, row (the last dimension is contiguous)
    int64_t k_sb, k_sh, k_sn;
    int64_t v_sb, v_sh, v_sn;
    int64_t o_sb, o_sh, o_sn;
    int Nq, Nk, H;
    int tiles;                 // query tiles per (batch, head)
    int total;                 // B H tiles workgroups
    float c;                   // |scale| log2(e)
    uint32_t qsign;            // 0x80008000 when the scale is negative, else 0
};

typedef short attn_i16x4 __attribute__((ext_vector_type(4)));
typedef short attn_i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) attn_i16x4 lds_attn_i16x4;
typedef __attribute__((address_space(3))) u32x4 lds_attn_u32x4;
typedef __attribute__((address_space(3))) char lds_attn_char;

// fp32 pair -> two 16-bit values of type IN (round to nearest even)
template <int IN>
__device__ __forceinline__ uint32_t attn_pack2(float a, float b) {
    if constexpr (IN == DT_F16) return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, f16x2));
    else return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

template <int IN>
__device__ __forceinline__ f32x4 attn_mfma(attn_i16x8 a, attn_i16x8 b, f32x4 c) {
    if constexpr (IN == DT_F16)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                      0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                       0, 0, 0);
}

// Workgroup g -> (batch-head, query tile).  Workgroups are dispatched to the
// 8 XCDs in turn (g % 8); the map gives each XCD a contiguous run of tiles,
// so that the tiles of one head share that XCD's L2 for K and V.  Causal
// (the tile of query rows q0.. walks q0 / 64 + 1 key blocks): the longest
// tiles first, across the heads of the XCD's run when it holds whole heads
// (all their last tiles, then all their second to last, ...), else within
// each head.  Longest-first over the run measured 5% faster than per head
// on 4 x 16 heads of 4096 positions (275-281 against 292-294 us).
__device__ __forceinline__ void attn_tile_of(int g, int total, int tiles, bool reverse, int& bh, int& qt) {
    const int full = total & ~7;
    const int run = full >> 3;
    if (reverse && g < full && run % tiles == 0) {
        const int nh = run / tiles, pos = g >> 3;
        qt = tiles - 1 - pos / nh;
        bh = (g & 7) * nh + pos % nh;
        return;
    }
    int lin = g;
    if (g < full) lin = (g & 7) * run + (g >> 3);
    bh = lin / tiles;
    qt = lin - bh * tiles;
    if (reverse) qt = tiles - 1 - qt;
}

// LDS bytes of a workgroup: two blocks of 64 keys of K and two of V (per
// wave when the waves split the keys).
template <int D, int NW, bool SPLIT>
constexpr int attn_lds_bytes() { return (SPLIT ? NW : 1) * 4 * 64 * D * 2; }

typedef __attribute__((address_space(3))) float lds_attn_float;

// D: head dimension (64 or 128); IN: DT_F16 / DT_BF16; OUT: IN or DT_F32;
// NW: waves per workgroup, each with 32 query rows of its own (32 NW rows),
// or (SPLIT) all on the same 32 rows, wave w taking key blocks w, w + NW,
// w + 2 NW, ... through an LDS ring of its own, the partial results combined
// through LDS at the end (for grids too small to fill the CUs: the chain of
// key blocks a wave walks in sequence is NW times shorter).
template <int D, int IN, int OUT, bool CAUSAL, int NW, bool SPLIT>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * NW, 64 * NW), amdgpu_waves_per_eu(2)))
void attention_kernel(AttnArgs p) {
    static_assert(D == 64 || D == 128, "");
    constexpr int BQ = SPLIT ? 32 : 32 * NW, BKV = 64;
    constexpr int KS = D / 32;              // k-steps of the score product
    constexpr int DB = D / 16;              // 16-column blocks of the output
    constexpr int K_BYTES = BKV * D * 2, V_BYTES = BKV * D * 2, BUF = K_BYTES + V_BYTES;
    static_assert((SPLIT ? NW : 1) * 2 * BUF == attn_lds_bytes<D, NW, SPLIT>(), "");
    constexpr float TH = 8.f;               // reference-point slack (log2 units)
    constexpr bool PRIO_S = D == 64;        // raised wave priority from the S phase (else from PV)
    // dynamic LDS of attn_lds_bytes<D, NW, SPLIT>() bytes (declared at launch: a
    // static array this size would make the compiler budget registers for
    // the one wave per SIMD that it leaves room for, and move the
    // accumulators through AGPRs)
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    lds_attn_char* const lds = (lds_attn_char*)smem;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int q = lane >> 4, i16 = lane & 15;
    int bh, qt;
    attn_tile_of(blockIdx.x, p.total, p.tiles, CAUSAL, bh, qt);
    const int b = bh / p.H, h = bh - b * p.H;
    const int q0 = qt * BQ;
    const int Nq = p.Nq, Nk = p.Nk;
    const char* Qh = p.Q + (b * p.q_sb + h * p.q_sh) * 2;
    const char* Kh = p.K + (b * p.k_sb + h * p.k_sh) * 2;
    const char* Vh = p.V + (b * p.v_sb + h * p.v_sh) * 2;

    // Q fragments of this lane's rows (zeros past Nq): d = 32 s + 8 q .. +7
    const int w_row0 = SPLIT ? q0 : q0 + 32 * wave;  // first row of the wave
    int my_row[2];
    attn_i16x8 qf[2][KS];
#pragma unroll
    for (int rs = 0; rs < 2; ++rs) {
        my_row[rs] = w_row0 + 16 * rs + i16;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            u32x4 v = zero4();
            if (my_row[rs] < Nq) v = load16(Qh + ((int64_t)my_row[rs] * p.q_sn + 32 * s + 8 * q) * 2);
            v ^= p.qsign;
            qf[rs][s] = __builtin_bit_cast(attn_i16x8, v);
        }
    }

    // keys this workgroup needs: all, or (causal) up to its last row
    const int kmax = CAUSAL ? (q0 + BQ < Nk ? q0 + BQ : Nk) : Nk;
    const int nblocks = (kmax + BKV - 1) / BKV;

    // global -> LDS without registers: buffer_load_dwordx4 ... lds writes the
    // 16 bytes of lane l at LDS byte M0 + 16 l, so each lane loads the chunk
    // that the swizzled layout puts at its position.  A buffer resource per
    // block starts at the block's first key and ends at the head's last
    // element, so keys past Nk read as zeros (range check).  K: 1 KiB block j
    // holds d-step j / 4, keys 16 (j % 4) + l / 4, slot l % 4 = chunk
    // (l % 4) ^ ((key / 2) % 4).  V: block j holds rows RPB j + l / LPR, slot
    // l % LPR = 32-byte group (slot / 2) ^ f(row), half slot % 2.
    constexpr int NKB = BKV * D * 2 / 1024;  // 1 KiB blocks of K (and of V) per key block
    constexpr int PW = SPLIT ? NKB : NKB / NW;  // of them per wave
    static_assert(SPLIT || PW * NW == NKB, "");
    constexpr int LPR = D / 8, RPB = 64 / LPR;  // V: lanes per row, rows per 1 KiB
    // SPLIT: each wave's ring in its own part of the LDS
    const int ring0 = SPLIT ? wave * 2 * BUF : 0;
    const int smem_base = (int)(uintptr_t)(lds_void*)smem + ring0;
    int voff_k[PW], voff_v[PW];
#pragma unroll
    for (int x = 0; x < PW; ++x) {
        const int j = SPLIT ? x : wave * PW + x;
        {
            const int s = j >> 2, key = 16 * (j & 3) + (lane >> 2);
            const int chunk = (lane & 3) ^ ((key >> 1) & 3);
            voff_k[x] = (int)((int64_t)key * p.k_sn * 2) + (32 * s + 8 * chunk) * 2;
        }
        {
            const int row = RPB * j + lane / LPR, slot = lane % LPR;
            const int f = D == 128 ? (row & 7) : ((row >> 1) & 3);
            voff_v[x] = (int)((int64_t)row * p.v_sn * 2) + ((slot >> 1) ^ f) * 32 + (slot & 1) * 16;
        }
    }
    auto make_rsrc = [&](const char* base, int64_t bytes) __attribute__((always_inline)) {
        const uint64_t a = (uint64_t)base;
        const uint32_t n = bytes <= 0 ? 0u : bytes > 0xffffffffLL ? 0xffffffffu : (uint32_t)bytes;
        return i32x4{__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
                     __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32)),
                     __builtin_amdgcn_readfirstlane((int)n), 0x00020000};
    };
    // issued through inline asm: the compiler then adds no waits for these
    // loads before LDS reads; the kernel waits for them itself (vmcnt) before
    // the barrier that publishes a buffer.  The block writes M0 (the LDS
    // destination) and names M0 as its output operand (the compiler keeps
    // nothing of its own in M0 across it).
    auto dma = [&](int lds_addr, int vo, i32x4 rs) __attribute__((always_inline)) {
        int m0_written;
        asm volatile("s_mov_b32 m0, %1\n\tbuffer_load_dwordx4 %2, %3, %4 offen lds"
                     : "={m0}"(m0_written)
                     : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(vo), "s"(rs), "s"(0)
                     : "memory");
        (void)m0_written;
    };
    // The i-th key block a wave walks: block i, or (SPLIT) wave + NW i.  LDS:
    // K of walk positions i, i + 1 at (i % 2) K_BYTES, V at 2 K_BYTES +
    // (i % 2) V_BYTES (from the wave's ring)
    auto kb_of = [&](int i) __attribute__((always_inline)) { return SPLIT ? wave + NW * i : i; };
    const int blk0 = SPLIT ? 0 : wave * PW;  // first of this wave's 1 KiB blocks
    auto issue_k = [&](int i) __attribute__((always_inline)) {
        const int64_t k_rows = (int64_t)kb_of(i) * BKV;
        const i32x4 rk = make_rsrc(Kh + k_rows * p.k_sn * 2, ((Nk - 1 - k_rows) * p.k_sn + D) * 2);
        const int base = smem_base + (i & 1) * K_BYTES;
#pragma unroll
        for (int x = 0; x < PW; ++x) dma(base + (blk0 + x) * 1024, voff_k[x], rk);
    };
    auto issue_v = [&](int i) __attribute__((always_inline)) {
        const int64_t k_rows = (int64_t)kb_of(i) * BKV;
        const i32x4 rv = make_rsrc(Vh + k_rows * p.v_sn * 2, ((Nk - 1 - k_rows) * p.v_sn + D) * 2);
        const int base = smem_base + 2 * K_BYTES + (i & 1) * V_BYTES;
#pragma unroll
        for (int x = 0; x < PW; ++x) dma(base + (blk0 + x) * 1024, voff_v[x], rv);
    };
    lds_attn_char* const ring = lds + ring0;

    // per-lane LDS offsets of the fragment reads (within a block's K or V)
    // K fragment (keys 16 g + l%16, d-step s, chunk q): s*4096 + (16 g + l%16)*64 + (q ^ key)*16
    const int koff = i16 * 64 + ((q ^ ((i16 >> 1) & 3)) * 16);
    // V fragment (keys 32 t + 4 q + i/4 [+16], columns 16 db + 4 (i%4) ..)
    auto voff = [&](int t, int half, int db) __attribute__((always_inline)) {
        const int r = 32 * t + 16 * half + 4 * q + (i16 >> 2);
        const int c = 4 * db + (i16 & 3);  // 8-byte unit of the row: 16 db + 4 (i%4) columns
        const int g = c >> 2, f = D == 128 ? (r & 7) : ((r >> 1) & 3);
        return r * (D * 2) + ((g ^ f) * 32) + (c & 3) * 8;
    };

    f32x4 o[2][DB];
#pragma unroll
    for (int rs = 0; rs < 2; ++rs)
#pragma unroll
        for (int j = 0; j < DB; ++j) o[rs][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run[2] = {-INFINITY, -INFINITY};  // reference point (scaled, log2 units) of the lane's row
    // normaliser L = sum of the rounded probabilities, on the MFMA against a
    // fragment of ones (every element of the result is the row's sum)
    f32x4 lacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    const uint32_t one2 = IN == DT_F16 ? 0x3C003C00u : 0x3F803F80u;
    const attn_i16x8 ones = __builtin_bit_cast(attn_i16x8, u32x4{one2, one2, one2, one2});
    const float c = p.c;

    // blocks that need no mask for any row of the workgroup: every key
    // exists and (causal) is at most the tile's first row
    int plain = Nk / BKV;
    if (CAUSAL && (q0 + 1) / BKV < plain) plain = (q0 + 1) / BKV;
    if (plain > nblocks) plain = nblocks;
    // the blocks this wave walks, and how many of them are plain
    const int nwalk = SPLIT ? (nblocks > wave ? (nblocks - wave + NW - 1) / NW : 0) : nblocks;
    const int pwalk = SPLIT ? (plain > wave ? (plain - wave + NW - 1) / NW : 0) : plain;

    // S = Q K^T of walk position kb (K from its ring slot) into sc, both row sets
    auto scores = [&](int kb, f32x4 (&sc)[2][4]) __attribute__((always_inline)) {
        lds_attn_char* const kbase = ring + (kb & 1) * K_BYTES + koff;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            sc[0][g] = f32x4{0.f, 0.f, 0.f, 0.f};
            sc[1][g] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const attn_i16x8 kf =
                    __builtin_bit_cast(attn_i16x8, *(const lds_attn_u32x4*)(kbase + s * (BKV * 64) + g * 1024));
                sc[0][g] = attn_mfma<IN>(kf, qf[0][s], sc[0][g]);
                sc[1][g] = attn_mfma<IN>(kf, qf[1][s], sc[1][g]);
            }
        }
    };

    // Iteration kb: sc holds S(kb); the MFMAs of S(kb + 1) into nx run
    // beside the softmax of block kb (independent work for the matrix cores
    // while the SIMD computes exponentials), then O += P(kb) V(kb).  Loads:
    // K(kb + 2) into the slot S(kb) used, V(kb + 1) into the slot PV(kb - 1)
    // used (both finished before the previous barrier); the barrier at the
    // end publishes K(kb + 2) and V(kb + 1).  MASKED: keys past Nk and
    // (causal) keys past a row are hidden; compile-time variants in separate
    // loops, so that the main loop carries no mask code and no merge of its
    // registers.
    auto step = [&](int kb, f32x4 (&sc)[2][4], f32x4 (&nx)[2][4], auto masked_t) __attribute__((always_inline)) {
        constexpr bool MASKED = decltype(masked_t)::value;
        lds_attn_char* const knext = ring + ((kb + 1) & 1) * K_BYTES + koff;
        lds_attn_char* const vbase = ring + 2 * K_BYTES + (kb & 1) * V_BYTES;
        // K fragments of S(kb + 1), key group g, d-step s
        auto read_k = [&](int g, attn_i16x8 (&dst)[KS]) __attribute__((always_inline)) {
#pragma unroll
            for (int s = 0; s < KS; ++s)
                dst[s] = __builtin_bit_cast(attn_i16x8, *(const lds_attn_u32x4*)(knext + s * (BKV * 64) + g * 1024));
        };
        // V fragment u = DB t + db: keys 32 t + ..., columns 16 db + ...
        auto read_v = [&](int u) __attribute__((always_inline)) {
            const int t = u / DB, db = u % DB;
            const attn_i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_attn_i16x4*)(vbase + voff(t, 0, db)));
            const attn_i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_attn_i16x4*)(vbase + voff(t, 1, db)));
            return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        };
        constexpr int NU = 2 * DB;
        attn_i16x8 kf[2][KS], vf[3];
        read_k(0, kf[0]);
        if (kb + 2 < nwalk) issue_k(kb + 2);
        if (kb + 1 < nwalk) issue_v(kb + 1);
        const int key0 = kb_of(kb) * BKV;
        // row maxima of this lane's scores (hidden ones -inf)
        float mx[2];
#pragma unroll
        for (int rs = 0; rs < 2; ++rs) {
            mx[rs] = -INFINITY;
#pragma unroll
            for (int g = 0; g < 4; ++g)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if constexpr (MASKED) {
                        const int key = key0 + 16 * g + 4 * q + e;  // key of score e of group g
                        bool hide = key >= Nk;
                        if constexpr (CAUSAL) hide = hide || key > my_row[rs];
                        sc[rs][g][e] = hide ? -INFINITY : sc[rs][g][e];
                    }
                    mx[rs] = fmaxf(mx[rs], sc[rs][g][e]);
                }
        }
        // move the reference point when a score passes it by more than TH
        float mxc[2];
#pragma unroll
        for (int rs = 0; rs < 2; ++rs) mxc[rs] = mx[rs] == -INFINITY ? -INFINITY : mx[rs] * c;
        const bool up = mxc[0] > m_run[0] + TH || mxc[1] > m_run[1] + TH;
        if (__builtin_amdgcn_ballot_w64(up) != 0) {
            // a real branch (the volatile no-op cannot be speculated): the
            // rescale runs only when the reference point moves
            asm volatile("s_nop 0");
#pragma unroll
            for (int rs = 0; rs < 2; ++rs) {
                float rm = mxc[rs];
                rm = fmaxf(rm, __shfl_xor(rm, 16));
                rm = fmaxf(rm, __shfl_xor(rm, 32));
                const float m_new = fmaxf(m_run[rs], rm);
                const float alpha = __builtin_amdgcn_exp2f(m_run[rs] - m_new);  // 0 on the first block
                m_run[rs] = m_new;
#pragma unroll
                for (int j = 0; j < DB; ++j) o[rs][j] *= alpha;
                lacc[rs] *= alpha;
            }
        }
        // Wave priority 1 over the MFMA phases (measured: the S and PV
        // phases with head dimension 64, the PV phase alone with 128), 0
        // over the row maxima and the rescale, so that of the two waves on
        // a SIMD the one issuing MFMAs is served first.
        if constexpr (PRIO_S) __builtin_amdgcn_s_setprio(1);
        // S(kb + 1) on the matrix cores and p = 2^(c s - m) on the SIMD, one
        // key group at a time (each group's 2 KS MFMAs beside its 8 exp2).
        // On the last block the next scores come from a stale LDS slot and
        // are not used: no branch splits the interleaved code.  LDS reads run
        // ahead of the MFMAs that take them: the K fragments of group g + 1
        // are read before the MFMAs of group g (group 0's at the top of the
        // step, before the row maxima), the first two V fragments with group
        // 3, and each V fragment two MFMA pairs ahead.
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            if (g + 1 < 4) read_k(g + 1, kf[(g + 1) & 1]);
            if (g == 3) {
                vf[0] = read_v(0);
                vf[1] = read_v(1);
            }
            nx[0][g] = f32x4{0.f, 0.f, 0.f, 0.f};
            nx[1][g] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                nx[0][g] = attn_mfma<IN>(kf[g & 1][s], qf[0][s], nx[0][g]);
                nx[1][g] = attn_mfma<IN>(kf[g & 1][s], qf[1][s], nx[1][g]);
            }
#pragma unroll
            for (int rs = 0; rs < 2; ++rs)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float sv = sc[rs][g][e];
                    float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sv, c, -m_run[rs]));
                    if constexpr (MASKED) pv = sv == -INFINITY ? 0.f : pv;
                    sc[rs][g][e] = pv;
                }
            if constexpr (D == 128) __builtin_amdgcn_sched_barrier(0);
        }
        // O += P V, 32 keys at a time: P = this lane's keys 4q..4q+3 of
        // groups 2t and 2t+1; V fragment u = DB t + db in vf[u % 3]
        attn_i16x8 pf[2];
        if constexpr (!PRIO_S) __builtin_amdgcn_s_setprio(1);
        static_for<0, NU>([&](auto u_t) __attribute__((always_inline)) {
            constexpr int u = decltype(u_t)::value, t = u / DB, db = u % DB;
            if constexpr (db == 0) {
#pragma unroll
                for (int rs = 0; rs < 2; ++rs) {
                    const uint32_t w0 = attn_pack2<IN>(sc[rs][2 * t][0], sc[rs][2 * t][1]);
                    const uint32_t w1 = attn_pack2<IN>(sc[rs][2 * t][2], sc[rs][2 * t][3]);
                    const uint32_t w2 = attn_pack2<IN>(sc[rs][2 * t + 1][0], sc[rs][2 * t + 1][1]);
                    const uint32_t w3 = attn_pack2<IN>(sc[rs][2 * t + 1][2], sc[rs][2 * t + 1][3]);
                    pf[rs] = __builtin_bit_cast(attn_i16x8, u32x4{w0, w1, w2, w3});
                }
            }
            if constexpr (u + 2 < NU) vf[(u + 2) % 3] = read_v(u + 2);
            o[0][db] = attn_mfma<IN>(vf[u % 3], pf[0], o[0][db]);
            o[1][db] = attn_mfma<IN>(vf[u % 3], pf[1], o[1][db]);
            // each read two fragments ahead of its MFMAs (the compiler would
            // otherwise move the reads down to their MFMAs)
            if constexpr (db == 0) __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);  // the 8 packs
            if constexpr (u + 2 < NU) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            if constexpr (db == DB - 1) {
                lacc[0] = attn_mfma<IN>(ones, pf[0], lacc[0]);
                lacc[1] = attn_mfma<IN>(ones, pf[1], lacc[1]);
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                if constexpr (D == 128) __builtin_amdgcn_sched_barrier(0);
            }
        });
        __builtin_amdgcn_s_setprio(0);
        wait_vmcnt<0>();
        if constexpr (!SPLIT) __syncthreads();  // SPLIT: the ring is the wave's own
    };

    // two score buffers, alternating (the loops run two blocks per trip so
    // that each buffer keeps its registers)
    f32x4 sa[2][4], sb[2][4];
    if (nwalk > 0) {
        issue_k(0);
        issue_v(0);
        if (nwalk > 1) issue_k(1);
        wait_vmcnt<0>();
        if constexpr (!SPLIT) __syncthreads();
        scores(0, sa);
        if constexpr (!SPLIT) __syncthreads();  // every wave has read K(0) before K(2) replaces it
    }
    // S(kb) is in sa for even kb, in sb for odd kb: every call below has its
    // buffers fixed at compile time
    int kb = 0;  // walk position
    for (; kb + 1 < pwalk; kb += 2) {
        step(kb, sa, sb, BoolTag<false>{});
        step(kb + 1, sb, sa, BoolTag<false>{});
    }
    if (kb < pwalk) {
        step(kb, sa, sb, BoolTag<false>{});
        ++kb;
    }
    if (kb < nwalk && (kb & 1)) {
        step(kb, sb, sa, BoolTag<true>{});
        ++kb;
    }
    for (; kb + 1 < nwalk; kb += 2) {
        step(kb, sa, sb, BoolTag<true>{});
        step(kb + 1, sb, sa, BoolTag<true>{});
    }
    if (kb < nwalk) step(kb, sa, sb, BoolTag<true>{});

    // epilogue: O / L, row my_row, columns 16 db + 4 q .. +3
    constexpr int OB = OUT == DT_F32 ? 4 : 2;
    if constexpr (SPLIT) {
        // combine the waves' partial results: each wave's O, reference point
        // m and L (relative to m) through the LDS its ring used, then wave w
        // finishes column blocks w DB / NW ..: O = sum_w 2^(m_w - M) O_w over
        // sum_w 2^(m_w - M) L_w with M = max_w m_w (finite: wave 0 walks
        // block 0, whose key 0 every row sees; a wave that walked nothing
        // has m = -inf and weight 0)
        static_assert(DB % NW == 0, "");
        __syncthreads();  // every wave is done with its ring
        lds_f32x4* const co = (lds_f32x4*)(lds_void*)smem;  // [NW][2][DB][64]
        lds_attn_float* const cm = (lds_attn_float*)(lds + NW * 2 * DB * 64 * 16);  // [NW][2][64]
        lds_attn_float* const cl = cm + NW * 2 * 64;                               // [NW][2][64]
#pragma unroll
        for (int rs = 0; rs < 2; ++rs) {
#pragma unroll
            for (int db = 0; db < DB; ++db) co[((wave * 2 + rs) * DB + db) * 64 + lane] = o[rs][db];
            cm[(wave * 2 + rs) * 64 + lane] = m_run[rs];
            cl[(wave * 2 + rs) * 64 + lane] = lacc[rs][0];
        }
        __syncthreads();
#pragma unroll
        for (int rs = 0; rs < 2; ++rs) {
            float M = -INFINITY;
#pragma unroll
            for (int w = 0; w < NW; ++w) M = fmaxf(M, cm[(w * 2 + rs) * 64 + lane]);
            float wt[NW], L = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                const float mw = cm[(w * 2 + rs) * 64 + lane];
                wt[w] = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - M);
                L += wt[w] * cl[(w * 2 + rs) * 64 + lane];
            }
            if (my_row[rs] < Nq) {
                const float inv = 1.f / L;
                char* orow = p.O + ((b * p.o_sb + h * p.o_sh) + (int64_t)my_row[rs] * p.o_sn) * OB;
#pragma unroll
                for (int c = 0; c < DB / NW; ++c) {
                    const int db = wave * (DB / NW) + c;
                    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int w = 0; w < NW; ++w) acc += wt[w] * co[((w * 2 + rs) * DB + db) * 64 + lane];
                    store4<OUT>(orow + (16 * db + 4 * q) * OB, acc[0] * inv, acc[1] * inv, acc[2] * inv,
                                acc[3] * inv, false);
                }
            }
        }
        return;
    }
#pragma unroll
    for (int rs = 0; rs < 2; ++rs) {
        const float l = lacc[rs][0];
        if (my_row[rs] < Nq) {
            const float inv = 1.f / l;
            char* orow = p.O + ((b * p.o_sb + h * p.o_sh) + (int64_t)my_row[rs] * p.o_sn) * OB;
#pragma unroll
            for (int db = 0; db < DB; ++db)
                store4<OUT>(orow + (16 * db + 4 * q) * OB, o[rs][db][0] * inv, o[rs][db][1] * inv,
                            o[rs][db][2] * inv, o[rs][db][3] * inv, false);
        }
    }
}

}  // namespace tgemm
