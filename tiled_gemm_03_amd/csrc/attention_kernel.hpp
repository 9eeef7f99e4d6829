// attention_kernel.hpp -- attention forward on the matrix-product pipeline
// of this library: O = softmax(scale Q K^T) V per (batch, head), computed
// blockwise with an online softmax (page "TileLang实战：用Python DSL自动生成
// 高性能GPU计算内核", §4.1 for the definition, §4.2 for the blockwise
// algorithm: walk K and V in blocks, keep per query the running maximum M,
// the normaliser L and the output, so that the Nq x Nk score matrix never
// exists in memory).
//
// One workgroup (4 waves) per 64 query rows of one (batch, head); wave w
// owns rows 16 w .. 16 w + 15.  Per block of 64 keys:
//   S = Q K^T      v_mfma_f32_16x16x32 with K (first operand) and Q (second):
//                  lane l holds S[row l % 16][keys 4 (l/16) .. +3] of each
//                  16-key group (Q stays in registers for the whole loop);
//   online softmax in fp32 with exp2 (the scale is folded into log2 e):
//                  m = max(m, rowmax), p = 2^(s - m), l = l 2^(m_old - m) +
//                  rowsum, O *= 2^(m_old - m); row reductions over the 4
//                  lanes that share a row;
//   O += P V       the same MFMA with V (first operand) and P (second).  The
//                  8 k-values a lane feeds per 32 keys are the keys it holds
//                  in S, 4 (l/16) .. +3 and 16 + 4 (l/16) .. +3, so P goes
//                  from the S registers straight into the MFMA; V is read in
//                  that key order with two transposing LDS reads (4 key rows
//                  each).
// K and V blocks go global -> registers -> LDS, the next block's loads in
// flight while the current one is computed.  LDS layouts (XOR swizzles, as
// the matrix-product kernels): K as [32 d][64 keys][64 bytes] with chunk
// c ^ ((key / 2) % 4) (a K fragment read is then the conflict-free read of
// the k-contiguous ring stage); V as [64 keys][d] with its 32-byte groups of
// row r at group g ^ f(r), f spreading the 8 rows of a half-wave's
// transposing read over the 8 bank groups.
//
// Masks: keys >= Nk (and, causal, keys > query) get score -inf; rows >= Nq
// are neither read nor written.  Rows with every key masked cannot occur
// (key 0 is visible to every query).
#pragma once
#include "gemm_kernel.hpp"

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
    int Nq, Nk;
    float scale_log2e;         // scale * log2(e)
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

// D: head dimension (64 or 128); IN: DT_F16 / DT_BF16; OUT: IN or DT_F32.
template <int D, int IN, int OUT, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2)))
void attention_kernel(AttnArgs p) {
    static_assert(D == 64 || D == 128, "");
    constexpr int BQ = 64, BKV = 64;
    constexpr int KS = D / 32;          // k-steps of the score product
    constexpr int DB = D / 16;          // 16-column blocks of the output
    constexpr int CPR = D / 8;          // 16-byte chunks per K / V row
    constexpr int LOADS = BKV * CPR / 256;  // chunks of K (and of V) per thread and block
    constexpr int K_BYTES = BKV * D * 2, V_BYTES = BKV * D * 2;
    __shared__ __attribute__((aligned(1024))) char smem[K_BYTES + V_BYTES];
    lds_attn_char* const lds = (lds_attn_char*)smem;
    lds_attn_char* const ks = lds;
    lds_attn_char* const vs = lds + K_BYTES;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int q = lane >> 4, i16 = lane & 15;
    const int qt = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int q0 = qt * BQ;
    const int Nq = p.Nq, Nk = p.Nk;
    const char* Qh = p.Q + (b * p.q_sb + h * p.q_sh) * 2;
    const char* Kh = p.K + (b * p.k_sb + h * p.k_sh) * 2;
    const char* Vh = p.V + (b * p.v_sb + h * p.v_sh) * 2;

    // Q fragments of this lane's row (zeros past Nq): d = 32 s + 8 q .. +7
    const int my_row = q0 + 16 * wave + i16;
    attn_i16x8 qf[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        u32x4 v = zero4();
        if (my_row < Nq) v = load16(Qh + ((int64_t)my_row * p.q_sn + 32 * s + 8 * q) * 2);
        qf[s] = __builtin_bit_cast(attn_i16x8, v);
    }

    // keys this workgroup needs: all, or (causal) up to its last row
    const int kmax = CAUSAL ? (q0 + BQ < Nk ? q0 + BQ : Nk) : Nk;
    const int nblocks = (kmax + BKV - 1) / BKV;

    // global -> registers: chunk x of this thread is row (tid + 256 x) / CPR,
    // chunk (tid + 256 x) % CPR of the block; zeros past Nk
    u32x4 kr[LOADS], vr[LOADS];
    auto load_block = [&](int kb) {
#pragma unroll
        for (int x = 0; x < LOADS; ++x) {
            const int idx = tid + 256 * x, r = idx / CPR, c = idx % CPR;
            const int key = kb * BKV + r;
            kr[x] = key < Nk ? load16(Kh + ((int64_t)key * p.k_sn + 8 * c) * 2) : zero4();
            vr[x] = key < Nk ? load16(Vh + ((int64_t)key * p.v_sn + 8 * c) * 2) : zero4();
        }
    };
    // registers -> LDS (swizzled)
    auto store_block = [&]() {
#pragma unroll
        for (int x = 0; x < LOADS; ++x) {
            const int idx = tid + 256 * x, r = idx / CPR, c = idx % CPR;
            // K: [d-step c/4][key r][chunk (c%4) ^ ((r/2)%4)]
            *(lds_attn_u32x4*)(ks + (c >> 2) * (BKV * 64) + r * 64 + (((c & 3) ^ ((r >> 1) & 3)) * 16)) = kr[x];
            // V: row r, 32-byte group (c/2) ^ f(r), half c % 2
            const int f = D == 128 ? (r & 7) : ((r >> 1) & 3);
            *(lds_attn_u32x4*)(vs + r * (D * 2) + (((c >> 1) ^ f) * 32) + (c & 1) * 16) = vr[x];
        }
    };

    // per-lane LDS bases of the fragment reads
    // K fragment (keys 16 g + l%16, d-step s, chunk q): ks + s*4096 + (16 g + l%16)*64 + (q ^ key)*16
    lds_attn_char* const kbase = ks + i16 * 64 + ((q ^ ((i16 >> 1) & 3)) * 16);
    // V fragment (keys 32 t + 4 q + i/4 [+16], columns 16 db + 4 (i%4) ..): one base per column block
    auto vaddr = [&](int t, int half, int db) __attribute__((always_inline)) {
        const int r = 32 * t + 16 * half + 4 * q + (i16 >> 2);
        const int c = 4 * db + (i16 & 3);  // 8-byte unit of the row: 16 db + 4 (i%4) columns
        const int g = c >> 2, f = D == 128 ? (r & 7) : ((r >> 1) & 3);
        return vs + r * (D * 2) + ((g ^ f) * 32) + (c & 3) * 8;
    };

    f32x4 o[DB];
#pragma unroll
    for (int j = 0; j < DB; ++j) o[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;
    const float sl2 = p.scale_log2e;

    if (nblocks > 0) load_block(0);
    for (int kb = 0; kb < nblocks; ++kb) {
        __syncthreads();  // every wave is done with the previous block's LDS
        store_block();
        __syncthreads();
        if (kb + 1 < nblocks) load_block(kb + 1);  // in flight during this block

        // S = Q K^T for the 4 key groups of 16
        f32x4 sc[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            sc[g] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const attn_i16x8 kf =
                    __builtin_bit_cast(attn_i16x8, *(const lds_attn_u32x4*)(kbase + s * (BKV * 64) + g * 1024));
                if constexpr (IN == DT_F16)
                    sc[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, kf),
                                                                   __builtin_bit_cast(f16x8, qf[s]), sc[g], 0, 0, 0);
                else
                    sc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kf),
                                                                    __builtin_bit_cast(bf16x8, qf[s]), sc[g], 0, 0, 0);
            }
        }
        // scale (in log2 units) and masks: key 16 g + 4 q + e of this block
        float mx = -INFINITY;
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int key = kb * BKV + 16 * g + 4 * q + e;
                bool hide = key >= Nk;
                if constexpr (CAUSAL) hide = hide || key > my_row;
                const float v = hide ? -INFINITY : sc[g][e] * sl2;
                sc[g][e] = v;
                mx = fmaxf(mx, v);
            }
        // row maximum over the 4 lanes of the row (lanes l, l ^ 16, l ^ 32, l ^ 48)
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;  // a row with nothing visible yet
        const float alpha = exp2f(m_run - m_use);               // 0 while m_run = -inf
        float rs = 0.f;
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float pv = exp2f(sc[g][e] - m_use);
                sc[g][e] = pv;
                rs += pv;
            }
        rs += __shfl_xor(rs, 16);
        rs += __shfl_xor(rs, 32);
        l_run = l_run * alpha + rs;
        m_run = m_new;
#pragma unroll
        for (int j = 0; j < DB; ++j) o[j] *= alpha;

        // O += P V, 32 keys at a time: P = this lane's keys 4q..4q+3 of
        // groups 2t and 2t+1
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const uint32_t w0 = attn_pack2<IN>(sc[2 * t][0], sc[2 * t][1]);
            const uint32_t w1 = attn_pack2<IN>(sc[2 * t][2], sc[2 * t][3]);
            const uint32_t w2 = attn_pack2<IN>(sc[2 * t + 1][0], sc[2 * t + 1][1]);
            const uint32_t w3 = attn_pack2<IN>(sc[2 * t + 1][2], sc[2 * t + 1][3]);
            const attn_i16x8 pf = __builtin_bit_cast(attn_i16x8, u32x4{w0, w1, w2, w3});
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const attn_i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_attn_i16x4*)vaddr(t, 0, db));
                const attn_i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_attn_i16x4*)vaddr(t, 1, db));
                const attn_i16x8 vf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                if constexpr (IN == DT_F16)
                    o[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, vf),
                                                                   __builtin_bit_cast(f16x8, pf), o[db], 0, 0, 0);
                else
                    o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vf),
                                                                    __builtin_bit_cast(bf16x8, pf), o[db], 0, 0, 0);
            }
        }
    }

    // epilogue: O / l, row my_row, columns 16 db + 4 q .. +3
    if (my_row < Nq) {
        const float inv = 1.f / l_run;
        constexpr int OB = OUT == DT_F32 ? 4 : 2;
        char* orow = p.O + ((b * p.o_sb + h * p.o_sh) + (int64_t)my_row * p.o_sn) * OB;
#pragma unroll
        for (int db = 0; db < DB; ++db)
            store4<OUT>(orow + (16 * db + 4 * q) * OB, o[db][0] * inv, o[db][1] * inv, o[db][2] * inv,
                        o[db][3] * inv, false);
    }
}

}  // namespace tgemm
