// gemm_kernel.hpp -- the tiled matrix-product kernel family for gfx950 (CDNA4).
//
// One workgroup computes one BM x BN tile of C = A x B (row-major A: M x K,
// row-major B: K x N).  This is the tiled kernel of page "企业官网建设流程全解析"
// (a TileLang article despite its title), §3.3, rebuilt for gfx950:
//
//   a1  tile scheduling   workgroup id -> (tile_m, tile_n), remapped so that
//                         the workgroups that the hardware deals to one XCD
//                         (round robin over 8 XCDs) own neighbouring tiles
//                         and share that XCD's L2 (the "block_wise" mapping
//                         idea of page "TileLang：GPU异构计算的声明式分块编程
//                         范式", §3.3).
//   a2  global -> LDS     16-byte coalesced loads, staged in registers; rows
//                         or columns outside M / N / K are filled with zero.
//                         B arrives k-major and is transposed in registers
//                         (v_perm) so that both LDS tiles are k-contiguous,
//                         the operand layout the MFMA unit reads.
//   a3  LDS layout        16-byte chunks XOR-swizzled per row so that the
//                         lanes of one ds_read_b128 / ds_write_b128 hit
//                         distinct banks (the swizzled layout of §4.1 of the
//                         first page, re-derived for gfx950's LDS).
//   a4  pipeline          two LDS buffers + one register stage: while the
//                         MFMAs consume buffer k, the loads for step k+1 are
//                         in flight and are written to the other buffer; one
//                         barrier per K step (num_stages of §3.3 / §4.2).
//   a5  MFMA inner loop   v_mfma_f32_32x32x16_{f16,bf16}, or 4 x
//                         v_mfma_f32_32x32x2f32 for fp32 inputs.
//   a6  accumulator       fp32, in registers (AGPR/VGPR), zeroed before the
//                         K loop (T.clear of §3.3).
//   a7  epilogue          fp32 -> output type (round to nearest even), masked
//                         stores for ragged M / N (the edge masks of the
//                         DeepSeek/Ascend TileLang toolkit page, §5.2).
//
// The MFMA is fed with B as its first operand and A as its second, so the
// accumulator holds C transposed: each lane then owns 4 consecutive columns
// of one row of C and stores them with one 8- or 16-byte write.

#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tgemm {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

enum { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };

struct GemmArgs {
    const char* A;
    const char* B;
    char* C;
    int64_t lda, ldb, ldc;  // in elements
    int M, N, K;
    int tiles_m, tiles_n;
    int group_m;            // tile rows per raster group
    int swz_mask;           // CPR-1: XOR-swizzled LDS; 0: plain row-major LDS
};

// Compile-time tile configuration.
//   BM x BN   output tile of one workgroup
//   BK        K step (elements) per pipeline stage
//   WM x WN   wavefronts per workgroup along M and N
//   EB        bytes per input element (2: f16/bf16, 4: f32)
//   OCC       workgroups per CU the kernel is compiled for (register budget)
template <int BM_, int BN_, int BK_, int WM_, int WN_, int EB_, int OCC_>
struct TileCfg {
    static constexpr int BM = BM_, BN = BN_, BK = BK_;
    static constexpr int WM = WM_, WN = WN_;
    static constexpr int THREADS = 64 * WM * WN;
    static constexpr int WAVES = WM * WN;
    static constexpr int EB = EB_;
    static constexpr int OCC = OCC_;
    static constexpr int VE = 16 / EB;            // elements per 16-byte chunk
    static constexpr int RB = BK * EB;            // bytes per LDS row
    static constexpr int CPR = RB / 16;           // 16-byte chunks per LDS row
    static constexpr int WTM = BM / WM, WTN = BN / WN;  // wave tile
    static constexpr int FM = WTM / 32, FN = WTN / 32;  // 32x32 MFMA blocks per wave
    static constexpr int KG = 2 * VE;             // K covered by one fragment read
    static constexpr int NKG = BK / KG;
    static constexpr int A_BYTES = BM * RB;
    static constexpr int B_BYTES = BN * RB;
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    static constexpr int STAGES = 2;
    static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
    // A: 16-byte chunks per thread.  B: VE x VE blocks (VE rows of 16 bytes).
    static constexpr int A_CHUNKS = BM * CPR / THREADS;
    static constexpr int KBN = BK / VE;           // k-blocks of B per step
    static constexpr int B_TOTAL = KBN * (BN / VE);
    static constexpr int B_BLOCKS = (B_TOTAL + THREADS - 1) / THREADS;
    static_assert(CPR == 4 || CPR == 8, "LDS rows of 64 or 128 bytes");
    static_assert(BM * CPR % THREADS == 0, "A chunks must spread evenly");
    static_assert(THREADS % CPR == 0, "");
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile of whole MFMA blocks");
    static_assert(BK % KG == 0, "");
    static_assert(LDS_BYTES <= 160 * 1024, "gfx950 LDS is 160 KiB per CU");
};

// ---------------------------------------------------------------- a1
// Workgroup id -> output tile.  Workgroups are dealt to the 8 XCDs round
// robin, so ids b, b+8, b+16, ... run on one XCD: they are renumbered to
// consecutive tiles, which the grouped raster then packs into group_m-row
// blocks of tiles that share A and B panels in that XCD's L2.  The map is a
// bijection of [0, tiles_m * tiles_n).
__host__ __device__ inline void tile_of(int bid, int tiles_m, int tiles_n, int group_m,
                                        int& tm, int& tn) {
    const int total = tiles_m * tiles_n;
    const int full = total & ~7;
    int id = bid;
    if (bid < full) id = (bid & 7) * (full >> 3) + (bid >> 3);
    const int per_group = group_m * tiles_n;
    const int g = id / per_group;
    const int first_m = g * group_m;
    const int rows = tiles_m - first_m < group_m ? tiles_m - first_m : group_m;
    const int r = id - g * per_group;
    tm = first_m + r % rows;
    tn = r / rows;
}

// ---------------------------------------------------------------- a3
// Physical 16-byte chunk of logical chunk c in LDS row `row`.  With 128-byte
// rows (CPR 8) the XOR key is row%8 ^ (row/8)%2, with 64-byte rows it is
// (row/2)%4 ^ (row/8)%2: 8 consecutive rows (one 128-byte bank sweep) and 16
// consecutive rows (two sweeps) then both use every chunk slot once, for
// reads of consecutive rows at one chunk and for writes of whole rows.
template <int CPR>
__device__ __forceinline__ int swizzle_key(int row) {
    return ((row / (8 / CPR)) ^ ((row >> 3) & 1)) & (CPR - 1);
}

// ---------------------------------------------------------------- helpers
__device__ __forceinline__ u32x4 zero4() { return u32x4{0u, 0u, 0u, 0u}; }

// One 16-byte chunk holding VE consecutive elements starting at `p`, of which
// only the first `valid` exist (the rest read as zero).  Element-wise loads:
// used for ragged edges and for operands that are not 16-byte aligned.
template <int EB>
__device__ __forceinline__ u32x4 load_chunk_partial(const char* p, int valid) {
    u32x4 v = zero4();
    if constexpr (EB == 4) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (e < valid) v[e] = *(const uint32_t*)(p + 4 * e);
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (e < valid) {
                const uint32_t h = *(const uint16_t*)(p + 2 * e);
                v[e >> 1] |= h << (16 * (e & 1));
            }
    }
    return v;
}

// Transpose of a VE x VE block held as VE chunks (rows) into VE chunks
// (columns).  16-bit elements: 32 v_perm_b32; 32-bit elements: renaming only.
template <int EB>
__device__ __forceinline__ void transpose_block(const u32x4 (&in)[16 / EB], u32x4 (&out)[16 / EB]) {
    if constexpr (EB == 4) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int q = 0; q < 4; ++q) out[e][q] = in[q][e];
    } else {
        // column e, dword q = (row 2q, col e) | (row 2q+1, col e) << 16
#pragma unroll
        for (int e = 0; e < 8; ++e)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                out[e][q] = __builtin_amdgcn_perm(in[2 * q + 1][e >> 1], in[2 * q][e >> 1],
                                                  (e & 1) ? 0x07060302u : 0x05040100u);
    }
}

template <int OUT>
__device__ __forceinline__ void store4(char* p, float a, float b, float c, float d, bool vec) {
    if constexpr (OUT == DT_F32) {
        if (vec) {
            *(u32x4*)p = u32x4{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
                               __builtin_bit_cast(uint32_t, c), __builtin_bit_cast(uint32_t, d)};
        } else {
            ((float*)p)[0] = a; ((float*)p)[1] = b; ((float*)p)[2] = c; ((float*)p)[3] = d;
        }
    } else {
        uint16_t h[4];
        if constexpr (OUT == DT_F16) {
            h[0] = __builtin_bit_cast(uint16_t, (_Float16)a);
            h[1] = __builtin_bit_cast(uint16_t, (_Float16)b);
            h[2] = __builtin_bit_cast(uint16_t, (_Float16)c);
            h[3] = __builtin_bit_cast(uint16_t, (_Float16)d);
        } else {
            h[0] = __builtin_bit_cast(uint16_t, (__bf16)a);
            h[1] = __builtin_bit_cast(uint16_t, (__bf16)b);
            h[2] = __builtin_bit_cast(uint16_t, (__bf16)c);
            h[3] = __builtin_bit_cast(uint16_t, (__bf16)d);
        }
        if (vec) {
            *(u32x2*)p = u32x2{h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16)};
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) ((uint16_t*)p)[e] = h[e];
        }
    }
}

template <int OUT>
__device__ __forceinline__ void store_elem(char* p, float v) {
    if constexpr (OUT == DT_F32) *(float*)p = v;
    else if constexpr (OUT == DT_F16) *(_Float16*)p = (_Float16)v;
    else *(__bf16*)p = (__bf16)v;
}

// ---------------------------------------------------------------- kernel
// IN: input type, OUT: output type.  ALIGNED: A, B, C 16-byte aligned and
// lda, ldb multiples of a 16-byte chunk, ldc a multiple of 4 elements (then
// whole chunks are loaded and 4-element groups stored with vector
// instructions; otherwise every access is element-wise).
template <class T, int IN, int OUT, bool ALIGNED>
__global__ __attribute__((amdgpu_flat_work_group_size(T::THREADS, T::THREADS),
                          amdgpu_waves_per_eu(T::OCC * T::WAVES / 4 > 0 ? T::OCC * T::WAVES / 4 : 1)))
void gemm_kernel(GemmArgs p) {
    constexpr int EB = T::EB, VE = T::VE, CPR = T::CPR, RB = T::RB;
    __shared__ __attribute__((aligned(16))) char smem[T::LDS_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / T::WN, wn = wave % T::WN;

    // a1: which tile
    int tm, tn;
    tile_of(blockIdx.x, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
    const int m0 = tm * T::BM, n0 = tn * T::BN;
    const int M = p.M, N = p.N, K = p.K;
    const bool interior = (m0 + T::BM <= M) && (n0 + T::BN <= N);
    const int swz = p.swz_mask;

    // a2: per-thread load assignment
    // A chunk i: row tid/CPR + i*(THREADS/CPR), chunk tid%CPR
    const int a_row0 = tid / CPR, a_c = tid % CPR;
    // B block i: idx = tid + i*THREADS; k-block idx%KBN, n-block idx/KBN
    const char* Ab = p.A;
    const char* Bb = p.B;
    const int64_t lda = p.lda, ldb = p.ldb;

    u32x4 ra[T::A_CHUNKS];
    u32x4 rb[T::B_BLOCKS][VE];

    auto load_step = [&](int k0, bool check) {
#pragma unroll
        for (int i = 0; i < T::A_CHUNKS; ++i) {
            const int r = a_row0 + i * (T::THREADS / CPR);
            const int gm = m0 + r, gk = k0 + a_c * VE;
            const char* src = Ab + ((int64_t)gm * lda + gk) * EB;
            if (!check && ALIGNED) {
                ra[i] = *(const u32x4*)src;
            } else {
                const int valid = gm < M ? (K - gk < VE ? K - gk : VE) : 0;
                if (ALIGNED && valid == VE) ra[i] = *(const u32x4*)src;
                else ra[i] = valid > 0 ? load_chunk_partial<EB>(src, valid) : zero4();
            }
        }
#pragma unroll
        for (int i = 0; i < T::B_BLOCKS; ++i) {
            const int idx = tid + i * T::THREADS;
            const bool live = (T::B_TOTAL % T::THREADS == 0) || idx < T::B_TOTAL;
            const int kb = idx % T::KBN, nb = idx / T::KBN;
            const int gn = n0 + nb * VE;
#pragma unroll
            for (int j = 0; j < VE; ++j) {
                const int gk = k0 + kb * VE + j;
                const char* src = Bb + ((int64_t)gk * ldb + gn) * EB;
                if (!live) {
                    rb[i][j] = zero4();
                } else if (!check && ALIGNED) {
                    rb[i][j] = *(const u32x4*)src;
                } else {
                    const int valid = gk < K ? (N - gn < VE ? N - gn : VE) : 0;
                    if (ALIGNED && valid == VE) rb[i][j] = *(const u32x4*)src;
                    else rb[i][j] = valid > 0 ? load_chunk_partial<EB>(src, valid) : zero4();
                }
            }
        }
    };

    auto store_step = [&](int stage) {
        char* As = smem + stage * T::STAGE_BYTES;
        char* Bs = As + T::A_BYTES;
#pragma unroll
        for (int i = 0; i < T::A_CHUNKS; ++i) {
            const int r = a_row0 + i * (T::THREADS / CPR);
            const int pc = a_c ^ (swizzle_key<CPR>(r) & swz);
            *(u32x4*)(As + r * RB + pc * 16) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < T::B_BLOCKS; ++i) {
            const int idx = tid + i * T::THREADS;
            if ((T::B_TOTAL % T::THREADS == 0) || idx < T::B_TOTAL) {
                const int kb = idx % T::KBN, nb = idx / T::KBN;
                u32x4 cols[VE];
                transpose_block<EB>(rb[i], cols);
#pragma unroll
                for (int e = 0; e < VE; ++e) {
                    const int n = nb * VE + e;
                    const int pc = kb ^ (swizzle_key<CPR>(n) & swz);
                    *(u32x4*)(Bs + n * RB + pc * 16) = cols[e];
                }
            }
        }
    };

    // a6: accumulators
    f32x16 acc[T::FM][T::FN];
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int j = 0; j < T::FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // fragment addressing: row (lane & 31) of each 32-row block, chunk 2g + lane/32
    const int frow = lane & 31, fhalf = lane >> 5;
    const int a_frow0 = wm * T::WTM + frow;
    const int b_frow0 = wn * T::WTN + frow;
    // the swizzle key of a fragment row depends only on the lane: block
    // starts are multiples of 32
    const int fkey_a = swizzle_key<CPR>(a_frow0) & swz;
    const int fkey_b = swizzle_key<CPR>(b_frow0) & swz;

    auto compute_step = [&](int stage) {
        const char* As = smem + stage * T::STAGE_BYTES;
        const char* Bs = As + T::A_BYTES;
#pragma unroll
        for (int g = 0; g < T::NKG; ++g) {
            u32x4 af[T::FM], bf[T::FN];
            const int ca = ((2 * g + fhalf) ^ fkey_a) * 16;
            const int cb = ((2 * g + fhalf) ^ fkey_b) * 16;
#pragma unroll
            for (int i = 0; i < T::FM; ++i) af[i] = *(const u32x4*)(As + (a_frow0 + 32 * i) * RB + ca);
#pragma unroll
            for (int j = 0; j < T::FN; ++j) bf[j] = *(const u32x4*)(Bs + (b_frow0 + 32 * j) * RB + cb);
#pragma unroll
            for (int i = 0; i < T::FM; ++i)
#pragma unroll
                for (int j = 0; j < T::FN; ++j) {
                    if constexpr (IN == DT_F16) {
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                            __builtin_bit_cast(f16x8, bf[j]), __builtin_bit_cast(f16x8, af[i]), acc[i][j], 0, 0, 0);
                    } else if constexpr (IN == DT_BF16) {
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            __builtin_bit_cast(bf16x8, bf[j]), __builtin_bit_cast(bf16x8, af[i]), acc[i][j], 0, 0, 0);
                    } else {
                        // Bit-cast whole vectors, then index: a bit-cast of a
                        // single ext-vector element is lowered as a cast of
                        // element 0 by this compiler.
                        const f32x4 bv = __builtin_bit_cast(f32x4, bf[j]);
                        const f32x4 av = __builtin_bit_cast(f32x4, af[i]);
#pragma unroll
                        for (int s = 0; s < 4; ++s)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(bv[s], av[s], acc[i][j], 0, 0, 0);
                    }
                }
        }
    };

    // a4: pipeline
    const int nk = (K + T::BK - 1) / T::BK;
    const int kfull = K / T::BK;  // steps with no K tail
    if (nk > 0) {
        load_step(0, !interior || 0 >= kfull);
        store_step(0);
        if (nk > 1) load_step(T::BK, !interior || 1 >= kfull);
        __syncthreads();
        for (int kt = 0; kt < nk; ++kt) {
            compute_step(kt & 1);
            if (kt + 1 < nk) {
                store_step((kt + 1) & 1);
                if (kt + 2 < nk) load_step((kt + 2) * T::BK, !interior || kt + 2 >= kfull);
            }
            __syncthreads();
        }
    }

    // a7: epilogue.  acc[i][j][4q + e] = C[row][col + e] with
    // row = m0 + wm*WTM + 32 i + lane%32, col = n0 + wn*WTN + 32 j + 8 q + 4 (lane/32)
    constexpr int OB = OUT == DT_F32 ? 4 : 2;
    const int64_t ldc = p.ldc;
#pragma unroll
    for (int i = 0; i < T::FM; ++i) {
        const int row = m0 + a_frow0 + 32 * i;
#pragma unroll
        for (int j = 0; j < T::FN; ++j) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int col = n0 + wn * T::WTN + 32 * j + 8 * q + 4 * fhalf;
                char* dst = p.C + ((int64_t)row * ldc + col) * OB;
                const float v0 = acc[i][j][4 * q + 0], v1 = acc[i][j][4 * q + 1];
                const float v2 = acc[i][j][4 * q + 2], v3 = acc[i][j][4 * q + 3];
                if (interior && ALIGNED) {
                    store4<OUT>(dst, v0, v1, v2, v3, true);
                } else if (row < M) {
                    if (ALIGNED && col + 4 <= N) {
                        store4<OUT>(dst, v0, v1, v2, v3, true);
                    } else {
                        if (col + 0 < N) store_elem<OUT>(dst + 0 * OB, v0);
                        if (col + 1 < N) store_elem<OUT>(dst + 1 * OB, v1);
                        if (col + 2 < N) store_elem<OUT>(dst + 2 * OB, v2);
                        if (col + 3 < N) store_elem<OUT>(dst + 3 * OB, v3);
                    }
                }
            }
        }
    }
}

}  // namespace tgemm
