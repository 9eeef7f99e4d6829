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

// element types; DT_FP8: an 8-bit floating-point output (output only, with
// the fused epilogue's kernels), its format OCP E4M3 or E5M2 chosen at run
// time by GemmArgs::fp8_e5m2
enum { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2, DT_FP8 = 3 };

// bytes per output element
template <int OUT>
__host__ __device__ constexpr int out_bytes() {
    return OUT == DT_F32 ? 4 : OUT == DT_FP8 ? 1 : 2;
}

struct GemmArgs {
    const char* A;
    const char* B;
    char* C;
    int64_t lda, ldb, ldc;  // in elements
    int M, N, K;
    int tiles_m, tiles_n;
    int group_m;            // tile rows per raster group
    int swz_mask;           // CPR-1: XOR-swizzled LDS; 0: plain row-major LDS
    int vec_ab;             // GENERAL kernels: A, B 16-byte aligned, lda, ldb whole chunks
    int vec_c;              // GENERAL kernels: C rows allow 4-element vector stores
    // fused epilogue (epi != 0): C := act(alpha * AB + beta * C + bias)
    int epi;
    float alpha, beta;      // beta == 0: C is not read
    const char* bias;       // bias_kind BIAS_ROW: M values, BIAS_COL: N values, of type bias_dt
    int bias_kind, bias_dt, act;
    int fp8_e5m2;           // DT_FP8 output: 0 = E4M3, 1 = E5M2
    // ring kernels: bytes added to A's / B's buffer range past its dword
    // rounding (0, or 2 when the last element would otherwise be dropped;
    // the host checks that they lie in the last element's page)
    int range_pad_a, range_pad_b;
    // ring kernels: bit 0 (A) / bit 1 (B): the operand's last element cannot
    // be kept by a pad (the 2 bytes after it start a new page); the K tail
    // loads it on its own, and a k-strided operand's last k-row is left to
    // the tail (the host then runs the KT variant)
    int last_fix;
    // split-K (ring kernels, plain fp32 output): splits > 1 slices of K of
    // k_split elements (the last one the rest), slice s written to C plus
    // s * split_stride bytes
    int splits, k_split;
    int64_t split_stride;
};

enum { ACT_NONE = 0, ACT_RELU = 1, ACT_GELU = 2, ACT_GELU_TANH = 3, ACT_SILU = 4 };
enum { BIAS_NONE = 0, BIAS_ROW = 1, BIAS_COL = 2 };

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
    static_assert(NKG >= 2 && NKG % 2 == 0, "fragment buffers alternate over an even number of k-groups");
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
template <bool B>
struct BoolTag {
    static constexpr bool value = B;
};
template <int I>
struct IntTag {
    static constexpr int value = I;
};

// f(IntTag<i>{}) for i = B .. E-1, expanded at compile time (register
// arrays are then only ever indexed by constants).
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(IntTag<B>{});
        static_for<B + 1, E>(f);
    }
}

__device__ __forceinline__ u32x4 zero4() { return u32x4{0u, 0u, 0u, 0u}; }

// 16 bytes from any element-aligned address: gfx950 runs in unaligned-access
// mode, so this is one global_load_dwordx4 whatever the alignment.
__device__ __forceinline__ u32x4 load16(const char* p) {
    u32x4 v;
    __builtin_memcpy(&v, p, 16);
    return v;
}

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

// Column e of a VE x VE block held as VE chunks (rows), as one chunk: the
// block's transpose, one row at a time.  16-bit elements: 4 v_perm_b32
// (dword q = (row 2q, col e) | (row 2q+1, col e) << 16); 32-bit elements:
// renaming only.
template <int EB>
__device__ __forceinline__ u32x4 transpose_col(const u32x4 (&in)[16 / EB], int e) {
    u32x4 out;
    if constexpr (EB == 4) {
#pragma unroll
        for (int q = 0; q < 4; ++q) out[q] = in[q][e];
    } else {
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
        for (int q = 0; q < 4; ++q) out[q] = __builtin_amdgcn_perm(in[2 * q + 1][e >> 1], in[2 * q][e >> 1], sel);
    }
    return out;
}

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------- 8-bit outputs
// The OCP 8-bit floating-point formats.  E4M3: 1 sign, 4 exponent (bias 7)
// and 3 fraction bits, no infinity, S.1111.111 NaN, largest finite value
// 1.75 * 2^8 = 448.  E5M2: 1 sign, 5 exponent (bias 15) and 2 fraction bits,
// IEEE-like (exponent 31: infinity or NaN), largest finite 1.75 * 2^15 =
// 57344.  Below 2^(1 - bias) the values are multiples of the subnormal
// spacing 2^(1 - bias - F).
//
// fp32 -> 8 bits: nearest, ties to even; magnitudes beyond the largest finite
// value, infinities included, become the largest finite value of the sign
// (the saturating conversion); NaN becomes the all-ones pattern with the sign.
// The rounding is the hardware conversion's (v_cvt_pk_fp8_f32 /
// v_cvt_pk_bf8_f32), which agrees with this definition for every value up to
// the largest finite one (checked on gfx950 over a stride of all fp32
// patterns, every midpoint between 8-bit values, subnormals and zeros); above
// it the instruction gives NaN (E4M3) or infinity (E5M2), so the input is
// clamped first, and NaN is set apart (the instruction drops its sign).
__device__ __forceinline__ float fp8_clamp(float x, int e5m2) {
    const float mx = e5m2 ? 57344.f : 448.f;
    return fminf(fmaxf(x, -mx), mx);
}
__device__ __forceinline__ uint32_t fp8_nan(float x) {
    return ((__builtin_bit_cast(uint32_t, x) >> 24) & 0x80u) | 0x7fu;
}
__device__ __forceinline__ uint32_t to_fp8(float x, int e5m2) {
    const float c = fp8_clamp(x, e5m2);
    const uint32_t r = (uint32_t)(e5m2 ? __builtin_amdgcn_cvt_pk_bf8_f32(c, 0.f, 0, false)
                                       : __builtin_amdgcn_cvt_pk_fp8_f32(c, 0.f, 0, false)) & 0xffu;
    return x != x ? fp8_nan(x) : r;
}
// four values -> their four 8-bit patterns, a in the low byte
__device__ __forceinline__ uint32_t to_fp8x4(float a, float b, float c, float d, int e5m2) {
    const float ca = fp8_clamp(a, e5m2), cb = fp8_clamp(b, e5m2), cc = fp8_clamp(c, e5m2), cd = fp8_clamp(d, e5m2);
    uint32_t w;
    if (e5m2) {
        w = (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(ca, cb, 0, false);
        w = (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(cc, cd, (int)w, true);
    } else {
        w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(ca, cb, 0, false);
        w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(cc, cd, (int)w, true);
    }
    if (a != a) w = (w & 0xffffff00u) | fp8_nan(a);
    if (b != b) w = (w & 0xffff00ffu) | (fp8_nan(b) << 8);
    if (c != c) w = (w & 0xff00ffffu) | (fp8_nan(c) << 16);
    if (d != d) w = (w & 0x00ffffffu) | (fp8_nan(d) << 24);
    return w;
}
__device__ __forceinline__ float from_fp8(uint32_t b, int e5m2) {
    if (e5m2) {
        // an E5M2 pattern is the upper byte of the binary16 of the same value
        return (float)__builtin_bit_cast(_Float16, (uint16_t)(b << 8));
    }
    const uint32_t sign = (b & 0x80u) << 24, e = (b >> 3) & 15u, m = b & 7u;
    if (e == 15u && m == 7u) return __builtin_bit_cast(float, sign | 0x7fc00000u);
    if (e == 0u) return __builtin_bit_cast(float, sign | __builtin_bit_cast(uint32_t, (float)m * 0.001953125f));
    return __builtin_bit_cast(float, sign | ((e + 120u) << 23) | (m << 20));
}

// Four consecutive outputs; fp32 -> fp16 / bf16 rounds to nearest even, fp32
// -> 8 bits as to_fp8 (fp8_e5m2 picks the format).
template <int OUT>
__device__ __forceinline__ void store4(char* p, float a, float b, float c, float d, bool vec, int fp8_e5m2 = 0) {
    if constexpr (OUT == DT_FP8) {
        const uint32_t w = to_fp8x4(a, b, c, d, fp8_e5m2);
        if (vec) *(uint32_t*)p = w;
        else __builtin_memcpy(p, &w, 4);
    } else if constexpr (OUT == DT_F32) {
        if (vec) {
            *(f32x4*)p = f32x4{a, b, c, d};
        } else {
            const f32x4 v = f32x4{a, b, c, d};
            __builtin_memcpy(p, &v, 16);  // one unaligned store (unaligned-access mode)
        }
    } else {
        uint32_t lo, hi;
        if constexpr (OUT == DT_F16) {
            lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, f16x2));
            hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{c, d}, f16x2));
        } else {
            lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
            hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{c, d}, bf16x2));
        }
        if (vec) {
            *(u32x2*)p = u32x2{lo, hi};
        } else {
            const u32x2 v = u32x2{lo, hi};
            __builtin_memcpy(p, &v, 8);
        }
    }
}

template <int OUT>
__device__ __forceinline__ void store_elem(char* p, float v, int fp8_e5m2 = 0) {
    if constexpr (OUT == DT_FP8) *(uint8_t*)p = (uint8_t)to_fp8(v, fp8_e5m2);
    else if constexpr (OUT == DT_F32) *(float*)p = v;
    else if constexpr (OUT == DT_F16) *(_Float16*)p = (_Float16)v;
    else *(__bf16*)p = (__bf16)v;
}

// ------------------------------------------------------- fused epilogue
// The operator fusion of page "企业官网建设流程全解析" §6.2 (further
// operators merged into the product's kernel, so that the product makes no
// round trip through memory), with the usual operators after a matrix
// product: C := act(alpha * AB + beta * C + bias), bias one value per row or
// per column of C, in fp32 before the output rounding.

__device__ __forceinline__ float load_value(const char* p, int64_t i, int dt, int fp8_e5m2 = 0) {
    if (dt == DT_FP8) return from_fp8(((const uint8_t*)p)[i], fp8_e5m2);
    if (dt == DT_F32) return ((const float*)p)[i];
    if (dt == DT_F16) return (float)((const _Float16*)p)[i];
    return (float)((const __bf16*)p)[i];
}

// relu(x) = max(x, 0); gelu(x) = x Phi(x) = x/2 (1 + erf(x / sqrt 2));
// gelu_tanh(x) = x/2 (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))) (the tanh
// approximation of gelu); silu(x) = x / (1 + exp(-x)).  Since
// (1 + tanh u) / 2 = 1 / (1 + exp(-2u)), gelu_tanh and silu are both x times
// a logistic function, evaluated with the hardware exp2 and reciprocal
// (a few ulp; exp2 overflowing to +inf gives the limit 0).
__device__ __forceinline__ float logistic_times(float x, float z) {  // x / (1 + exp(-z))
    return x * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-1.4426950408889634f * z));
}
template <int ACT>
__device__ __forceinline__ float activate_t(float x) {
    if constexpr (ACT == ACT_RELU) return x > 0.f ? x : 0.f;
    else if constexpr (ACT == ACT_GELU) return 0.5f * x * (1.f + erff(x * 0.70710678118654752f));
    else if constexpr (ACT == ACT_GELU_TANH) return logistic_times(x, 1.5957691216057308f * (x + 0.044715f * x * x * x));
    else if constexpr (ACT == ACT_SILU) return logistic_times(x, x);
    else return x;
}
__device__ __forceinline__ float activate(float x, int act) {
    switch (act) {
        case ACT_RELU: return activate_t<ACT_RELU>(x);
        case ACT_GELU: return activate_t<ACT_GELU>(x);
        case ACT_GELU_TANH: return activate_t<ACT_GELU_TANH>(x);
        case ACT_SILU: return activate_t<ACT_SILU>(x);
        default: return x;
    }
}

// Four consecutive elements of type dt from any element-aligned address, as
// fp32 (one load: unaligned-access mode).
__device__ __forceinline__ f32x4 load4_values(const char* p, int dt, int fp8_e5m2 = 0) {
    if (dt == DT_FP8) {
        uint32_t w;
        __builtin_memcpy(&w, p, 4);
        return f32x4{from_fp8(w & 0xffu, fp8_e5m2), from_fp8((w >> 8) & 0xffu, fp8_e5m2),
                     from_fp8((w >> 16) & 0xffu, fp8_e5m2), from_fp8(w >> 24, fp8_e5m2)};
    }
    if (dt == DT_F32) {
        f32x4 v;
        __builtin_memcpy(&v, p, 16);
        return v;
    }
    // one 64-bit scalar split by shifts: a memcpy into a two-dword vector
    // followed by an element read loads only the first dword (hipcc 7.2)
    uint64_t w;
    __builtin_memcpy(&w, p, 8);
    const uint32_t lo = (uint32_t)w, hi = (uint32_t)(w >> 32);
    if (dt == DT_F16) {
        const f16x2 a = __builtin_bit_cast(f16x2, lo), b = __builtin_bit_cast(f16x2, hi);
        return f32x4{(float)a[0], (float)a[1], (float)b[0], (float)b[1]};
    }
    const bf16x2 a = __builtin_bit_cast(bf16x2, lo), b = __builtin_bit_cast(bf16x2, hi);
    return f32x4{(float)a[0], (float)a[1], (float)b[0], (float)b[1]};
}

// The epilogue of four consecutive outputs C[row][col .. col + 3], of which
// the first n (> 0) lie inside C, in two halves: fused_pre forms
// alpha * AB + beta * C + bias (whole groups with one load of C and one of
// the bias), fused_post applies the activation and stores (vec: 4-element
// vector store).  Kernels with many groups per lane run the first half for
// a whole batch of groups before the second, so that the loads of the batch
// are in flight together.
// A float kernel argument (uniform) as a value of its own, through
// readfirstlane.  Multiplied into a vector straight from the argument, its
// read is widened by the compiler into one vector read of it and its
// neighbours (alpha, beta, the bias pointer); the kernel's copy of those
// arguments then stays in memory, promoted to a per-thread LDS array whose
// indexing makes every wave read the workgroup size from the dispatch packet
// at its start and wait for it: ~10 us per wave of workgroups, measured on
// every fused-epilogue kernel (2048^3 with the identity epilogue: 37.6 us
// against 27.4 us once the arguments pass through here).
__device__ __forceinline__ float arg_value(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
}

template <int OUT>
__device__ __forceinline__ f32x4 fused_pre(const GemmArgs& p, int row, int col, int n, f32x4 v) {
    constexpr int OB = out_bytes<OUT>();
    const char* src = p.C + ((int64_t)row * p.ldc + col) * OB;
    const int beb = p.bias_dt == DT_F32 ? 4 : 2;
    const float alpha = arg_value(p.alpha), beta = arg_value(p.beta);
    f32x4 t = v * alpha;
    if (n == 4) {
        if (beta != 0.f) t += beta * load4_values(src, OUT, p.fp8_e5m2);
        if (p.bias_kind == BIAS_COL) t += load4_values(p.bias + (int64_t)col * beb, p.bias_dt);
    } else {
#pragma unroll
        for (int e = 0; e < 3; ++e) {
            if (e >= n) break;
            if (beta != 0.f) t[e] += beta * load_value(src, e, OUT, p.fp8_e5m2);
            if (p.bias_kind == BIAS_COL) t[e] += load_value(p.bias, col + e, p.bias_dt);
        }
    }
    if (p.bias_kind == BIAS_ROW) t += load_value(p.bias, row, p.bias_dt);
    return t;
}

template <int OUT>
__device__ __forceinline__ void fused_post(const GemmArgs& p, int row, int col, int n, bool vec, f32x4 t) {
    constexpr int OB = out_bytes<OUT>();
    char* dst = p.C + ((int64_t)row * p.ldc + col) * OB;
    float o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = activate(t[e], p.act);
    if (n == 4) {
        store4<OUT>(dst, o[0], o[1], o[2], o[3], vec, p.fp8_e5m2);
    } else {
#pragma unroll
        for (int e = 0; e < 3; ++e)
            if (e < n) store_elem<OUT>(dst + e * OB, o[e], p.fp8_e5m2);
    }
}

template <int OUT>
__device__ __forceinline__ void store4_fused(const GemmArgs& p, int row, int col, int n, bool vec, f32x4 v) {
    fused_post<OUT>(p, row, col, n, vec, fused_pre<OUT>(p, row, col, n, v));
}

// The fused epilogue of a wave's NB accumulator blocks of VPL fp32 values
// per lane (VPL / 4 groups of 4 consecutive columns), through this wave's LDS
// region, PB blocks (a pass) at a time.  get(IntTag<b>): block b's values;
// where(b, g, row, col, n, vec): the output position of group g of block b
// (n outputs inside C, 0: nothing to store; vec: 4-element vector stores).
// The caller has made sure that no wave still reads the LDS it reuses, and
// has staged the workgroup tile's bias (stage_bias) in LDS.
//
// Every decision that depends on the epilogue's arguments (beta, the bias,
// its kind and type, the activation) is taken at run time and is the same for
// every lane; the code that takes it exists once per kernel, in loops, so
// that the epilogue runs a few thousand instructions per wave rather than one
// copy of every branch per group.  Per pass:
//  1. the pass's accumulators go to the region (compile-time register
//     indices, no loads), group i at region[64 i + lane];
//  2. when C is read (beta != 0), the whole groups are taken EB at a time:
//     the old C of all EB is loaded together (one wait), then each group's
//     alpha * acc + beta * C + bias (the bias from LDS) is written back in
//     place;
//  3. one loop over the whole groups, compiled once per activation and
//     chosen by one uniform switch, applies alpha and the bias (when step 2
//     did not run), the activation and the output rounding, and stores; then
//     the partial groups (n < 4) are formed and stored element by element.
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
typedef __attribute__((address_space(3))) float lds_float;

// The bias of a workgroup tile (rows m0 .. m0 + BM - 1, columns n0 .. n0 +
// BN - 1) as fp32 in LDS: bias_col[j] for column n0 + j (BIAS_COL), bias_row[i]
// for row m0 + i (BIAS_ROW); the array of the other kind, and entries past M
// or N, hold zeros.  Every thread of the workgroup takes part; a barrier must
// follow before the values are read.
template <int THREADS, int BM, int BN>
__device__ __forceinline__ void stage_bias(const GemmArgs& p, lds_float* bias_col, lds_float* bias_row, int m0, int n0) {
    for (int j = threadIdx.x; j < BN; j += THREADS)
        bias_col[j] = p.bias_kind == BIAS_COL && n0 + j < p.N ? load_value(p.bias, n0 + j, p.bias_dt) : 0.f;
    for (int i = threadIdx.x; i < BM; i += THREADS)
        bias_row[i] = p.bias_kind == BIAS_ROW && m0 + i < p.M ? load_value(p.bias, m0 + i, p.bias_dt) : 0.f;
}

// The old C of one whole group (4 outputs), raw: one register of a type fixed
// by the output type, so that several groups' loads can be in flight at once.
template <int OUT>
struct RawC {
    typedef uint64_t type;   // 16-bit outputs: 4 x 16 bits
};
template <>
struct RawC<DT_F32> {
    typedef f32x4 type;
};
template <>
struct RawC<DT_FP8> {
    typedef uint32_t type;
};

template <int OUT>
__device__ __forceinline__ typename RawC<OUT>::type load_raw_c(const char* src) {
    typename RawC<OUT>::type v;
    __builtin_memcpy(&v, src, sizeof(v));
    return v;
}

template <int OUT>
__device__ __forceinline__ f32x4 raw_c_values(typename RawC<OUT>::type w, int fp8_e5m2) {
    if constexpr (OUT == DT_F32) {
        return w;
    } else if constexpr (OUT == DT_FP8) {
        return f32x4{from_fp8(w & 0xffu, fp8_e5m2), from_fp8((w >> 8) & 0xffu, fp8_e5m2),
                     from_fp8((w >> 16) & 0xffu, fp8_e5m2), from_fp8(w >> 24, fp8_e5m2)};
    } else {
        // the two halves of the 64-bit scalar by shifts (a two-dword vector
        // read element by element is miscompiled by hipcc 7.2: the second
        // dword is taken from the first)
        const uint32_t lo = (uint32_t)w, hi = (uint32_t)(w >> 32);
        if constexpr (OUT == DT_F16) {
            const f16x2 a = __builtin_bit_cast(f16x2, lo), b = __builtin_bit_cast(f16x2, hi);
            return f32x4{(float)a[0], (float)a[1], (float)b[0], (float)b[1]};
        } else {
            return f32x4{__builtin_bit_cast(float, lo << 16), __builtin_bit_cast(float, lo & 0xffff0000u),
                         __builtin_bit_cast(float, hi << 16), __builtin_bit_cast(float, hi & 0xffff0000u)};
        }
    }
}

// WHOLE: every group is wholly inside C or wholly outside (n is 4 or 0), so
// the partial-group code is not compiled.  row0 / col0: the first row and
// column of the workgroup tile (the origin of the staged bias).
template <int OUT, int NB, int VPL, int PB, bool WHOLE, class Get, class Where>
__device__ __forceinline__ void fused_epilogue(const GemmArgs& p, lds_f32x4* region, const lds_float* bias_col,
                                               const lds_float* bias_row, int row0, int col0, Get&& get,
                                               Where&& where) {
    static_assert(NB % PB == 0 && VPL % 4 == 0, "");
    constexpr int G = VPL / 4;   // groups per block
    constexpr int NG = PB * G;   // groups per pass
    // groups whose loads of C are in flight together (16 measured no faster
    // at 8192^3; 32 made the compiler move accumulators in the main loop)
    constexpr int EB = NG < 8 ? NG : 8;
    static_assert(NG % EB == 0, "");
    constexpr int OB = out_bytes<OUT>();
    const int lane = threadIdx.x & 63;
    const float alpha = arg_value(p.alpha), beta = arg_value(p.beta);
    const bool rd_c = beta != 0.f;
    const bool has_bias = p.bias_kind != BIAS_NONE;
    // step 2 runs only when C is read; a bias alone is added in step 3
    const bool combine = rd_c;
    static_for<0, NB / PB>([&](auto pass_t) {
        constexpr int b0 = decltype(pass_t)::value * PB;
        // 1: the pass's accumulators into the region
        static_for<0, PB>([&](auto t_t) {
            constexpr int t = decltype(t_t)::value;
            const auto blk = get(IntTag<b0 + t>{});
            static_for<0, G>([&](auto g_t) {
                constexpr int g = decltype(g_t)::value;
                region[(t * G + g) * 64 + lane] = f32x4{blk[4 * g + 0], blk[4 * g + 1], blk[4 * g + 2], blk[4 * g + 3]};
            });
        });
        // The steps pass their values through the region, not through
        // registers the compiler forwards them in: forwarded across step 2,
        // hipcc 7.2 wrote one group's first value into all four of its
        // accumulator registers (the 32 x 32 register-staged kernel with C
        // and a bias).  A compiler barrier between the steps.
        asm volatile("" ::: "memory");
        auto at = [&](int i, int& row, int& col, int& n, bool& vec) __attribute__((always_inline)) {
            where(b0 + i / G, i % G, row, col, n, vec);
        };
        // 2: alpha * acc + beta * C + bias of the whole groups, EB at a time
        if (combine) {
            // not unrolled: with the batches unrolled the register allocator
            // moves accumulators inside the main loop of the ring kernel
#pragma unroll 1
            for (int i0 = 0; i0 < NG; i0 += EB) {
                typename RawC<OUT>::type cw[EB];
                int ns[EB], rows[EB], cols[EB];
                static_for<0, EB>([&](auto d_t) {
                    constexpr int d = decltype(d_t)::value;
                    bool vec;
                    at(i0 + d, rows[d], cols[d], ns[d], vec);
                    if (rd_c && ns[d] == 4) cw[d] = load_raw_c<OUT>(p.C + ((int64_t)rows[d] * p.ldc + cols[d]) * OB);
                });
                static_for<0, EB>([&](auto d_t) {
                    constexpr int d = decltype(d_t)::value;
                    if (ns[d] == 4) {
                        lds_f32x4* slot = region + (i0 + d) * 64 + lane;
                        // both bias arrays are read (the one of the other
                        // kind holds zeros); only the bias of the call's kind
                        // is added
                        const f32x4 bc = *(const lds_f32x4*)(bias_col + (cols[d] - col0));
                        const float br = bias_row[rows[d] - row0];
                        f32x4 t = *slot * alpha;
                        if (rd_c) t += beta * raw_c_values<OUT>(cw[d], p.fp8_e5m2);
                        if (has_bias) t += p.bias_kind == BIAS_COL ? bc : f32x4{br, br, br, br};
                        *slot = t;
                    }
                });
            }
        }
        asm volatile("" ::: "memory");
        // 3: activation, output rounding and stores of the whole groups, in
        // a loop compiled for the call's activation (one uniform switch),
        // then the partial groups (N % 4 != 0: element by element, rare)
        const bool scale = !combine && alpha != 1.f;
        const bool late_bias = !combine && has_bias;
        auto whole = [&](auto act_t) __attribute__((always_inline)) {
            constexpr int ACT = decltype(act_t)::value;
            for (int i = 0; i < NG; ++i) {
                int row, col, n;
                bool vec;
                at(i, row, col, n, vec);
                if (WHOLE ? n <= 0 : n != 4) continue;
                f32x4 t = region[i * 64 + lane];
                if (scale) t *= alpha;
                if (late_bias) {
                    const f32x4 bc = *(const lds_f32x4*)(bias_col + (col - col0));
                    const float br = bias_row[row - row0];
                    t += p.bias_kind == BIAS_COL ? bc : f32x4{br, br, br, br};
                }
                store4<OUT>(p.C + ((int64_t)row * p.ldc + col) * OB, activate_t<ACT>(t[0]), activate_t<ACT>(t[1]),
                            activate_t<ACT>(t[2]), activate_t<ACT>(t[3]), vec, p.fp8_e5m2);
            }
        };
        switch (p.act) {
            case ACT_RELU: whole(IntTag<ACT_RELU>{}); break;
            case ACT_GELU: whole(IntTag<ACT_GELU>{}); break;
            case ACT_GELU_TANH: whole(IntTag<ACT_GELU_TANH>{}); break;
            case ACT_SILU: whole(IntTag<ACT_SILU>{}); break;
            default: whole(IntTag<ACT_NONE>{}); break;
        }
        if constexpr (!WHOLE) {
            for (int i = 0; i < NG; ++i) {
                int row, col, n;
                bool vec;
                at(i, row, col, n, vec);
                if (n <= 0 || n == 4) continue;
                fused_post<OUT>(p, row, col, n, vec, fused_pre<OUT>(p, row, col, n, region[i * 64 + lane]));
            }
        }
    });
}

// ---------------------------------------------------------------- kernel
// IN: input type, OUT: output type.
// FAST: every tile is whole (M % BM == 0, N % BN == 0) and A, B, C are
// 16-byte aligned with lda, ldb whole 16-byte chunks and ldc a multiple of 4:
// the main loop has no bounds checks (only a ragged last K step is masked).
// Otherwise (GENERAL) every load and store is checked; whole 16-byte chunks
// and 4-element stores still take one access each (unaligned where p.vec_ab /
// p.vec_c say so).
template <class T, int IN, int OUT, bool FAST, bool EPI = false>
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
    const int swz = p.swz_mask;
    const bool vec_ab = FAST || p.vec_ab;

    // a2: per-thread load assignment
    // A chunk i: row tid/CPR + i*(THREADS/CPR), chunk tid%CPR
    const int a_row0 = tid / CPR, a_c = tid % CPR;
    // B block i: idx = tid + i*THREADS; k-block idx%KBN, n-block idx/KBN
    const char* Ab = p.A;
    const char* Bb = p.B;
    const int64_t lda = p.lda, ldb = p.ldb;

    u32x4 ra[T::A_CHUNKS];
    u32x4 rb[T::B_BLOCKS][VE];

    // a2: global -> registers, one 16-byte chunk per call: w < A_CHUNKS is
    // chunk w of this thread's A rows, otherwise row (w - A_CHUNKS) % VE of B
    // block (w - A_CHUNKS) / VE, for the K step starting at k0.
    // Without CHECK (FAST kernels, full K steps) it is one buffer_load_dwordx4
    // whose resource starts at the tile's corner at k0 (a few scalar adds per
    // step), with one per-lane offset per operand and the chunk's row step as
    // the scalar offset; the host guarantees that these offsets fit in 31
    // bits.  With CHECK the chunk is tested against M / N / K and zero-filled
    // outside, through plain global loads.
    const int a_voff = (int)(((int64_t)a_row0 * lda + a_c * VE) * EB);
    int b_voff[T::B_BLOCKS];
#pragma unroll
    for (int i = 0; i < T::B_BLOCKS; ++i) {
        const int idx = tid + i * T::THREADS;
        const int kb = idx % T::KBN, nb = idx / T::KBN;
        b_voff[i] = (int)(((int64_t)kb * VE * ldb + nb * VE) * EB);
    }
    auto rsrc_a = [&](int k0) {
        return __builtin_amdgcn_make_buffer_rsrc((void*)(Ab + ((int64_t)m0 * lda + k0) * EB), (short)0, -1,
                                                 0x00020000);
    };
    auto rsrc_b = [&](int k0) {
        return __builtin_amdgcn_make_buffer_rsrc((void*)(Bb + ((int64_t)k0 * ldb + n0) * EB), (short)0, -1,
                                                 0x00020000);
    };
    auto load_one = [&](auto check_tag, int k0, int w) {
        constexpr bool CHECK = decltype(check_tag)::value || !FAST;
        if (w < T::A_CHUNKS) {
            if constexpr (!CHECK) {
                const int soff = (int)((int64_t)w * (T::THREADS / CPR) * lda * EB);
                ra[w] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc_a(k0), a_voff, soff, 0));
            } else {
                const int r = a_row0 + w * (T::THREADS / CPR);
                const int gm = m0 + r, gk = k0 + a_c * VE;
                const char* src = Ab + ((int64_t)gm * lda + gk) * EB;
                const int valid = gm < M ? (K - gk < VE ? K - gk : VE) : 0;
                if (valid == VE) ra[w] = vec_ab ? *(const u32x4*)src : load16(src);
                else ra[w] = valid > 0 ? load_chunk_partial<EB>(src, valid) : zero4();
            }
        } else {
            const int i = (w - T::A_CHUNKS) / VE, j = (w - T::A_CHUNKS) % VE;
            const int idx = tid + i * T::THREADS;
            const bool live = (T::B_TOTAL % T::THREADS == 0) || idx < T::B_TOTAL;
            if constexpr (!CHECK) {
                const int soff = (int)((int64_t)j * ldb * EB);
                const u32x4 v =
                    __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc_b(k0), b_voff[i], soff, 0));
                rb[i][j] = live ? v : zero4();
            } else {
                const int kb = idx % T::KBN, nb = idx / T::KBN;
                const int gn = n0 + nb * VE;
                const int gk = k0 + kb * VE + j;
                const char* src = Bb + ((int64_t)gk * ldb + gn) * EB;
                const int valid = (live && gk < K) ? (N - gn < VE ? N - gn : VE) : 0;
                if (valid == VE) rb[i][j] = vec_ab ? *(const u32x4*)src : load16(src);
                else rb[i][j] = valid > 0 ? load_chunk_partial<EB>(src, valid) : zero4();
            }
        }
    };
    constexpr int NLOAD = T::A_CHUNKS + T::B_BLOCKS * VE;

    // a2/a3: registers -> swizzled LDS stage.  A chunk w as loaded; B column
    // w % VE of block w / VE, transposed to a k-contiguous row on the way.
    auto store_a_one = [&](int stage, int w) {
        char* As = smem + stage * T::STAGE_BYTES;
        const int r = a_row0 + w * (T::THREADS / CPR);
        const int pc = a_c ^ (swizzle_key<CPR>(r) & swz);
        *(u32x4*)(As + r * RB + pc * 16) = ra[w];
    };
    auto store_b_one = [&](int stage, int w) {
        char* Bs = smem + stage * T::STAGE_BYTES + T::A_BYTES;
        const int i = w / VE, e = w % VE;
        const int idx = tid + i * T::THREADS;
        if ((T::B_TOTAL % T::THREADS == 0) || idx < T::B_TOTAL) {
            const int kb = idx % T::KBN, nb = idx / T::KBN;
            const int n = nb * VE + e;
            const int pc = kb ^ (swizzle_key<CPR>(n) & swz);
            *(u32x4*)(Bs + n * RB + pc * 16) = transpose_col<EB>(rb[i], e);
        }
    };
    constexpr int NSA = T::A_CHUNKS, NSB = T::B_BLOCKS * VE;

    // a6: accumulators
    f32x16 acc[T::FM][T::FN];
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int j = 0; j < T::FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // a5: fragments.  Lane l reads row (l & 31) of each 32-row block at
    // chunk 2g + l/32 of k-group g; the swizzle key of a fragment row depends
    // only on the lane (block starts are multiples of 32).
    const int frow = lane & 31, fhalf = lane >> 5;
    const int a_frow0 = wm * T::WTM + frow;
    const int b_frow0 = wn * T::WTN + frow;
    const int fkey_a = swizzle_key<CPR>(a_frow0) & swz;
    const int fkey_b = swizzle_key<CPR>(b_frow0) & swz;
    u32x4 fa[2][T::FM], fb[2][T::FN];
    constexpr int NREAD = T::FM + T::FN;

    auto read_frag = [&](int stage, int g, int buf, int r) {
        const char* As = smem + stage * T::STAGE_BYTES;
        const char* Bs = As + T::A_BYTES;
        if (r < T::FM) {
            const int ca = ((2 * g + fhalf) ^ fkey_a) * 16;
            fa[buf][r] = *(const u32x4*)(As + (a_frow0 + 32 * r) * RB + ca);
        } else {
            const int cb = ((2 * g + fhalf) ^ fkey_b) * 16;
            fb[buf][r - T::FM] = *(const u32x4*)(Bs + (b_frow0 + 32 * (r - T::FM)) * RB + cb);
        }
    };

    constexpr int NMF = T::FM * T::FN;
    auto mfma_one = [&](int buf, int m) {
        const int i = m / T::FN, j = m % T::FN;
        if constexpr (IN == DT_F16) {
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                __builtin_bit_cast(f16x8, fb[buf][j]), __builtin_bit_cast(f16x8, fa[buf][i]), acc[i][j], 0, 0, 0);
        } else if constexpr (IN == DT_BF16) {
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, fb[buf][j]), __builtin_bit_cast(bf16x8, fa[buf][i]), acc[i][j], 0, 0,
                0);
        } else {
            // Bit-cast whole vectors, then index: a bit-cast of a single
            // ext-vector element is lowered as a cast of element 0 by this
            // compiler.
            const f32x4 bv = __builtin_bit_cast(f32x4, fb[buf][j]);
            const f32x4 av = __builtin_bit_cast(f32x4, fa[buf][i]);
#pragma unroll
            for (int s = 0; s < 4; ++s)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(bv[s], av[s], acc[i][j], 0, 0, 0);
        }
    };

    // a4: one pipelined K step.  On entry LDS stage `cur` holds this step,
    // the fragments of k-group 0 are in buffer 0 and, with STORE, ra/rb hold
    // the next step.  k-group g issues its NMF MFMAs one by one; between them
    // go, spread evenly, the reads of the fragments of group g+1 and: in
    // group 0 the LDS writes of A of the next step followed (with LOAD) by
    // the global loads of A of the step after, in group 1 the same for B.
    // Each load thus has almost a whole K step to arrive before its register
    // is written to LDS again.  The barrier comes before the last group, whose
    // MFMAs overlap the reads of the next step's first fragments.
    // sched_barrier fences keep this order.
    auto kstep = [&](auto check_tag, auto store_tag, auto load_tag, int cur, int k_load) {
        constexpr bool STORE = decltype(store_tag)::value;
        constexpr bool LOAD = decltype(load_tag)::value;
        constexpr int NKG = T::NKG;
        constexpr int G_B = NKG - 2 < 1 ? NKG - 2 : 1;
        constexpr int NLA = T::A_CHUNKS, NLB = T::B_BLOCKS * VE;
        const int nxt = cur ^ 1;
        static_for<0, NKG>([&](auto gt) {
            constexpr int g = decltype(gt)::value;
            constexpr bool last = g == NKG - 1;
            if constexpr (last) __syncthreads();
            // work items of this group, in issue order
            constexpr int n_read = last ? (STORE ? NREAD : 0) : NREAD;
            constexpr bool do_a = STORE && g == 0 && !last;
            constexpr bool do_b = STORE && g == G_B && !last;
            constexpr int n_sa = do_a ? NSA : 0;
            constexpr int n_la = (do_a && LOAD) ? NLA : 0;
            constexpr int n_sb = do_b ? NSB : 0;
            constexpr int n_lb = (do_b && LOAD) ? NLB : 0;
            constexpr int n_work = n_read + n_sa + n_la + n_sb + n_lb;
            static_for<0, NMF>([&](auto mt) {
                constexpr int m = decltype(mt)::value;
                mfma_one(g & 1, m);
                // items [ceil(m n / NMF), ceil((m+1) n / NMF)) follow MFMA m
                constexpr int wb = (m * n_work + NMF - 1) / NMF;
                constexpr int we = ((m + 1) * n_work + NMF - 1) / NMF;
                static_for<wb, we>([&](auto wt) {
                    constexpr int w = decltype(wt)::value;
                    if constexpr (w < n_read) {
                        if constexpr (last) read_frag(nxt, 0, 0, w);
                        else read_frag(cur, g + 1, (g + 1) & 1, w);
                    } else if constexpr (w < n_read + n_sa) {
                        store_a_one(nxt, w - n_read);
                    } else if constexpr (w < n_read + n_sa + n_la) {
                        load_one(check_tag, k_load, w - n_read - n_sa);
                    } else if constexpr (w < n_read + n_sa + n_la + n_sb) {
                        store_b_one(nxt, w - n_read - n_sa - n_la);
                    } else {
                        load_one(check_tag, k_load, NLA + (w - n_read - n_sa - n_la - n_sb));
                    }
                });
                __builtin_amdgcn_sched_barrier(0);
            });
        });
    };

    auto run = [&](auto check_tag) {
        constexpr BoolTag<true> yes{};
        constexpr BoolTag<false> no{};
        const int nkf = K / T::BK;  // full K steps
        auto fill = [&](auto ctag, int k0, int stage) {
            static_for<0, NLOAD>([&](auto w) { load_one(ctag, k0, decltype(w)::value); });
            static_for<0, NSA>([&](auto w) { store_a_one(stage, decltype(w)::value); });
            static_for<0, NSB>([&](auto w) { store_b_one(stage, decltype(w)::value); });
        };
        auto read_all = [&](int stage) {
            static_for<0, NREAD>([&](auto r) { read_frag(stage, 0, 0, decltype(r)::value); });
        };
        if (nkf > 0) {
            fill(check_tag, 0, 0);
            if (nkf > 1) static_for<0, NLOAD>([&](auto w) { load_one(check_tag, T::BK, decltype(w)::value); });
            __syncthreads();
            read_all(0);
            int kt = 0;
            for (; kt + 2 < nkf; ++kt) kstep(check_tag, yes, yes, kt & 1, (kt + 2) * T::BK);
            if (kt + 1 < nkf) {
                kstep(check_tag, yes, no, kt & 1, 0);
                ++kt;
            }
            kstep(check_tag, no, no, kt & 1, 0);
        }
        if (K % T::BK) {
            // the ragged last K step, zero-filled beyond K, not overlapped
            const int st = nkf & 1;
            fill(yes, nkf * T::BK, st);
            __syncthreads();
            read_all(st);
            kstep(yes, no, no, st, 0);
        }
    };
    run(BoolTag<!FAST>{});

    // a7: epilogue.  acc[i][j][4q + e] = C[row][col + e] with
    // row = m0 + wm*WTM + 32 i + lane%32, col = n0 + wn*WTN + 32 j + 8 q + 4 (lane/32).
    constexpr int OB = out_bytes<OUT>();
    const int64_t ldc = p.ldc;
    if constexpr (EPI) {
        // fused epilogue through LDS, once no wave reads it any more; the
        // tile's bias in an LDS array of its own
        __shared__ __attribute__((aligned(16))) float ebias_[T::BM + T::BN];
        lds_float* const ebias = (lds_float*)(lds_void*)ebias_;
        stage_bias<T::THREADS, T::BM, T::BN>(p, ebias, ebias + T::BN, m0, n0);
        __syncthreads();
        constexpr int REGION = T::LDS_BYTES / T::WAVES;                   // bytes per wave
        constexpr int PB0 = REGION / (64 * 64) < T::FM * T::FN ? REGION / (64 * 64) : T::FM * T::FN;
        constexpr int PB = (T::FM * T::FN) % PB0 == 0 ? PB0 : 1;
        static_assert(PB >= 1, "the LDS holds a block of accumulators per wave");
        lds_f32x4* region = (lds_f32x4*)(lds_void*)smem + wave * (REGION / 16);
        fused_epilogue<OUT, T::FM * T::FN, 16, PB, FAST>(
            p, region, ebias, ebias + T::BN, m0, n0,
            [&](auto b_t) { constexpr int b = decltype(b_t)::value; return acc[b / T::FN][b % T::FN]; },
            [&](int b, int q, int& row, int& col, int& n, bool& vec) {
                const int i = b / T::FN, j = b % T::FN;
                row = m0 + a_frow0 + 32 * i;
                col = n0 + wn * T::WTN + 32 * j + 8 * q + 4 * fhalf;
                if constexpr (FAST) {
                    n = 4;
                    vec = true;
                } else {
                    n = row < M ? (N - col >= 4 ? 4 : N - col > 0 ? N - col : 0) : 0;
                    vec = p.vec_c != 0;
                }
            });
        return;
    }
    // One 32x32 block at a time (fenced), so that only one block's values are
    // moved out of the accumulator registers at once.
    static_for<0, T::FM * T::FN>([&](auto bt) {
        constexpr int i = decltype(bt)::value / T::FN, j = decltype(bt)::value % T::FN;
        const int row = m0 + a_frow0 + 32 * i;
        static_for<0, 4>([&](auto qt) {
            constexpr int q = decltype(qt)::value;
            const int col = n0 + wn * T::WTN + 32 * j + 8 * q + 4 * fhalf;
            char* dst = p.C + ((int64_t)row * ldc + col) * OB;
            const float v0 = acc[i][j][4 * q + 0], v1 = acc[i][j][4 * q + 1];
            const float v2 = acc[i][j][4 * q + 2], v3 = acc[i][j][4 * q + 3];
            if constexpr (FAST) {
                store4<OUT>(dst, v0, v1, v2, v3, true);
            } else if (row < M) {
                if (col + 4 <= N) {
                    store4<OUT>(dst, v0, v1, v2, v3, p.vec_c);
                } else {
                    if (col + 0 < N) store_elem<OUT>(dst + 0 * OB, v0);
                    if (col + 1 < N) store_elem<OUT>(dst + 1 * OB, v1);
                    if (col + 2 < N) store_elem<OUT>(dst + 2 * OB, v2);
                    if (col + 3 < N) store_elem<OUT>(dst + 3 * OB, v3);
                }
            }
        });
        __builtin_amdgcn_sched_barrier(0);
    });
}

}  // namespace tgemm
