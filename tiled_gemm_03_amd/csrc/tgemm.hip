// tgemm.hip -- C ABI of libtgemm.so: argument checks, the per-shape tile
// configuration table and the kernel launch.  The kernels are in
// gemm_kernel.hpp (register-staged; every shape, type and alignment) and
// gemm_kernel_ring.hpp (direct-to-LDS rings; whole tiles of 16-bit inputs)
// and gemm_kernel_direct.hpp (operands straight to registers; small, ragged
// or unaligned products); the ABI is declared (and documented) in
// include/tgemm.h.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include "gemm_kernel.hpp"
#include "gemm_kernel_direct.hpp"
#include "gemm_kernel_ring.hpp"
#include "tgemm.h"

using namespace tgemm;

namespace {

// ------------------------------------------------------------- configurations
// Tile-config tuples (block_M, block_N, block_K, waves, occupancy) in the
// spirit of the tuning tables of page "企业官网建设流程全解析", §3.3 / §4.4, and
// of the DeepSeek/Ascend TileLang toolkit page, §4.3, sized for gfx950:
// 160 KiB LDS per CU, 512 registers per lane at one wave per SIMD.
using CfgBig = TileCfg<256, 256, 64, 2, 2, 2, 1>;    // 4 waves, 128x128 per wave
using CfgMid = TileCfg<128, 128, 64, 2, 2, 2, 2>;    // 4 waves, 64x64 per wave
using CfgSmall = TileCfg<64, 64, 64, 2, 2, 2, 2>;    // 4 waves, 32x32 per wave
using CfgTiny = TileCfg<32, 32, 64, 1, 1, 2, 4>;     // 1 wave
using CfgF32Mid = TileCfg<64, 64, 32, 2, 2, 4, 2>;   // fp32 inputs
using CfgF32Tiny = TileCfg<32, 32, 32, 1, 1, 4, 4>;  // fp32 inputs, 1 wave

typedef void (*KernelFn)(GemmArgs);

struct ConfigEntry {
    const char* name;
    int in_family;  // TGEMM_F16 (serves F16 and BF16) or TGEMM_F32
    bool direct;    // the direct kernel (32 x 32 per workgroup, no LDS)
    int bm, bn, bk, wm, wn, eb, lds_bytes, threads, cpr;
    KernelFn (*pick)(int in, int out, bool fast);
    // direct-to-LDS ring kernel of the same output tile (whole tiles, K a
    // multiple of ring_k_mult); its block_k and stage count
    KernelFn (*pick_ring)(int in, int out);
    int ring_bk, ring_stages, ring_k_mult, ring_lds;
};

template <class R>
KernelFn pick_ring(int in, int out) {
    if (in == TGEMM_F16 && out == TGEMM_F16) return gemm_kernel_ring<R, DT_F16, DT_F16>;
    if (in == TGEMM_F16 && out == TGEMM_F32) return gemm_kernel_ring<R, DT_F16, DT_F32>;
    if (in == TGEMM_BF16 && out == TGEMM_BF16) return gemm_kernel_ring<R, DT_BF16, DT_BF16>;
    if (in == TGEMM_BF16 && out == TGEMM_F32) return gemm_kernel_ring<R, DT_BF16, DT_F32>;
    return nullptr;
}
using RingBig = RingCfg<256, 256, 2, 2, 4, 1>;
using RingMid = RingCfg<128, 128, 2, 2, 4, 2>;
static_assert(RingBig::LDS_BYTES == CfgBig::LDS_BYTES && RingMid::LDS_BYTES == CfgMid::LDS_BYTES,
              "both kernels of a configuration use the same LDS budget");

template <class T, int IN>
KernelFn pick_out(int out, bool fast) {
    if (out == TGEMM_F32)
        return fast ? gemm_kernel<T, IN, DT_F32, true> : gemm_kernel<T, IN, DT_F32, false>;
    if (IN == DT_F16 && out == TGEMM_F16)
        return fast ? gemm_kernel<T, IN, DT_F16, true> : gemm_kernel<T, IN, DT_F16, false>;
    if (IN == DT_BF16 && out == TGEMM_BF16)
        return fast ? gemm_kernel<T, IN, DT_BF16, true> : gemm_kernel<T, IN, DT_BF16, false>;
    return nullptr;
}

template <class T>
KernelFn pick_half(int in, int out, bool fast) {
    if (in == TGEMM_F16) return pick_out<T, DT_F16>(out, fast);
    if (in == TGEMM_BF16) return pick_out<T, DT_BF16>(out, fast);
    return nullptr;
}

template <class T>
KernelFn pick_f32(int in, int out, bool fast) {
    if (in == TGEMM_F32 && out == TGEMM_F32)
        return fast ? gemm_kernel<T, DT_F32, DT_F32, true> : gemm_kernel<T, DT_F32, DT_F32, false>;
    return nullptr;
}

#define ENTRY(name, fam, T, pk)                                                                         \
    {name, fam, false, T::BM, T::BN, T::BK, T::WM, T::WN, T::EB, T::LDS_BYTES, T::THREADS, T::CPR, pk<T>, nullptr, \
     0, 0, 0, 0}
#define ENTRY_RING(name, fam, T, pk, R)                                                                          \
    {name, fam, false, T::BM, T::BN, T::BK, T::WM, T::WN, T::EB, T::LDS_BYTES, T::THREADS, T::CPR, pk<T>,        \
     pick_ring<R>, R::BK, R::S, R::K_MULT, R::LDS_BYTES}
// direct kernel: 32 x 32 per workgroup of 2 x 2 waves, steps of 32 of K
#define ENTRY_DIRECT(name, fam, eb, pk) \
    {name, fam, true, 32, 32, 32, 2, 2, eb, 0, 256, 1, pk, nullptr, 0, 0, 0, 0}

// direct kernel for (in, out); `avec`: A rows are whole 16-byte chunks
KernelFn pick_direct(int in, int out, bool avec) {
    if (in == TGEMM_F32) return out == TGEMM_F32 ? gemm_kernel_direct<DT_F32, DT_F32, false> : nullptr;
    if (in == TGEMM_F16 && out == TGEMM_F16)
        return avec ? gemm_kernel_direct<DT_F16, DT_F16, true> : gemm_kernel_direct<DT_F16, DT_F16, false>;
    if (in == TGEMM_F16 && out == TGEMM_F32)
        return avec ? gemm_kernel_direct<DT_F16, DT_F32, true> : gemm_kernel_direct<DT_F16, DT_F32, false>;
    if (in == TGEMM_BF16 && out == TGEMM_BF16)
        return avec ? gemm_kernel_direct<DT_BF16, DT_BF16, true> : gemm_kernel_direct<DT_BF16, DT_BF16, false>;
    if (in == TGEMM_BF16 && out == TGEMM_F32)
        return avec ? gemm_kernel_direct<DT_BF16, DT_F32, true> : gemm_kernel_direct<DT_BF16, DT_F32, false>;
    return nullptr;
}

const ConfigEntry kConfigs[] = {
    ENTRY_RING("h256x256_w2x2", TGEMM_F16, CfgBig, pick_half, RingBig),
    ENTRY_RING("h128x128_w2x2", TGEMM_F16, CfgMid, pick_half, RingMid),
    ENTRY("h64x64x64_w2x2", TGEMM_F16, CfgSmall, pick_half),
    ENTRY("h32x32x64_w1x1", TGEMM_F16, CfgTiny, pick_half),
    ENTRY("s64x64x32_w2x2", TGEMM_F32, CfgF32Mid, pick_f32),
    ENTRY("s32x32x32_w1x1", TGEMM_F32, CfgF32Tiny, pick_f32),
    ENTRY_DIRECT("h32x32_direct", TGEMM_F16, 2, pick_direct),
    ENTRY_DIRECT("s32x32_direct", TGEMM_F32, 4, pick_direct),
};
constexpr int kNumConfigs = sizeof(kConfigs) / sizeof(kConfigs[0]);
enum { CFG_BIG = 0, CFG_MID = 1, CFG_SMALL = 2, CFG_TINY = 3, CFG_F32_MID = 4, CFG_F32_TINY = 5,
       CFG_DIRECT = 6, CFG_F32_DIRECT = 7 };

// Measurement-only switches, read once from the environment:
//   TGEMM_GROUP_M=<n>    tile rows per raster group (default 4)
//   TGEMM_NO_SWIZZLE=1   plain row-major LDS tiles (for bank-conflict A/B runs)
//   TGEMM_NO_DL=1        register-staged kernel instead of the direct-to-LDS ring
struct Tuning {
    int group_m = 4;
    bool swizzle = true;
    bool direct_lds = true;
    Tuning() {
        if (const char* s = getenv("TGEMM_GROUP_M")) {
            const int g = atoi(s);
            if (g > 0) group_m = g;
        }
        if (const char* s = getenv("TGEMM_NO_SWIZZLE")) swizzle = !(s[0] == '1');
        if (const char* s = getenv("TGEMM_NO_DL")) direct_lds = !(s[0] == '1');
    }
};
const Tuning& tuning() {
    static const Tuning t;
    return t;
}

int elem_bytes(int dt) { return dt == TGEMM_F32 ? 4 : 2; }

bool pair_supported(int in, int out) {
    switch (in) {
        case TGEMM_F32: return out == TGEMM_F32;
        case TGEMM_F16: return out == TGEMM_F16 || out == TGEMM_F32;
        case TGEMM_BF16: return out == TGEMM_BF16 || out == TGEMM_F32;
        default: return false;
    }
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int validate(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb,
             const void* C, int64_t ldc, int in, int out) {
    if (M < 0 || N < 0 || K < 0 || M > TGEMM_MAX_DIM || N > TGEMM_MAX_DIM || K > TGEMM_MAX_DIM)
        return TGEMM_ERR_DIM;
    if (!pair_supported(in, out)) return TGEMM_ERR_DTYPE;
    if (lda < K || ldb < N || ldc < N) return TGEMM_ERR_LD;
    if (M == 0 || N == 0) return TGEMM_OK;
    if (C == nullptr) return TGEMM_ERR_NULL;
    if (K > 0 && (A == nullptr || B == nullptr)) return TGEMM_ERR_NULL;
    if (K > 0) {
        const uintptr_t ie = elem_bytes(in), oe = elem_bytes(out);
        const uintptr_t c0 = (uintptr_t)C, c1 = c0 + (uintptr_t)((M - 1) * ldc + N) * oe;
        const uintptr_t a0 = (uintptr_t)A, a1 = a0 + (uintptr_t)((M - 1) * lda + K) * ie;
        const uintptr_t b0 = (uintptr_t)B, b1 = b0 + (uintptr_t)((K - 1) * ldb + N) * ie;
        if ((c0 < a1 && a0 < c1) || (c0 < b1 && b0 < c1)) return TGEMM_ERR_ALIAS;
    }
    return TGEMM_OK;
}

// 16-byte loads of A and B need 16-byte aligned bases and leading dimensions
// that are whole 16-byte chunks.
bool loads_aligned(const ConfigEntry& c, const void* A, int64_t lda, const void* B, int64_t ldb) {
    const int ve = 16 / c.eb;
    return ((uintptr_t)A % 16 == 0) && ((uintptr_t)B % 16 == 0) && (lda % ve == 0) && (ldb % ve == 0);
}

// 4-element stores of C need a base aligned to 4 elements and ldc % 4 == 0.
bool stores_aligned(const void* C, int64_t ldc, int out) {
    return ((uintptr_t)C % (4 * (uintptr_t)elem_bytes(out)) == 0) && (ldc % 4 == 0);
}

int64_t tiles_for(const ConfigEntry& c, int64_t M, int64_t N) { return ceil_div(M, c.bm) * ceil_div(N, c.bn); }

// Whether a register-staged configuration runs its unchecked path: whole
// tiles, 16-byte aligned operands, 4-element aligned C rows, offsets within
// 31 bits.
bool tiled_fast(const ConfigEntry& c, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
                int64_t ldb, const void* C, int64_t ldc, int out) {
    const bool offsets_fit = (int64_t)c.bm * lda * c.eb + K * c.eb < (1LL << 31) &&
                             (int64_t)c.bk * ldb * c.eb + N * c.eb < (1LL << 31);
    return loads_aligned(c, A, lda, B, ldb) && stores_aligned(C, ldc, out) && offsets_fit && M % c.bm == 0 &&
           N % c.bn == 0;
}

// Whether a configuration with a ring kernel runs it.
bool ring_applies(const ConfigEntry& c, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
                  int64_t ldb, const void* C, int64_t ldc, int out) {
    return c.pick_ring != nullptr && tiled_fast(c, M, N, K, A, lda, B, ldb, C, ldc, out) &&
           ((int64_t)c.bm * lda + K + (int64_t)c.ring_stages * c.ring_bk) * c.eb < (1LL << 31) &&
           ((K + (int64_t)c.ring_stages * c.ring_bk) * ldb + c.bn) * c.eb < (1LL << 31) &&
           K % c.ring_k_mult == 0 && tuning().direct_lds;
}

// The per-shape table (measured on MI355X; kernel times from rocprofv3
// traces of the five workloads under every configuration):
//  * enough 256 x 256 tiles for all 256 CUs: the 256 x 256 configuration
//    (the direct-to-LDS ring kernel when it applies);
//  * the 128 x 128 ring kernel from 128 tiles up when it applies (it beats
//    64 x 64 register-staged tiles at 1024 x 2048 x 512: 8.6 vs 11.1 us),
//    otherwise the largest register-staged tile that still gives 256 tiles;
//  * small products (M N <= 2^18) whose register-staged tile would run its
//    checked path (ragged or unaligned operands) take the direct kernel
//    (127 x 255 x 512 with ldb = 255: about 8 us instead of 60-90 us);
//  * other small products the smallest register-staged tile, which
//    maximises parallelism where launch latency and one workgroup's K loop
//    set the time.
int table_choice(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb,
                 const void* C, int64_t ldc, int in, int out) {
    const bool small = M * N <= (1LL << 18);
    if (in == TGEMM_F32) {
        if (tiles_for(kConfigs[CFG_F32_MID], M, N) >= 256) return CFG_F32_MID;
        if (small && !tiled_fast(kConfigs[CFG_F32_TINY], M, N, K, A, lda, B, ldb, C, ldc, out)) return CFG_F32_DIRECT;
        return CFG_F32_TINY;
    }
    if (tiles_for(kConfigs[CFG_BIG], M, N) >= 256) return CFG_BIG;
    if (tiles_for(kConfigs[CFG_MID], M, N) >= 128 && ring_applies(kConfigs[CFG_MID], M, N, K, A, lda, B, ldb, C, ldc, out))
        return CFG_MID;
    if (tiles_for(kConfigs[CFG_MID], M, N) >= 256) return CFG_MID;
    if (tiles_for(kConfigs[CFG_SMALL], M, N) >= 256) return CFG_SMALL;
    if (small && !tiled_fast(kConfigs[CFG_TINY], M, N, K, A, lda, B, ldb, C, ldc, out)) return CFG_DIRECT;
    return CFG_TINY;
}

int family_of(int in) { return in == TGEMM_F32 ? TGEMM_F32 : TGEMM_F16; }

// What one call runs: the configuration, the kernel and its kind.
struct Plan {
    int config;
    int kind;  // TGEMM_KERNEL_*
    KernelFn fn;
};

int plan_tiled(const ConfigEntry& c, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
               int64_t ldb, const void* C, int64_t ldc, int in, int out, Plan& plan);

// Validates the arguments and picks the kernel; returns TGEMM_OK (plan
// filled; M == 0 or N == 0 leaves plan.fn null) or a negative error code.
int make_plan(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb,
              const void* C, int64_t ldc, int in, int out, int config_id, Plan& plan) {
    const int v = validate(M, N, K, A, lda, B, ldb, C, ldc, in, out);
    if (v != TGEMM_OK) return v;
    if (config_id < -1 || config_id >= kNumConfigs) return TGEMM_ERR_CONFIG;
    if (config_id >= 0 && kConfigs[config_id].in_family != family_of(in)) return TGEMM_ERR_CONFIG;
    plan.config = config_id >= 0 ? config_id : table_choice(M, N, K, A, lda, B, ldb, C, ldc, in, out);
    plan.fn = nullptr;
    plan.kind = TGEMM_KERNEL_GENERAL;
    if (M == 0 || N == 0) return TGEMM_OK;
    const ConfigEntry& c = kConfigs[plan.config];
    if (c.direct) {
        // buffer offsets: 32 rows of A plus K + 320 columns; K + 320 rows of B
        if (((int64_t)32 * lda + K + 320) * c.eb >= (1LL << 31) || ((K + 320) * ldb + 32) * c.eb >= (1LL << 31))
            plan.config = in == TGEMM_F32 ? CFG_F32_TINY : CFG_TINY;  // offsets too wide: the checked kernel
        else {
            const bool avec = in != TGEMM_F32 && (uintptr_t)A % 16 == 0 && lda % 8 == 0 && K % 8 == 0;
            plan.kind = TGEMM_KERNEL_DIRECT;
            plan.fn = c.pick(in, out, avec);
            if (plan.fn == nullptr) return TGEMM_ERR_DTYPE;
            if (ceil_div(M, c.bm) * ceil_div(N, c.bn) > 0x7fffffff) return TGEMM_ERR_DIM;
            return TGEMM_OK;
        }
    }
    const ConfigEntry& t = kConfigs[plan.config];
    return plan_tiled(t, M, N, K, A, lda, B, ldb, C, ldc, in, out, plan);
}

int plan_tiled(const ConfigEntry& c, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
               int64_t ldb, const void* C, int64_t ldc, int in, int out, Plan& plan) {
    const bool fast = tiled_fast(c, M, N, K, A, lda, B, ldb, C, ldc, out);
    const bool ring = ring_applies(c, M, N, K, A, lda, B, ldb, C, ldc, out);
    plan.kind = ring ? TGEMM_KERNEL_RING : fast ? TGEMM_KERNEL_TILED : TGEMM_KERNEL_GENERAL;
    plan.fn = ring ? c.pick_ring(in, out) : c.pick(in, out, fast);
    if (plan.fn == nullptr) return TGEMM_ERR_DTYPE;
    const int64_t grid = ceil_div(M, c.bm) * ceil_div(N, c.bn);
    if (grid > 0x7fffffff) return TGEMM_ERR_DIM;
    return TGEMM_OK;
}

int run(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb, void* C,
        int64_t ldc, int in, int out, void* stream, int config_id) {
    Plan plan;
    const int v = make_plan(M, N, K, A, lda, B, ldb, C, ldc, in, out, config_id, plan);
    if (v != TGEMM_OK || plan.fn == nullptr) return v;
    const ConfigEntry& c = kConfigs[plan.config];

    GemmArgs args;
    args.A = (const char*)A;
    args.B = (const char*)B;
    args.C = (char*)C;
    args.lda = lda;
    args.ldb = ldb;
    args.ldc = ldc;
    args.M = (int)M;
    args.N = (int)N;
    args.K = (int)K;
    args.tiles_m = (int)ceil_div(M, c.bm);
    args.tiles_n = (int)ceil_div(N, c.bn);
    args.group_m = tuning().group_m;
    args.swz_mask = tuning().swizzle ? c.cpr - 1 : 0;
    args.vec_ab = loads_aligned(c, A, lda, B, ldb);
    args.vec_c = stores_aligned(C, ldc, out);
    const int64_t grid = (int64_t)args.tiles_m * args.tiles_n;

    void* kargs[] = {&args};
    hipError_t e = hipLaunchKernel((const void*)plan.fn, dim3((unsigned)grid), dim3(c.threads), kargs, 0,
                                   (hipStream_t)stream);
    if (e == hipSuccess) e = hipGetLastError();
    return e == hipSuccess ? TGEMM_OK : (int)e;
}

}  // namespace

extern "C" {

int gemm(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb, void* C,
         int64_t ldc, int in_dtype, int out_dtype, void* stream) {
    return run(M, N, K, A, lda, B, ldb, C, ldc, in_dtype, out_dtype, stream, -1);
}

int gemm_ex(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb, void* C,
            int64_t ldc, int in_dtype, int out_dtype, void* stream, int config_id) {
    return run(M, N, K, A, lda, B, ldb, C, ldc, in_dtype, out_dtype, stream, config_id);
}

const char* gemm_strerror(int code) {
    switch (code) {
        case TGEMM_OK: return "success";
        case TGEMM_ERR_DIM: return "M, N or K negative or too large";
        case TGEMM_ERR_NULL: return "NULL pointer for a non-empty operand";
        case TGEMM_ERR_LD: return "leading dimension smaller than the row width (lda < K, ldb < N or ldc < N)";
        case TGEMM_ERR_DTYPE: return "unsupported (in_dtype, out_dtype) pair";
        case TGEMM_ERR_ALIAS: return "C overlaps A or B";
        case TGEMM_ERR_CONFIG: return "unknown tile configuration or configuration for another input type";
        default: break;
    }
    if (code > 0) return hipGetErrorString((hipError_t)code);
    return "unknown error code";
}

int gemm_num_configs(void) { return kNumConfigs; }

int gemm_config_info(int id, tgemm_config_info* out) {
    if (id < 0 || id >= kNumConfigs || out == nullptr) return TGEMM_ERR_CONFIG;
    const ConfigEntry& c = kConfigs[id];
    const bool ring = c.pick_ring != nullptr;
    out->id = id;
    out->in_dtype = c.in_family;
    out->block_m = c.bm;
    out->block_n = c.bn;
    out->threads = c.threads;
    out->waves_m = c.wm;
    out->waves_n = c.wn;
    out->name = c.name;
    if (c.direct) {
        // operands go straight to registers: no LDS stage
        out->block_k = 32;
        out->stages = 0;
        out->mfma_m = 16;
        out->mfma_n = 16;
        out->mfma_k = c.eb == 4 ? 4 : 32;
        out->lds_bytes = 0;
        return TGEMM_OK;
    }
    out->block_k = ring ? c.ring_bk : c.bk;
    out->stages = ring ? c.ring_stages : 2;
    out->mfma_m = ring ? 16 : 32;
    out->mfma_n = ring ? 16 : 32;
    out->mfma_k = ring ? 32 : (c.eb == 4 ? 2 : 16);
    out->lds_bytes = ring ? c.ring_lds : c.lds_bytes;
    return TGEMM_OK;
}

int gemm_select_config(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb,
                       const void* C, int64_t ldc, int in_dtype, int out_dtype) {
    const int v = validate(M, N, K, A, lda, B, ldb, C, ldc, in_dtype, out_dtype);
    if (v != TGEMM_OK) return v;
    return table_choice(M, N, K, A, lda, B, ldb, C, ldc, in_dtype, out_dtype);
}

int gemm_select_kernel(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb,
                       const void* C, int64_t ldc, int in_dtype, int out_dtype, int config_id) {
    Plan plan;
    const int v = make_plan(M, N, K, A, lda, B, ldb, C, ldc, in_dtype, out_dtype, config_id, plan);
    return v != TGEMM_OK ? v : plan.kind;
}

int gemm_tile_map(int bid, int tiles_m, int tiles_n, int group_m, int* tm, int* tn) {
    if (tiles_m <= 0 || tiles_n <= 0 || group_m <= 0 || bid < 0 || bid >= tiles_m * tiles_n || !tm || !tn)
        return TGEMM_ERR_DIM;
    tile_of(bid, tiles_m, tiles_n, group_m, *tm, *tn);
    return TGEMM_OK;
}

const char* gemm_version(void) { return "tgemm 0.1 gfx950"; }

}  // extern "C"
