// tgemm.hip -- C ABI of libtgemm.so: argument checks, the per-shape tile
// configuration table and the kernel launch.  The kernels are in
// gemm_kernel.hpp (register-staged; every shape, type and alignment, both
// operands row-major), gemm_kernel_ring.hpp (direct-to-LDS rings; 16-bit
// inputs, aligned, K a multiple of 128, N % 4 == 0, any operand layout) and gemm_kernel_direct.hpp (operands
// straight to registers; small, ragged or unaligned products, any operand
// layout), compiled in units of their own (k_*.hip) behind the selectors of
// kernels.hpp; the ABI is declared (and documented) in include/tgemm.h.
#include <hip/hip_runtime.h>
#include <mutex>
#include <stdint.h>
#include <stdlib.h>

#include "kernels.hpp"
#include "tgemm.h"

using namespace tgemm;

namespace {

// ------------------------------------------------------------- configurations
struct ConfigEntry {
    const char* name;
    int in_family;  // TGEMM_F16 (serves F16 and BF16) or TGEMM_F32
    bool direct;    // the direct kernel (32 x 32 per workgroup, or 16 x 16 with K over its waves)
    int bm, bn, bk, wm, wn, eb, lds_bytes, threads, cpr;
    // register-staged kernels (row-major operands only)
    KernelFn (*tiled)(int in, int out, bool fast, bool epi);
    // direct-to-LDS ring kernels of the same output tile (aligned operands,
    // any M and N, any operand layout; the rings walk K in multiples of
    // ring_k_mult, kt: the variant that adds the rest of K; epi: the fused
    // epilogue, also taken when the plain one cannot store C), with their
    // block_k, stage count and LDS bytes
    KernelFn (*ring)(int in, int out, int la, int lb, bool epi, bool kt);
    int ring_bk, ring_stages, ring_k_mult, ring_lds;
    int ring_lookahead;               // steps of ring_bk that the ring loads past K
    int ring_a_bk, ring_a_stages;     // the ring of a row-major A
    bool ring_a_col;                  // whether the ring kernels take a column-major A
};

KernelFn tiled_f32_big(int in, int out, bool fast, bool epi) { return tiled_kernel_f32(CFG_F32_BIG, in, out, fast, epi); }
KernelFn tiled_f32_mid(int in, int out, bool fast, bool epi) { return tiled_kernel_f32(CFG_F32_MID, in, out, fast, epi); }
KernelFn tiled_f32_tiny(int in, int out, bool fast, bool epi) {
    return tiled_kernel_f32(CFG_F32_TINY, in, out, fast, epi);
}

#define ENTRY(name, fam, T, sel)                                                                                \
    {name, fam, false, T::BM, T::BN, T::BK, T::WM, T::WN, T::EB, T::LDS_BYTES, T::THREADS, T::CPR, sel, nullptr, \
     0, 0, 0, 0, 0, 0, 0, false}
#define ENTRY_RING(name, fam, T, sel, R, rsel)                                                              \
    {name, fam, false, T::BM, T::BN, T::BK, T::WM, T::WN, T::EB, T::LDS_BYTES, T::THREADS, T::CPR, sel, rsel, \
     R::B_BK, R::B_STAGES, R::K_MULT, R::LDS_BYTES, R::LOOKAHEAD, R::A_BK, R::A_STAGES, R::A_COL_OK}
// a configuration with only a ring kernel (16-bit inputs; calls it does not
// take run the 128 x 128 configuration)
#define ENTRY_RING_ONLY(name, R, rsel)                                                                          \
    {name, TGEMM_F16, false, R::BM, R::BN, R::BK, R::WM, R::WN, 2, R::LDS_BYTES, R::THREADS, 1, nullptr, rsel, \
     R::B_BK, R::B_STAGES, R::K_MULT, R::LDS_BYTES, R::LOOKAHEAD, R::A_BK, R::A_STAGES, R::A_COL_OK}
// direct kernel: 32 x 32 per workgroup of 2 x 2 waves (16 x 16 when its four
// waves split K), steps of 32 of K
#define ENTRY_DIRECT(name, fam, eb) \
    {name, fam, true, 32, 32, 32, 2, 2, eb, 0, 256, 1, nullptr, nullptr, 0, 0, 0, 0, 0, 0, 0, false}

const ConfigEntry kConfigs[] = {
    ENTRY_RING("h256x256_w2x2", TGEMM_F16, CfgBig, tiled_kernel_big, RingBig, ring_kernel_big),
    ENTRY_RING("h128x128_w2x2", TGEMM_F16, CfgMid, tiled_kernel_mid, RingMid, ring_kernel_mid),
    ENTRY("h64x64x64_w2x2", TGEMM_F16, CfgSmall, tiled_kernel_small),
    ENTRY("h32x32x64_w1x1", TGEMM_F16, CfgTiny, tiled_kernel_tiny),
    ENTRY("s64x64x32_w2x2", TGEMM_F32, CfgF32Mid, tiled_f32_mid),
    ENTRY("s32x32x32_w1x1", TGEMM_F32, CfgF32Tiny, tiled_f32_tiny),
    ENTRY_DIRECT("h32x32_direct", TGEMM_F16, 2),
    ENTRY_DIRECT("s32x32_direct", TGEMM_F32, 4),
    ENTRY_RING_ONLY("h64x128_w2x2", RingSmall, ring_kernel_small),
    ENTRY("s128x128x32_w2x2", TGEMM_F32, CfgF32Big, tiled_f32_big),
};
constexpr int kNumConfigs = sizeof(kConfigs) / sizeof(kConfigs[0]);
static_assert(kNumConfigs == NUM_CONFIGS, "");

// Measurement-only switches, read once from the environment:
//   TGEMM_GROUP_M=<n>    tile rows per raster group (default: group_rows)
//   TGEMM_NO_SWIZZLE=1   plain LDS rows (for bank-conflict A/B runs)
//   TGEMM_NO_DL=1        register-staged kernel instead of the direct-to-LDS ring
struct Tuning {
    int group_m = 0;  // 0: group_rows decides
    bool swizzle = true;
    bool direct_lds = true;
    bool split_k = true;
    Tuning() {
        if (const char* s = getenv("TGEMM_GROUP_M")) {
            const int g = atoi(s);
            if (g > 0) group_m = g;
        }
        if (const char* s = getenv("TGEMM_NO_SWIZZLE")) swizzle = !(s[0] == '1');
        if (const char* s = getenv("TGEMM_NO_DL")) direct_lds = !(s[0] == '1');
        if (const char* s = getenv("TGEMM_NO_SPLITK")) split_k = !(s[0] == '1');
    }
};
const Tuning& tuning() {
    static const Tuning t;
    return t;
}

bool is_fp8(int dt) { return dt == TGEMM_FP8_E4M3 || dt == TGEMM_FP8_E5M2; }

int elem_bytes(int dt) { return dt == TGEMM_F32 ? 4 : is_fp8(dt) ? 1 : 2; }

bool pair_supported(int in, int out) {
    switch (in) {
        case TGEMM_F32: return out == TGEMM_F32;
        case TGEMM_F16: return out == TGEMM_F16 || out == TGEMM_F32 || is_fp8(out);
        case TGEMM_BF16: return out == TGEMM_BF16 || out == TGEMM_F32 || is_fp8(out);
        default: return false;
    }
}

// The kernels' output type: an 8-bit format is one kernel type (DT_FP8), its
// format a kernel argument.
int kernel_out(int out) { return is_fp8(out) ? DT_FP8 : out; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// The fused epilogue of a call (on = false: C := AB).
struct Epi {
    bool on = false;
    float alpha = 1.f, beta = 0.f;
    const void* bias = nullptr;
    int bias_kind = TGEMM_BIAS_NONE, bias_dt = TGEMM_F32, act = TGEMM_ACT_NONE;
};

// One product after a column-major C has been turned into a row-major one
// (C^T = B^T A^T): logical A is M x K, B is K x N, C row-major M x N.
struct Problem {
    int64_t M, N, K;
    const void* A;
    int64_t lda;
    int la;  // LAYOUT_ROW: A(i, k) at A[i * lda + k]; LAYOUT_COL: at A[k * lda + i]
    const void* B;
    int64_t ldb;
    int lb;  // LAYOUT_ROW: B(k, j) at B[k * ldb + j]; LAYOUT_COL: at B[j * ldb + k]
    void* C;
    int64_t ldc;
    int in, out;
    Epi ep;
};

bool layout_ok(int l) { return l == TGEMM_ROW_MAJOR || l == TGEMM_COL_MAJOR; }

// Bytes spanned by a stored matrix of `rows` x `cols` in its storage order.
uintptr_t span(int64_t rows, int64_t cols, int64_t ld, int eb) { return (uintptr_t)((rows - 1) * ld + cols) * eb; }

// Every pointer aligned to its element's size (8-bit outputs: any address).
bool elems_aligned(const Problem& p) {
    const uintptr_t ie = elem_bytes(p.in), oe = elem_bytes(p.out);
    if ((uintptr_t)p.A % ie != 0 || (uintptr_t)p.B % ie != 0 || (uintptr_t)p.C % oe != 0) return false;
    return !(p.ep.on && p.ep.bias_kind != TGEMM_BIAS_NONE && (uintptr_t)p.ep.bias % elem_bytes(p.ep.bias_dt) != 0);
}

int validate(const Problem& p) {
    const int64_t M = p.M, N = p.N, K = p.K;
    if (M < 0 || N < 0 || K < 0 || M > TGEMM_MAX_DIM || N > TGEMM_MAX_DIM || K > TGEMM_MAX_DIM)
        return TGEMM_ERR_DIM;
    if (!pair_supported(p.in, p.out)) return TGEMM_ERR_DTYPE;
    // stored shapes: A is M x K (row-major) or K x M (column-major); so is B
    const int64_t a_rows = p.la == LAYOUT_ROW ? M : K, a_cols = p.la == LAYOUT_ROW ? K : M;
    const int64_t b_rows = p.lb == LAYOUT_ROW ? K : N, b_cols = p.lb == LAYOUT_ROW ? N : K;
    if (p.lda < a_cols || p.ldb < b_cols || p.ldc < N) return TGEMM_ERR_LD;
    if (M == 0 || N == 0) return TGEMM_OK;
    if (p.C == nullptr) return TGEMM_ERR_NULL;
    if (K > 0 && (p.A == nullptr || p.B == nullptr)) return TGEMM_ERR_NULL;
    if (!elems_aligned(p)) return TGEMM_ERR_ALIGN;
    const uintptr_t c0 = (uintptr_t)p.C, c1 = c0 + span(M, N, p.ldc, elem_bytes(p.out));
    if (K > 0) {
        const int ie = elem_bytes(p.in);
        const uintptr_t a0 = (uintptr_t)p.A, a1 = a0 + span(a_rows, a_cols, p.lda, ie);
        const uintptr_t b0 = (uintptr_t)p.B, b1 = b0 + span(b_rows, b_cols, p.ldb, ie);
        if ((c0 < a1 && a0 < c1) || (c0 < b1 && b0 < c1)) return TGEMM_ERR_ALIAS;
    }
    if (p.ep.on && p.ep.bias_kind != TGEMM_BIAS_NONE) {
        // the bias is read while C is written: it may not overlap C
        const int64_t n = p.ep.bias_kind == TGEMM_BIAS_ROW ? M : N;
        const uintptr_t x0 = (uintptr_t)p.ep.bias, x1 = x0 + (uintptr_t)n * elem_bytes(p.ep.bias_dt);
        if (c0 < x1 && x0 < c1) return TGEMM_ERR_ALIAS;
    }
    return TGEMM_OK;
}

// The epilogue's own arguments (checked before the sizes: they are wrong
// whatever the sizes).
int validate_epi(const Epi& e) {
    if (!e.on) return TGEMM_OK;
    if (e.act < TGEMM_ACT_NONE || e.act > TGEMM_ACT_SILU) return TGEMM_ERR_EPILOGUE;
    if (e.bias_kind < TGEMM_BIAS_NONE || e.bias_kind > TGEMM_BIAS_COL) return TGEMM_ERR_EPILOGUE;
    if (e.bias_kind != TGEMM_BIAS_NONE) {
        if (e.bias_dt != TGEMM_F32 && e.bias_dt != TGEMM_F16 && e.bias_dt != TGEMM_BF16) return TGEMM_ERR_EPILOGUE;
        if (e.bias == nullptr) return TGEMM_ERR_EPILOGUE;
    }
    return TGEMM_OK;
}

// 16-byte loads of A and B need 16-byte aligned bases and leading dimensions
// that are whole 16-byte chunks.
bool loads_aligned(const ConfigEntry& c, const Problem& p) {
    const int ve = 16 / c.eb;
    return ((uintptr_t)p.A % 16 == 0) && ((uintptr_t)p.B % 16 == 0) && (p.lda % ve == 0) && (p.ldb % ve == 0);
}

// 4-element stores of C need a base aligned to 4 elements and ldc % 4 == 0.
bool stores_aligned(const Problem& p) {
    return ((uintptr_t)p.C % (4 * (uintptr_t)elem_bytes(p.out)) == 0) && (p.ldc % 4 == 0);
}

int64_t tiles_for(const ConfigEntry& c, int64_t M, int64_t N) { return ceil_div(M, c.bm) * ceil_div(N, c.bn); }

bool row_row(const Problem& p) { return p.la == LAYOUT_ROW && p.lb == LAYOUT_ROW; }

// Whether a register-staged configuration runs its unchecked path: whole
// tiles, 16-byte aligned operands, 4-element aligned C rows, offsets within
// 31 bits.
bool tiled_fast(const ConfigEntry& c, const Problem& p) {
    const bool offsets_fit = (int64_t)c.bm * p.lda * c.eb + p.K * c.eb < (1LL << 31) &&
                             (int64_t)c.bk * p.ldb * c.eb + p.N * c.eb < (1LL << 31);
    return loads_aligned(c, p) && stores_aligned(p) && offsets_fit && p.M % c.bm == 0 && p.N % c.bn == 0;
}

// Largest buffer offset (bytes) of an operand whose tile spans `ext` rows /
// columns, read over K + extra of K: k contiguous in memory (row-major A,
// column-major B) or strided.
int64_t operand_reach(bool kcontig, int64_t ext, int64_t ld, int64_t K, int64_t extra, int eb) {
    return (kcontig ? ext * ld + K + extra : (K + extra) * ld + ext) * eb;
}

// Buffer-range pad that makes the ring kernel read every element of a 16-bit
// operand stored with rows of `outer` elements (k contiguous: the row is K
// long) at leading dimension ld from base X: 0, 2, or -1 for none.  Its
// 16-byte loads (any even address) keep a 4-byte part only when the part ends
// inside the buffer range, which ends at the dword boundary after the
// operand's last element: the last element is dropped if it starts a part
// (an odd element count from the row's first loaded one: K for a
// k-contiguous operand, M or N for a k-strided one) at an address of 2 mod 4.
// Then 2 more bytes keep it; they are read (their values reach only outputs
// past N or positions past K), so they must lie in the element's page: -1
// when they start a new 4 KiB page, and the kernel then loads that element
// on its own in its K tail (GemmArgs::last_fix).  Rows of whole 16-byte
// chunks never need a pad.
int ring_range_pad(const void* X, int64_t ld, bool kcontig, int64_t outer, int64_t K) {
    const int64_t rows = kcontig ? outer : K, cols = kcontig ? K : outer;
    if (rows <= 0 || cols <= 0) return 0;
    const uintptr_t last = (uintptr_t)X + (uintptr_t)((rows - 1) * ld + cols - 1) * 2;
    if ((cols % 2) == 0 || last % 4 != 2) return 0;
    return (last + 2) % 4096 != 0 ? 2 : -1;
}
int ring_pad_a(const Problem& p) { return ring_range_pad(p.A, p.lda, p.la == LAYOUT_ROW, p.M, p.K); }
int ring_pad_b(const Problem& p) { return ring_range_pad(p.B, p.ldb, p.lb == LAYOUT_COL, p.N, p.K); }
// GemmArgs::last_fix of a ring call, and whether it needs the KT variant for
// it (a k-strided operand's last k-row left to the tail)
int ring_last_fix(const Problem& p) { return (ring_pad_a(p) < 0 ? 1 : 0) | (ring_pad_b(p) < 0 ? 2 : 0); }
bool ring_fix_needs_tail(const Problem& p) {
    const int f = ring_last_fix(p);
    return ((f & 1) && p.la == LAYOUT_COL) || ((f & 2) && p.lb == LAYOUT_ROW);
}

// Whether a configuration with a ring kernel runs it.
bool ring_applies(const ConfigEntry& c, const Problem& p) {
    if (c.ring == nullptr || !tuning().direct_lds) return false;
    if (p.la == LAYOUT_COL && !c.ring_a_col) return false;
    // the ring loads ring_lookahead steps past K
    const int64_t extra = (int64_t)c.ring_lookahead * c.ring_bk;
    // 16-bit elements at even addresses: rows of whole 16-byte chunks, or
    // ranges padded where needed, or the last element loaded on its own
    // (ring_range_pad)
    const bool loads_ok = (uintptr_t)p.A % 2 == 0 && (uintptr_t)p.B % 2 == 0;
    // any K: a multiple of ring_k_mult, or the K-tail variant, which below
    // ring_k_mult runs the tail alone (steps of 32 with fragments loaded
    // straight from global memory; measured as fast as the register-staged
    // tiles for 16-bit outputs at 4096^2 x 16..100, and 2-7x faster than the
    // direct kernel that 8-bit outputs took there); any N and C alignment
    // (ring_plain_stores)
    return loads_ok && p.K > 0 &&
           operand_reach(p.la == LAYOUT_ROW, c.bm, p.lda, p.K, extra, c.eb) < (1LL << 31) &&
           operand_reach(p.lb == LAYOUT_COL, c.bn, p.ldb, p.K, extra, c.eb) < (1LL << 31);
}

// Whether the ring kernel's plain epilogue can store C: whole groups of four
// columns (N % 4 == 0) in rows aligned for 4-element stores.  Otherwise the
// fused epilogue runs, with the identity epilogue when none was asked for.
bool ring_plain_stores(const Problem& p) { return stores_aligned(p) && p.N % 4 == 0; }

// Whether the direct kernel's buffer offsets fit (32 rows / columns of each
// operand over K + 320 of K).
bool direct_fits(const Problem& p) {
    const int eb = elem_bytes(p.in);
    return operand_reach(p.la == LAYOUT_ROW, 32, p.lda, p.K, 320, eb) < (1LL << 31) &&
           operand_reach(p.lb == LAYOUT_COL, 32, p.ldb, p.K, 320, eb) < (1LL << 31);
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
// Column-major operands have no register-staged kernel: the ring kernels
// where they apply, the direct kernel elsewhere.
// Exact calls timed by the configuration search (tune.py): the measured
// winner, before the rule.  Row-major operands and C only; the last entry is
// a sentinel that matches nothing.
struct TunedEntry {
    int64_t M, N, K, lda, ldb, ldc;
    int in, out, config;
};
const TunedEntry kTuned[] = {
#include "tuned_table.inc"
    {-1, -1, -1, -1, -1, -1, -1, -1, -1},
};

int tuned_choice(const Problem& p) {
    if (!row_row(p)) return -1;
    for (const TunedEntry& e : kTuned)
        if (e.M == p.M && e.N == p.N && e.K == p.K && e.lda == p.lda && e.ldb == p.ldb && e.ldc == p.ldc &&
            e.in == p.in && e.out == p.out && e.config >= 0 && e.config < kNumConfigs &&
            kConfigs[e.config].in_family == (p.in == TGEMM_F32 ? TGEMM_F32 : TGEMM_F16))
            return e.config;
    return -1;
}

// Split-K: slices of K for a ring configuration whose tiles leave CUs idle
// (128 workgroups or fewer on the 256 CUs) when K is long (4096 or more;
// at 2048 the second kernel and the workspace cost more than the slices
// gain: 1024 x 512 x 2048 28 against 26 us).  Each slice is
// a multiple of the ring's K step (the last one takes the rest, with the K
// tail when K is not a multiple), at least 256 long, and the slices bring
// the workgroups to about 256; the fp32 partials go through a workspace of
// splits x M x roundup(N, 4) floats (at most 256 MiB).  Needs the plain
// epilogue's whole groups (N % 4 == 0) and rows of whole 16-byte chunks.
// Returns the slice count (1: no split) and the slice length.
int split_count(const ConfigEntry& c, const Problem& p, int& k_split) {
    k_split = (int)p.K;
    if (!tuning().split_k || c.ring == nullptr || p.N % 4 != 0 || !loads_aligned(c, p)) return 1;
    const int64_t tiles = tiles_for(c, p.M, p.N);
    if (tiles > 128 || p.K < 4096) return 1;
    const int64_t km = c.ring_k_mult;
    // workgroups the CUs hold at once: two per CU where the ring's LDS allows
    const int64_t slots = 256 * (c.ring_lds <= 80 * 1024 ? 2 : 1);
    int64_t s = slots / tiles;
    if (s > p.K / 256) s = p.K / 256;
    if (s > 32) s = 32;
    const int64_t ldw = (p.N + 3) / 4 * 4;
    while (s > 1 && s * p.M * ldw * 4 > ((int64_t)256 << 20)) --s;
    for (; s > 1; --s) {
        const int64_t len = ((p.K + s - 1) / s + km - 1) / km * km;
        const int64_t n = (p.K + len - 1) / len;
        const int64_t last = p.K - (n - 1) * len;
        // every slice a whole number of K steps or above one (the K tail)
        if (n > 1 && (last % km == 0 || last > km)) {
            k_split = (int)len;
            return (int)n;
        }
    }
    return 1;
}

// Whether 256 x 256 tiles beat 128 x 128 ones: when they fill every CU, or
// when 128 x 128 tiles would take three or more rounds of the 256 CUs (a
// 256 x 256 tile does its four times the work in ~2.4 times the time of a
// 128 x 128 one, measured: 3072^3 62 against 75 us; with two rounds the
// smaller tile still wins, 8192 x 1024 x 8192 118 against 134 us).
bool big_tiles_pay(int64_t M, int64_t N) {
    return tiles_for(kConfigs[CFG_BIG], M, N) >= 256 || tiles_for(kConfigs[CFG_MID], M, N) > 512;
}

// Steps of 32 of K that the direct kernel keeps in flight (its register
// ring): as many as keep its loads within the 63 that vmcnt counts, 2 to 8.
int direct_depth(const Problem& p, bool va, bool vb) {
    const int per_step = p.in == TGEMM_F32 ? 16 : (va ? 1 : 8) + (vb ? 1 : 8);
    const int d = 63 / per_step;
    return d < 2 ? 2 : d > 8 ? 8 : d;
}

// How the direct kernel runs a call: its 16-byte load flags, whether K goes
// over the four waves (when one ring of steps does not cover K and a quarter
// of the steps fits one), whether all of a wave's loads are in flight at
// once (one memory round trip), and its workgroups.
struct DirectShape {
    bool va, vb, wave_split, one_trip;
    int64_t workgroups;
};
DirectShape direct_shape(const Problem& p) {
    DirectShape d;
    const bool kca = p.la == LAYOUT_ROW, kcb = p.lb == LAYOUT_COL;
    const bool half = p.in != TGEMM_F32;
    d.va = half && kca && (uintptr_t)p.A % 16 == 0 && p.lda % 8 == 0 && p.K % 8 == 0;
    d.vb = half && kcb && (uintptr_t)p.B % 16 == 0 && p.ldb % 8 == 0 && p.K % 8 == 0;
    const int64_t steps = p.K / 32, depth = direct_depth(p, d.va, d.vb);
    d.wave_split = steps > depth && (steps + 3) / 4 <= depth;
    d.one_trip = steps <= depth || d.wave_split;
    const int t = d.wave_split ? 16 : 32;
    d.workgroups = ceil_div(p.M, t) * ceil_div(p.N, t);
    return d;
}

int table_choice(const Problem& p) {
    const int tuned = tuned_choice(p);
    if (tuned >= 0) return tuned;
    const int64_t M = p.M, N = p.N;
    const bool small = M * N <= (1LL << 18);
    if (p.in == TGEMM_F32) {
        if (!row_row(p)) return CFG_F32_DIRECT;
        // 128 x 128 tiles where they fill the CUs (4096^3: 977 against
        // 1099 us on 64 x 64, 2048^3: 138 against 145 us), else 64 x 64
        if (tiles_for(kConfigs[CFG_F32_BIG], M, N) >= 256) return CFG_F32_BIG;
        if (tiles_for(kConfigs[CFG_F32_MID], M, N) >= 256) return CFG_F32_MID;
        // the direct kernel where all of K's loads go out at once, from
        // K = 128 and up to 256 workgroups (traced: 128^3 3.8 against 5.2 us
        // on 32 x 32 tiles, 256^2 x 256 5.0 against 7.9; K = 64, longer K
        // or more workgroups: the 32 x 32 tile)
        if (small && p.K >= 128 && direct_fits(p)) {
            const DirectShape d = direct_shape(p);
            if (d.one_trip && d.workgroups <= 256) return CFG_F32_DIRECT;
        }
        if (small && !tiled_fast(kConfigs[CFG_F32_TINY], p)) return CFG_F32_DIRECT;
        return CFG_F32_TINY;
    }
    if (!row_row(p)) {
        if (big_tiles_pay(M, N) && ring_applies(kConfigs[CFG_BIG], p)) return CFG_BIG;
        // small products whose C the ring could store only through the fused
        // epilogue stay on the direct kernel, unless K is long enough for
        // slices of K
        int k_split;
        if (ring_applies(kConfigs[CFG_MID], p) &&
            (ring_plain_stores(p) || !small || split_count(kConfigs[CFG_MID], p, k_split) > 1))
            return CFG_MID;
        return CFG_DIRECT;
    }
    if (big_tiles_pay(M, N)) return CFG_BIG;
    // fewer 128 x 128 tiles than CUs: 64 x 128 tiles (twice the workgroups)
    if (tiles_for(kConfigs[CFG_MID], M, N) >= 64 && tiles_for(kConfigs[CFG_MID], M, N) < 256 &&
        ring_applies(kConfigs[CFG_RING_SMALL], p))
        return CFG_RING_SMALL;
    if (tiles_for(kConfigs[CFG_MID], M, N) >= 128 && ring_applies(kConfigs[CFG_MID], p)) return CFG_MID;
    if (tiles_for(kConfigs[CFG_MID], M, N) >= 256) return CFG_MID;
    // small products with 128 <= K <= 512: the direct kernel where all of
    // K's loads go out at once and it runs at most 576 workgroups (traced
    // kernel times: 128^2 x 512 3.4 us against 5.0 on the 64 x 128 ring and
    // 7.5 on 32 x 32 tiles, 384^2 x 512 5.2 against 5.8; 512^2 x 256, 1024
    // workgroups: 5.2 against 4.9 on the ring)
    if (small && p.K >= 128 && p.K <= 512 && direct_fits(p)) {
        const DirectShape d = direct_shape(p);
        if (d.one_trip && d.workgroups <= 576) return CFG_DIRECT;
    }
    // fewer tiles: the 64 x 128 ring (in slices of K when K is long).  It
    // beats the register-staged 64 x 64 tile on every product measured from
    // 256^3 to 768^3 and 512 x 512 x 2048 (7.8 against 9.3 us at 512^3, 12.8
    // against 23.6 us at 512 x 512 x 2048), and from K = 1024 every other
    // kernel even on one or two of its tiles (64^2 x 1024 6.1 us against 7.5
    // direct and 11.9 on 32 x 32 tiles); below 4 of its tiles and a shorter
    // K, or with a small C it could store only through the fused epilogue,
    // the other kernels stay
    int k_split;
    if ((tiles_for(kConfigs[CFG_RING_SMALL], M, N) >= 4 || p.K >= 1024) &&
        ring_applies(kConfigs[CFG_RING_SMALL], p) &&
        (ring_plain_stores(p) || !small || split_count(kConfigs[CFG_RING_SMALL], p, k_split) > 1))
        return CFG_RING_SMALL;
    if (tiles_for(kConfigs[CFG_SMALL], M, N) >= 256) return CFG_SMALL;
    if (small && !tiled_fast(kConfigs[CFG_TINY], p)) return CFG_DIRECT;
    return CFG_TINY;
}

int family_of(int in) { return in == TGEMM_F32 ? TGEMM_F32 : TGEMM_F16; }

// What one call runs: the configuration, the kernel and its kind.
struct Plan {
    int config;
    int kind;  // TGEMM_KERNEL_*
    KernelFn fn;
    int splits = 1, k_split = 0;          // split-K (kind TGEMM_KERNEL_RING_SPLITK)
    bool wave_split = false;              // direct kernel: K over the four waves, 16 x 16 tiles
    SplitkReduceFn reduce = nullptr;      // the sum of the slices
};

int plan_direct(const Problem& p, Plan& plan) {
    const DirectShape d = direct_shape(p);
    plan.kind = TGEMM_KERNEL_DIRECT;
    plan.fn = direct_kernel(p.in, kernel_out(p.out), p.la, p.lb, d.va, d.vb, p.ep.on || is_fp8(p.out));
    if (plan.fn == nullptr) return TGEMM_ERR_DTYPE;
    plan.wave_split = d.wave_split;
    if (d.workgroups > 0x7fffffff) return TGEMM_ERR_DIM;
    return TGEMM_OK;
}

// Validates the arguments and picks the kernel; returns TGEMM_OK (plan
// filled; M == 0 or N == 0 leaves plan.fn null) or a negative error code.
int make_plan(const Problem& p, int config_id, Plan& plan) {
    const int ve = validate_epi(p.ep);
    if (ve != TGEMM_OK) return ve;
    const int v = validate(p);
    if (v != TGEMM_OK) return v;
    if (config_id < -1 || config_id >= kNumConfigs) return TGEMM_ERR_CONFIG;
    if (config_id >= 0 && kConfigs[config_id].in_family != family_of(p.in)) return TGEMM_ERR_CONFIG;
    // configurations with only a register-staged kernel serve row-major
    // operands only
    if (config_id >= 0 && !row_row(p) && !kConfigs[config_id].direct && kConfigs[config_id].ring == nullptr)
        return TGEMM_ERR_CONFIG;
    plan.config = config_id >= 0 ? config_id : table_choice(p);
    plan.fn = nullptr;
    plan.kind = TGEMM_KERNEL_GENERAL;
    if (p.M == 0 || p.N == 0) return TGEMM_OK;
    // a ring-only configuration whose ring kernel does not take the call
    // (unaligned operands, short K, a column-major A it has no kernel for)
    // runs the 128 x 128 configuration instead
    if (!kConfigs[plan.config].direct && kConfigs[plan.config].tiled == nullptr &&
        !ring_applies(kConfigs[plan.config], p))
        plan.config = CFG_MID;
    const ConfigEntry& c = kConfigs[plan.config];
    if (!c.direct && ring_applies(c, p) && config_id < 0) {
        int k_split;
        const int splits = split_count(c, p, k_split);
        if (splits > 1) {
            // fp32 partials of the slices (plain epilogue), then their sum
            // with the call's epilogue and output type
            plan.kind = TGEMM_KERNEL_RING_SPLITK;
            plan.splits = splits;
            plan.k_split = k_split;
            plan.fn = c.ring(p.in, DT_F32, p.la, p.lb, false, p.K % c.ring_k_mult != 0);
            plan.reduce = splitk_reduce_kernel_for(kernel_out(p.out));
            if (plan.fn == nullptr || plan.reduce == nullptr) return TGEMM_ERR_DTYPE;
            return ceil_div(p.M, c.bm) * ceil_div(p.N, c.bn) * splits > 0x7fffffff ? TGEMM_ERR_DIM : TGEMM_OK;
        }
    }
    if (!c.direct && ring_applies(c, p)) {
        plan.kind = TGEMM_KERNEL_RING;
        // 8-bit outputs are written by the fused epilogue's kernels
        plan.fn = c.ring(p.in, kernel_out(p.out), p.la, p.lb, p.ep.on || is_fp8(p.out) || !ring_plain_stores(p),
                         p.K % c.ring_k_mult != 0 || ring_fix_needs_tail(p));
        if (plan.fn == nullptr) return TGEMM_ERR_DTYPE;
        return ceil_div(p.M, c.bm) * ceil_div(p.N, c.bn) > 0x7fffffff ? TGEMM_ERR_DIM : TGEMM_OK;
    }
    if (c.direct || !row_row(p) || is_fp8(p.out)) {
        // column-major operands outside the ring kernel's cases run direct,
        // and so do 8-bit outputs (the register-staged kernels write 16- and
        // 32-bit outputs only)
        if (direct_fits(p)) {
            if (!c.direct) plan.config = p.in == TGEMM_F32 ? CFG_F32_DIRECT : CFG_DIRECT;
            return plan_direct(p, plan);
        }
        if (!row_row(p) || is_fp8(p.out)) return TGEMM_ERR_DIM;  // offsets beyond 31 bits: no kernel
        plan.config = p.in == TGEMM_F32 ? CFG_F32_TINY : CFG_TINY;  // the checked kernel instead
    }
    const ConfigEntry& t = kConfigs[plan.config];
    const bool fast = tiled_fast(t, p);
    plan.kind = fast ? TGEMM_KERNEL_TILED : TGEMM_KERNEL_GENERAL;
    plan.fn = t.tiled(p.in, p.out, fast, p.ep.on);
    if (plan.fn == nullptr) return TGEMM_ERR_DTYPE;
    return ceil_div(p.M, t.bm) * ceil_div(p.N, t.bn) > 0x7fffffff ? TGEMM_ERR_DIM : TGEMM_OK;
}

// The problem of a call: a column-major C is computed as the row-major
// C^T = B^T A^T (M and N swapped, A and B swapped, each operand's layout
// flipped: a row-major K x N B read as an N x K matrix is column-major).
// A fused epilogue goes along; its bias per row of C becomes one per column
// of C^T and the other way round.
int make_problem(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, int la, const void* B, int64_t ldb,
                 int lb, void* C, int64_t ldc, int lc, int in, int out, Problem& p,
                 const tgemm_epilogue* ep = nullptr) {
    if (!layout_ok(la) || !layout_ok(lb) || !layout_ok(lc)) return TGEMM_ERR_LAYOUT;
    if (lc == TGEMM_ROW_MAJOR)
        p = Problem{M, N, K, A, lda, la, B, ldb, lb, C, ldc, in, out};
    else
        p = Problem{N, M, K, B, ldb, lb ^ 1, A, lda, la ^ 1, C, ldc, in, out};
    if (ep != nullptr) {
        p.ep.on = true;
        p.ep.alpha = ep->alpha;
        p.ep.beta = ep->beta;
        p.ep.bias = ep->bias;
        p.ep.bias_kind = ep->bias_kind;
        p.ep.bias_dt = ep->bias_dtype;
        p.ep.act = ep->activation;
        if (lc == TGEMM_COL_MAJOR && ep->bias_kind == TGEMM_BIAS_ROW) p.ep.bias_kind = TGEMM_BIAS_COL;
        else if (lc == TGEMM_COL_MAJOR && ep->bias_kind == TGEMM_BIAS_COL) p.ep.bias_kind = TGEMM_BIAS_ROW;
    }
    return TGEMM_OK;
}

// The scratch of the allocation-free entry point (gemm_fused_noalloc): the
// split-K workspace as a file-scope device array, which every GPU that loads
// the library holds until the process ends, each its own copy.  32 MiB: the
// largest workspace a split plan takes (slices x tiles stay within the 512
// workgroups that the CUs hold at once, each partial tile at most 128 x 128
// fp32 values).  Host code uses its device address (scratch_address), never
// the array's name.
constexpr int64_t kScratchFloats = (int64_t)8 << 20;
static __device__ __align__(256) float scratch[kScratchFloats];

// This GPU's address of `scratch`: looked up once per device, with that
// device current, and kept.
int scratch_address(float** out) {
    static std::mutex mu;
    static float* addr[64] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return (int)e;
    if (dev < 0 || dev >= 64) return TGEMM_ERR_SCRATCH;
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return (int)e;
        if (ptr == nullptr) return TGEMM_ERR_SCRATCH;
        addr[dev] = (float*)ptr;
    }
    *out = addr[dev];
    return TGEMM_OK;
}

// The library's memory pool of the current device, for split-K workspaces:
// stream-ordered allocations (a workspace of one stream is never another's
// while in use), and memory kept in the pool rather than released to the HIP
// runtime at each synchronisation (the default pool's release threshold is
// 0).
hipMemPool_t workspace_pool(hipError_t& e) {
    static std::mutex mu;
    static hipMemPool_t pools[64] = {};
    int dev = 0;
    e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if (pools[dev] == nullptr) {
        hipMemPoolProps props = {};
        props.allocType = hipMemAllocationTypePinned;
        props.location.type = hipMemLocationTypeDevice;
        props.location.id = dev;
        hipMemPool_t pool = nullptr;
        e = hipMemPoolCreate(&pool, &props);
        if (e != hipSuccess) return nullptr;
        uint64_t keep = UINT64_MAX;
        e = hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &keep);
        if (e != hipSuccess) return nullptr;
        pools[dev] = pool;
    }
    return pools[dev];
}

// Split-K workspaces kept between calls: one per stream for the last
// kWorkspaces streams of each device.  Taking a workspace from the pool and
// giving it back cost 10 to 30 us of host time per call (measured on MI355X
// with ROCm 7), more than the two kernels of a small product take on the
// GPU; an event recorded after a call's kernels and waited on by the next
// user of the workspace costs about 1.6 us.  The wait also covers a stream
// handle that the runtime hands out again after a stream was destroyed with
// work still queued on the workspace.  An entry that must grow, or that
// another stream takes over (the least recently used one), gives its memory
// back to the pool in the new user's stream order after that event.
constexpr int kWorkspaces = 8;
struct StreamWorkspace {
    hipStream_t stream = nullptr;
    void* ptr = nullptr;
    size_t bytes = 0;
    hipEvent_t last = nullptr;  // recorded after the last call's kernels
    uint64_t used = 0;          // least recently used: smallest stamp
};
std::mutex workspace_mu;  // held across a call's kernels (see run_split)
StreamWorkspace workspaces[64][kWorkspaces];
uint64_t workspace_clock = 0;

// The workspace of `st` on device `dev` with at least `need` bytes, ordered
// after the previous call that used its memory (workspace_mu held).
hipError_t stream_workspace(int dev, hipStream_t st, size_t need, StreamWorkspace*& out) {
    StreamWorkspace* row = workspaces[dev];
    StreamWorkspace* w = nullptr;
    for (int i = 0; i < kWorkspaces && w == nullptr; ++i)
        if (row[i].ptr != nullptr && row[i].stream == st) w = &row[i];
    if (w == nullptr) {  // a free entry, else the least recently used one
        w = &row[0];
        for (int i = 0; i < kWorkspaces; ++i) {
            if (row[i].ptr == nullptr) { w = &row[i]; break; }
            if (row[i].used < w->used) w = &row[i];
        }
    }
    hipError_t e = hipSuccess;
    if (w->last == nullptr && (e = hipEventCreateWithFlags(&w->last, hipEventDisableTiming)) != hipSuccess) return e;
    if (w->ptr != nullptr && (e = hipStreamWaitEvent(st, w->last, 0)) != hipSuccess) return e;
    if (w->ptr == nullptr || w->bytes < need) {
        if (w->ptr != nullptr) {
            e = hipFreeAsync(w->ptr, st);
            w->ptr = nullptr;
            w->bytes = 0;
            if (e != hipSuccess) return e;
        }
        hipMemPool_t pool = workspace_pool(e);
        if (pool == nullptr) return e;
        const size_t bytes = (need + ((size_t)2 << 20) - 1) / ((size_t)2 << 20) * ((size_t)2 << 20);  // 2 MiB steps
        if ((e = hipMallocFromPoolAsync(&w->ptr, bytes, pool, st)) != hipSuccess) {
            w->ptr = nullptr;
            return e;
        }
        w->bytes = bytes;
    }
    w->stream = st;
    w->used = ++workspace_clock;
    out = w;
    return hipSuccess;
}

// Split-K: the slices' fp32 partials into the stream's workspace, then their
// sum with the call's epilogue into C.  The library's lock is held from the
// workspace lookup to the event after the second kernel, so that two host
// threads calling on one stream cannot interleave their kernels on one
// workspace.
// With `fixed` (the allocation-free entry point) the workspace is that
// device array instead, and nothing is allocated, freed or recorded.
int run_split(const Problem& p, const Plan& plan, const ConfigEntry& c, const GemmArgs& args, void* stream,
              float* fixed) {
    const hipStream_t st = (hipStream_t)stream;
    const int64_t ldw = (p.N + 3) / 4 * 4, slice = p.M * ldw;
    float* w = fixed;
    hipError_t e = hipSuccess;
    std::unique_lock<std::mutex> lock(workspace_mu, std::defer_lock);
    StreamWorkspace* ws = nullptr;
    if (fixed != nullptr) {
        if (plan.splits * slice > kScratchFloats) return TGEMM_ERR_SCRATCH;
    } else {
        int dev = 0;
        if ((e = hipGetDevice(&dev)) != hipSuccess) return (int)e;
        if (dev < 0 || dev >= 64) return (int)hipErrorInvalidDevice;
        lock.lock();
        if ((e = stream_workspace(dev, st, (size_t)(plan.splits * slice * 4), ws)) != hipSuccess) return (int)e;
        w = (float*)ws->ptr;
    }
    GemmArgs pa = args;
    pa.C = (char*)w;
    pa.ldc = ldw;
    pa.epi = 0;
    pa.vec_c = 1;
    pa.range_pad_a = pa.range_pad_b = 0;
    pa.last_fix = 0;
    pa.splits = plan.splits;
    pa.k_split = plan.k_split;
    pa.split_stride = slice * 4;
    const int64_t tiles = (int64_t)pa.tiles_m * pa.tiles_n;
    void* kargs[] = {&pa};
    e = hipLaunchKernel((const void*)plan.fn, dim3((unsigned)(tiles * plan.splits)), dim3(c.threads), kargs, 0, st);
    if (e == hipSuccess) e = hipGetLastError();
    if (e == hipSuccess) {
        GemmArgs ra = args;
        if (!p.ep.on) {  // the identity epilogue: C := the sum
            ra.alpha = 1.f;
            ra.beta = 0.f;
            ra.bias_kind = TGEMM_BIAS_NONE;
            ra.act = ACT_NONE;
        }
        const int64_t groups = p.M * ((p.N + 3) / 4);
        const float* wc = w;
        int64_t ldw_ = ldw, slice_ = slice;
        int splits = plan.splits;
        void* rargs[] = {&ra, &wc, &ldw_, &slice_, &splits};
        const int64_t rb = (groups + kSplitkReduceThreads - 1) / kSplitkReduceThreads;
        e = hipLaunchKernel((const void*)plan.reduce, dim3((unsigned)rb), dim3(kSplitkReduceThreads), rargs, 0, st);
        if (e == hipSuccess) e = hipGetLastError();
    }
    if (ws != nullptr) {
        const hipError_t f = hipEventRecord(ws->last, st);
        if (e == hipSuccess) e = f;
    }
    return e == hipSuccess ? TGEMM_OK : (int)e;
}

// Tile rows per raster group of the tile map.  4 (8 ties at 8192^3; 2 and
// 16 are 1-4% slower there), except for a short K with rows of C a multiple
// of 32 KiB apart, where 2 is faster (medians on one box, ring kernel:
// 16384^2 x 1024 fp16 547 against 587 us, x 512 379 against 403, x 2048 895
// against 926; 8192 x 16384 x 1024 275 against 289; 8192^2 x 1024 with fp32
// C 144 against 161), and 4 stays ahead with other row pitches (12288^2 x
// 1536 399 against 408, 8192^2 x 1024 to 4096 with fp16 C by 0.5-1%).
int group_rows(const Problem& p) {
    const int64_t pitch = p.ldc * elem_bytes(p.out);
    return p.K <= 2048 && pitch % (32 * 1024) == 0 ? 2 : 4;
}

int run(const Problem& p, void* stream, int config_id, float* fixed = nullptr) {
    Plan plan;
    const int v = make_plan(p, config_id, plan);
    if (v != TGEMM_OK || plan.fn == nullptr) return v;
    const ConfigEntry& c = kConfigs[plan.config];

    GemmArgs args;
    args.A = (const char*)p.A;
    args.B = (const char*)p.B;
    args.C = (char*)p.C;
    args.lda = p.lda;
    args.ldb = p.ldb;
    args.ldc = p.ldc;
    args.M = (int)p.M;
    args.N = (int)p.N;
    args.K = (int)p.K;
    args.tiles_m = (int)ceil_div(p.M, plan.wave_split ? 16 : c.bm);
    args.tiles_n = (int)ceil_div(p.N, plan.wave_split ? 16 : c.bn);
    args.group_m = tuning().group_m > 0 ? tuning().group_m : group_rows(p);
    args.swz_mask = tuning().swizzle ? c.cpr - 1 : 0;
    if (plan.kind == TGEMM_KERNEL_RING || plan.kind == TGEMM_KERNEL_RING_SPLITK)
        args.swz_mask = tuning().swizzle ? 1 : 0;
    args.vec_ab = loads_aligned(c, p);
    args.vec_c = stores_aligned(p);
    args.epi = p.ep.on ? 1 : 0;
    args.alpha = p.ep.alpha;
    args.beta = p.ep.beta;
    args.bias = (const char*)p.ep.bias;
    args.bias_kind = p.ep.on ? p.ep.bias_kind : TGEMM_BIAS_NONE;
    args.bias_dt = p.ep.bias_dt;
    args.act = p.ep.act;
    args.fp8_e5m2 = p.out == TGEMM_FP8_E5M2 ? 1 : 0;
    args.splits = plan.wave_split ? 4 : 1;  // the direct kernel's K over its waves
    args.k_split = (int)p.K;
    args.split_stride = 0;
    const bool ring = plan.kind == TGEMM_KERNEL_RING;
    args.range_pad_a = ring && ring_pad_a(p) > 0 ? ring_pad_a(p) : 0;
    args.range_pad_b = ring && ring_pad_b(p) > 0 ? ring_pad_b(p) : 0;
    args.last_fix = ring ? ring_last_fix(p) : 0;
    const int64_t grid = (int64_t)args.tiles_m * args.tiles_n;

    if (plan.kind == TGEMM_KERNEL_RING_SPLITK) return run_split(p, plan, c, args, stream, fixed);
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
    return gemm_t(M, N, K, A, lda, TGEMM_ROW_MAJOR, B, ldb, TGEMM_ROW_MAJOR, C, ldc, TGEMM_ROW_MAJOR, in_dtype,
                  out_dtype, stream, -1);
}

int gemm_ex(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb, void* C,
            int64_t ldc, int in_dtype, int out_dtype, void* stream, int config_id) {
    return gemm_t(M, N, K, A, lda, TGEMM_ROW_MAJOR, B, ldb, TGEMM_ROW_MAJOR, C, ldc, TGEMM_ROW_MAJOR, in_dtype,
                  out_dtype, stream, config_id);
}

int gemm_t(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, int layout_a, const void* B, int64_t ldb,
           int layout_b, void* C, int64_t ldc, int layout_c, int in_dtype, int out_dtype, void* stream,
           int config_id) {
    Problem p;
    const int v = make_problem(M, N, K, A, lda, layout_a, B, ldb, layout_b, C, ldc, layout_c, in_dtype, out_dtype, p);
    if (v != TGEMM_OK) return v;
    return run(p, stream, config_id);
}

int gemm_fused(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, int layout_a, const void* B,
               int64_t ldb, int layout_b, void* C, int64_t ldc, int layout_c, int in_dtype, int out_dtype,
               const tgemm_epilogue* epilogue, void* stream, int config_id) {
    Problem p;
    const int v = make_problem(M, N, K, A, lda, layout_a, B, ldb, layout_b, C, ldc, layout_c, in_dtype, out_dtype, p,
                               epilogue);
    if (v != TGEMM_OK) return v;
    return run(p, stream, config_id);
}

int gemm_fused_noalloc(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, int layout_a, const void* B,
                       int64_t ldb, int layout_b, void* C, int64_t ldc, int layout_c, int in_dtype, int out_dtype,
                       const tgemm_epilogue* epilogue, void* stream, int config_id) {
    Problem p;
    const int v = make_problem(M, N, K, A, lda, layout_a, B, ldb, layout_b, C, ldc, layout_c, in_dtype, out_dtype, p,
                               epilogue);
    if (v != TGEMM_OK) return v;
    float* fixed = nullptr;
    const int a = scratch_address(&fixed);
    if (a != TGEMM_OK) return a;
    return run(p, stream, config_id, fixed);
}

const char* gemm_strerror(int code) {
    switch (code) {
        case TGEMM_OK: return "success";
        case TGEMM_ERR_DIM: return "a size negative or too large (attention: also keys = 0 with queries)";
        case TGEMM_ERR_NULL: return "NULL pointer for a non-empty operand";
        case TGEMM_ERR_LD: return "leading dimension smaller than the stored row width (attention: output elements overlap)";
        case TGEMM_ERR_DTYPE: return "unsupported (in_dtype, out_dtype) pair";
        case TGEMM_ERR_ALIAS: return "output overlaps an input";
        case TGEMM_ERR_CONFIG:
            return "unknown tile configuration, configuration for another input type, or one without a kernel for "
                   "column-major operands";
        case TGEMM_ERR_LAYOUT: return "layout is neither TGEMM_ROW_MAJOR nor TGEMM_COL_MAJOR";
        case TGEMM_ERR_EPILOGUE:
            return "epilogue: unknown activation, bias kind or bias type, or a bias kind without a bias pointer";
        case TGEMM_ERR_HEAD_DIM: return "attention: head dimension is neither 64 nor 128";
        case TGEMM_ERR_SCRATCH:
            return "gemm_fused_noalloc: the call needs more workspace than the library's fixed scratch holds";
        case TGEMM_ERR_ALIGN: return "a pointer not aligned to the size of its element type";
        default: break;
    }
    if (code > 0) return hipGetErrorString((hipError_t)code);
    return "unknown error code";
}

int gemm_num_configs(void) { return kNumConfigs; }

int gemm_config_info(int id, tgemm_config_info* out) {
    if (id < 0 || id >= kNumConfigs || out == nullptr) return TGEMM_ERR_CONFIG;
    const ConfigEntry& c = kConfigs[id];
    const bool ring = c.ring != nullptr;
    out->id = id;
    out->in_dtype = c.in_family;
    out->block_m = c.bm;
    out->block_n = c.bn;
    out->threads = c.threads;
    out->waves_m = c.wm;
    out->waves_n = c.wn;
    out->name = c.name;
    if (c.direct) {
        // operands go straight to registers: no LDS stage (the 3 KiB where the
        // waves' partial blocks meet when they split K are not a stage)
        out->block_k = 32;
        out->stages = 0;
        out->mfma_m = 16;
        out->mfma_n = 16;
        out->mfma_k = c.eb == 4 ? 4 : 32;
        out->lds_bytes = 0;
        out->a_block_k = out->block_k;
        out->a_stages = out->stages;
        return TGEMM_OK;
    }
    out->block_k = ring ? c.ring_bk : c.bk;
    out->stages = ring ? c.ring_stages : 2;
    out->a_block_k = ring ? c.ring_a_bk : out->block_k;
    out->a_stages = ring ? c.ring_a_stages : out->stages;
    out->mfma_m = ring ? 16 : 32;
    out->mfma_n = ring ? 16 : 32;
    out->mfma_k = ring ? 32 : (c.eb == 4 ? 2 : 16);
    out->lds_bytes = ring ? c.ring_lds : c.lds_bytes;
    return TGEMM_OK;
}

int gemm_select_config(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb,
                       const void* C, int64_t ldc, int in_dtype, int out_dtype) {
    const Problem p{M, N, K, A, lda, LAYOUT_ROW, B, ldb, LAYOUT_ROW, (void*)C, ldc, in_dtype, out_dtype};
    const int v = validate(p);
    if (v != TGEMM_OK) return v;
    return table_choice(p);
}

int gemm_select_kernel(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb,
                       const void* C, int64_t ldc, int in_dtype, int out_dtype, int config_id) {
    return gemm_select_kernel_t(M, N, K, A, lda, TGEMM_ROW_MAJOR, B, ldb, TGEMM_ROW_MAJOR, C, ldc, TGEMM_ROW_MAJOR,
                                in_dtype, out_dtype, config_id, nullptr);
}

int gemm_select_kernel_t(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, int layout_a, const void* B,
                         int64_t ldb, int layout_b, const void* C, int64_t ldc, int layout_c, int in_dtype,
                         int out_dtype, int config_id, int* config_out) {
    Problem p;
    int v = make_problem(M, N, K, A, lda, layout_a, B, ldb, layout_b, (void*)C, ldc, layout_c, in_dtype, out_dtype, p);
    if (v != TGEMM_OK) return v;
    if (!elems_aligned(p)) return TGEMM_ERR_ALIGN;
    Plan plan;
    v = make_plan(p, config_id, plan);
    if (v != TGEMM_OK) return v;
    if (config_out != nullptr) *config_out = plan.config;
    return plan.kind;
}

int gemm_split_count_t(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, int layout_a, const void* B,
                       int64_t ldb, int layout_b, const void* C, int64_t ldc, int layout_c, int in_dtype,
                       int out_dtype) {
    Problem p;
    int v = make_problem(M, N, K, A, lda, layout_a, B, ldb, layout_b, (void*)C, ldc, layout_c, in_dtype, out_dtype, p);
    if (v != TGEMM_OK) return v;
    if (!elems_aligned(p)) return TGEMM_ERR_ALIGN;
    Plan plan;
    v = make_plan(p, -1, plan);
    if (v != TGEMM_OK) return v;
    return plan.splits;
}

int gemm_tile_map(int bid, int tiles_m, int tiles_n, int group_m, int* tm, int* tn) {
    if (tiles_m <= 0 || tiles_n <= 0 || group_m <= 0 || bid < 0 || bid >= tiles_m * tiles_n || !tm || !tn)
        return TGEMM_ERR_DIM;
    tile_of(bid, tiles_m, tiles_n, group_m, *tm, *tn);
    return TGEMM_OK;
}

const char* gemm_version(void) { return "tgemm 0.2 gfx950"; }

}  // extern "C"
