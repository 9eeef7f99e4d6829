// attention.hip -- C ABI of the attention forward (include/tgemm_attention.h):
// argument checks, kernel choice and launch.  The kernel is in
// attention_kernel.hpp.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "attention_kernel.hpp"
#include "tgemm_attention.h"

using namespace tgemm;

namespace {

typedef void (*AttnFn)(AttnArgs);

template <int D, int IN, bool CAUSAL, int NW, bool SPLIT>
AttnFn attn_pick_out(int out) {
    if (out == DT_F32) return attention_kernel<D, IN, DT_F32, CAUSAL, NW, SPLIT>;
    return attention_kernel<D, IN, IN, CAUSAL, NW, SPLIT>;
}

template <int D, int NW, bool SPLIT>
AttnFn attn_pick_nw(int in, int out, bool causal) {
    if (in == DT_F16)
        return causal ? attn_pick_out<D, DT_F16, true, NW, SPLIT>(out) : attn_pick_out<D, DT_F16, false, NW, SPLIT>(out);
    return causal ? attn_pick_out<D, DT_BF16, true, NW, SPLIT>(out) : attn_pick_out<D, DT_BF16, false, NW, SPLIT>(out);
}

// The kernel for head dimension d and tile rows / 32 (4: four waves with 32
// rows each; 1: two waves splitting the keys of 32 rows), its threads and LDS.
constexpr int kSplitWaves = 2;
AttnFn attn_pick(int d, int row_waves, int in, int out, bool causal, int& threads, int& lds) {
    if (d == 128) {
        threads = 256;
        lds = attn_lds_bytes<128, 4, false>();
        return attn_pick_nw<128, 4, false>(in, out, causal);
    }
    if (row_waves == 4) {
        threads = 256;
        lds = attn_lds_bytes<64, 4, false>();
        return attn_pick_nw<64, 4, false>(in, out, causal);
    }
    threads = 64 * kSplitWaves;
    lds = attn_lds_bytes<64, kSplitWaves, true>();
    return attn_pick_nw<64, kSplitWaves, true>(in, out, causal);
}

int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Query rows per workgroup, in units of 32: 4 (four waves, 32 rows each)
// unless that leaves CUs idle (fewer workgroups than the 256 CUs) with head
// dimension 64, then 1 (32 rows, two waves splitting the keys: half the
// chain of dependent key blocks per wave).  Head dimension 128 always 4: its
// registers leave no room for the split's second ring beside two workgroups
// per CU.
int waves_for(int64_t batch, int64_t heads, int64_t n_q, int64_t d) {
    if (d == 128) return 4;
    return batch * heads * ceil_div64(n_q, 128) >= 256 ? 4 : 1;
}

struct Tensor4 {
    const void* p;
    int64_t s[3];  // batch, head, row strides (elements); the last dimension is contiguous
};

// Strides of a [B, H, n, d] operand: the given ones or the packed layout.
bool strides_of(const int64_t* given, int64_t H, int64_t n, int64_t d, int64_t out[3]) {
    if (given == nullptr) {
        out[0] = H * n * d;
        out[1] = n * d;
        out[2] = d;
        return true;
    }
    for (int i = 0; i < 3; ++i) {
        if (given[i] < 0 || given[i] > ((int64_t)1 << 40)) return false;
        out[i] = given[i];
    }
    return true;
}

// [first, last] byte range touched by a [B, H, n, d] operand (all sizes > 0).
void byte_range(const Tensor4& t, int64_t B, int64_t H, int64_t n, int64_t d, int eb, uintptr_t& lo,
                uintptr_t& hi) {
    const int64_t last = (B - 1) * t.s[0] + (H - 1) * t.s[1] + (n - 1) * t.s[2] + (d - 1);
    lo = (uintptr_t)t.p;
    hi = (uintptr_t)t.p + (uintptr_t)(last + 1) * eb;
}

// No two elements of the output coincide: ordered by stride, every dimension
// of extent > 1 steps over everything the smaller ones span.
bool non_overlapping(const int64_t s[3], int64_t B, int64_t H, int64_t n, int64_t d) {
    int64_t st[4] = {1, s[2], s[1], s[0]};
    int64_t ex[4] = {d, n, H, B};
    // insertion sort by stride (ties keep the inner dimension first)
    for (int i = 1; i < 4; ++i)
        for (int j = i; j > 0 && st[j] < st[j - 1]; --j) {
            int64_t t = st[j]; st[j] = st[j - 1]; st[j - 1] = t;
            t = ex[j]; ex[j] = ex[j - 1]; ex[j - 1] = t;
        }
    int64_t span = 1;  // elements spanned by the dimensions so far, as an extent
    for (int i = 0; i < 4; ++i) {
        if (ex[i] <= 1) continue;
        if (st[i] < span) return false;
        span = st[i] * (ex[i] - 1) + span;
    }
    return true;
}

}  // namespace

extern "C" {

int attention_fwd(int64_t batch, int64_t heads, int64_t n_q, int64_t n_k, int64_t head_dim, const void* Q,
                  const int64_t* q_stride, const void* K, const int64_t* k_stride, const void* V,
                  const int64_t* v_stride, void* O, const int64_t* o_stride, int in_dtype, int out_dtype,
                  float scale, int causal, void* stream) {
    if (batch < 0 || heads < 0 || n_q < 0 || n_k < 0 || batch > 65535 || heads > 65535 || n_q > TGEMM_MAX_DIM ||
        n_k > TGEMM_MAX_DIM)
        return TGEMM_ERR_DIM;
    if (head_dim != 64 && head_dim != 128) return TGEMM_ERR_HEAD_DIM;
    if (in_dtype != TGEMM_F16 && in_dtype != TGEMM_BF16) return TGEMM_ERR_DTYPE;
    if (out_dtype != in_dtype && out_dtype != TGEMM_F32) return TGEMM_ERR_DTYPE;
    if (!isfinite(scale)) return TGEMM_ERR_DIM;
    if (batch == 0 || heads == 0 || n_q == 0) return TGEMM_OK;
    if (n_k == 0) return TGEMM_ERR_DIM;
    const int64_t d = head_dim;
    Tensor4 q{Q, {}}, k{K, {}}, v{V, {}}, o{O, {}};
    if (!strides_of(q_stride, heads, n_q, d, q.s) || !strides_of(k_stride, heads, n_k, d, k.s) ||
        !strides_of(v_stride, heads, n_k, d, v.s) || !strides_of(o_stride, heads, n_q, d, o.s))
        return TGEMM_ERR_LD;
    // the kernel addresses the 64 rows of a key block from the block's first
    // row with 32-bit byte offsets
    if ((64 * (k.s[2] > v.s[2] ? k.s[2] : v.s[2]) + d) * 2 >= ((int64_t)1 << 31)) return TGEMM_ERR_LD;
    if (Q == nullptr || K == nullptr || V == nullptr || O == nullptr) return TGEMM_ERR_NULL;
    const int ob = out_dtype == TGEMM_F32 ? 4 : 2;
    if ((uintptr_t)Q % 2 != 0 || (uintptr_t)K % 2 != 0 || (uintptr_t)V % 2 != 0 || (uintptr_t)O % ob != 0)
        return TGEMM_ERR_ALIGN;
    if (!non_overlapping(o.s, batch, heads, n_q, d)) return TGEMM_ERR_LD;
    uintptr_t o0, o1;
    byte_range(o, batch, heads, n_q, d, ob, o0, o1);
    const Tensor4* ins[3] = {&q, &k, &v};
    const int64_t ns[3] = {n_q, n_k, n_k};
    for (int i = 0; i < 3; ++i) {
        uintptr_t a0, a1;
        byte_range(*ins[i], batch, heads, ns[i], d, 2, a0, a1);
        if (o0 < a1 && a0 < o1) return TGEMM_ERR_ALIAS;
    }

    AttnArgs a;
    a.Q = (const char*)Q;
    a.K = (const char*)K;
    a.V = (const char*)V;
    a.O = (char*)O;
    a.q_sb = q.s[0]; a.q_sh = q.s[1]; a.q_sn = q.s[2];
    a.k_sb = k.s[0]; a.k_sh = k.s[1]; a.k_sn = k.s[2];
    a.v_sb = v.s[0]; a.v_sh = v.s[1]; a.v_sn = v.s[2];
    a.o_sb = o.s[0]; a.o_sh = o.s[1]; a.o_sn = o.s[2];
    a.Nq = (int)n_q;
    a.Nk = (int)n_k;
    a.H = (int)heads;
    const int nw = waves_for(batch, heads, n_q, d);
    const int64_t bq = 32 * nw;
    const int64_t tiles = (n_q + bq - 1) / bq;
    if (batch * heads * tiles >= ((int64_t)1 << 24)) return TGEMM_ERR_DIM;  // grid limit
    a.tiles = (int)tiles;
    a.total = (int)(batch * heads * tiles);
    a.c = fabsf(scale) * 1.4426950408889634f;
    a.qsign = scale < 0.f ? 0x80008000u : 0u;
    const int in = in_dtype == TGEMM_F16 ? DT_F16 : DT_BF16;
    const int out = out_dtype == TGEMM_F32 ? DT_F32 : in;
    int lds = 0, threads = 0;
    const AttnFn fn = attn_pick((int)d, nw, in, out, causal != 0, threads, lds);
    hipLaunchKernelGGL(fn, dim3((unsigned)a.total), dim3(threads), (unsigned)lds, (hipStream_t)stream, a);
    return (int)hipGetLastError();
}

int attention_waves(int64_t batch, int64_t heads, int64_t n_q, int64_t head_dim) {
    if (batch <= 0 || heads <= 0 || n_q <= 0 || batch > 65535 || heads > 65535 || n_q > TGEMM_MAX_DIM)
        return TGEMM_ERR_DIM;
    if (head_dim != 64 && head_dim != 128) return TGEMM_ERR_HEAD_DIM;
    return waves_for(batch, heads, n_q, head_dim);
}

}  // extern "C"
