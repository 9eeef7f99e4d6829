/*
 * oracle_gemm.c -- reference implementation of the dense matrix product
 * C = A x B, used ONLY as test infrastructure.
 *
 * Who may use it: the test-suite (tests/), the smoke check in
 * __graft_entry__.smoke() and the "cpu_baseline" leg of bench.py.  The GPU
 * library never includes, links or calls this file, and this file includes
 * nothing from the GPU library: the two share no code, header, table or
 * constant.
 *
 * What it computes (the plain definition, written out):
 *   C[i][j] = sum_{k=0}^{K-1} a(i,k) * b(k,j)
 * where A is M x K, B is K x N and C is M x N, all row-major.  This is the
 * product that the tiled kernel of page "企业官网建设流程全解析" (a TileLang
 * article despite its title), §3.3, is written to compute, with A of size
 * M x K, B of size K x N and C of size M x N, and the triple loop of page
 * "TileLang实战：用Python DSL自动生成高性能GPU计算内核", §3.1.  The
 * page about the DeepSeek/Ascend TileLang toolkit, §3.3 (first step of its
 * verification procedure), asks for exactly this: a naive CPU implementation
 * that only aims at being right, used as ground truth.
 *
 * Precision: a(i,k) and b(k,j) are the EXACT values of the stored binary16,
 * bfloat16 or binary32 inputs, widened to binary64 by the decoders below,
 * which are written from the bit-level definitions of those formats (IEEE
 * 754-2008 binary16/binary32; bfloat16 = the upper 16 bits of a binary32).
 * Every product of two such values is exact in binary64 (at most 22 or 48
 * significant bits), so the only rounding is that of the binary64 running
 * sum, taken in increasing k.  The result is returned in binary64.
 *
 * Steps, in order:
 *   1. decode the requested rows of A and columns of B to binary64;
 *   2. for every requested (i, j): s = 0; for k = 0 .. K-1: s += a*b;
 *   3. store s.
 * K == 0 gives s = 0 (the empty sum).  Rows and columns may be a subset
 * (the "sampled" mode used at large sizes); the value of an entry does not
 * depend on which other entries are requested.
 *
 * Threads: output rows are dealt round-robin to plain POSIX threads; each
 * entry is still summed by one thread in increasing k, so the result does not
 * depend on the thread count.
 *
 * Build: gcc -O2 -ffp-contract=off -fPIC -shared -pthread (see build.py).
 * -ffp-contract=off keeps "s += a*b" a separate multiply and add; since the
 * product is exact it makes no numerical difference, but it keeps the code
 * literally what it says.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Element type codes understood by this file (its own numbering). */
#define ORACLE_BINARY32 0
#define ORACLE_BINARY16 1
#define ORACLE_BFLOAT16 2

/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 *   e == 0      : (-1)^s * f * 2^-24            (zero and subnormals)
 *   e == 31     : infinity (f == 0) or NaN
 *   otherwise   : (-1)^s * (1024 + f) * 2^(e-25) */
double oracle_decode_binary16(uint16_t h) {
    int s = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);
    return s ? -v : v;
}

/* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits.
 *   e == 0      : (-1)^s * f * 2^-133           (zero and subnormals)
 *   e == 255    : infinity (f == 0) or NaN
 *   otherwise   : (-1)^s * (128 + f) * 2^(e-134) */
double oracle_decode_bfloat16(uint16_t h) {
    int s = (h >> 15) & 1;
    int e = (h >> 7) & 0xff;
    int f = h & 0x7f;
    double v;
    if (e == 0)
        v = ldexp((double)f, -133);
    else if (e == 255)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(128 + f), e - 134);
    return s ? -v : v;
}

/* binary32: 1 sign bit, 8 exponent bits (bias 127), 23 fraction bits.
 *   e == 0      : (-1)^s * f * 2^-149
 *   e == 255    : infinity or NaN
 *   otherwise   : (-1)^s * (2^23 + f) * 2^(e-150) */
double oracle_decode_binary32(uint32_t w) {
    int s = (int)((w >> 31) & 1u);
    int e = (int)((w >> 23) & 0xffu);
    uint32_t f = w & 0x7fffffu;
    double v;
    if (e == 0)
        v = ldexp((double)f, -149);
    else if (e == 255)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(8388608u + f), e - 150);
    return s ? -v : v;
}

/*
 * 8-bit floating-point formats of the OCP specification, the output types of
 * the fused epilogue (their own codes in this file):
 *   E4M3: 1 sign bit, 4 exponent bits (bias 7), 3 fraction bits.  No
 *         infinity: S.1111.111 is NaN, so the largest finite value is
 *         S.1111.110 = 1.75 * 2^8 = 448.
 *   E5M2: 1 sign bit, 5 exponent bits (bias 15), 2 fraction bits, laid out
 *         like IEEE: e == 31 is infinity (f == 0) or NaN; the largest finite
 *         value is 1.75 * 2^15 = 57344.
 * With F fraction bits and bias b:
 *   e == 0      : (-1)^s * f * 2^(1-b-F)          (zero and subnormals)
 *   otherwise   : (-1)^s * (2^F + f) * 2^(e-b-F)
 */
#define ORACLE_FP8_E4M3 3
#define ORACLE_FP8_E5M2 4

double oracle_decode_fp8(uint8_t x, int fmt) {
    const int F = fmt == ORACLE_FP8_E4M3 ? 3 : 2;
    const int bias = fmt == ORACLE_FP8_E4M3 ? 7 : 15;
    const int emax = fmt == ORACLE_FP8_E4M3 ? 15 : 31;
    int s = (x >> 7) & 1;
    int e = (x >> F) & emax;
    int f = x & ((1 << F) - 1);
    double v;
    if (e == 0)
        v = ldexp((double)f, 1 - bias - F);
    else if (fmt == ORACLE_FP8_E4M3 && e == 15 && f == 7)
        v = NAN;
    else if (fmt == ORACLE_FP8_E5M2 && e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)((1 << F) + f), e - bias - F);
    return s ? -v : v;
}

/*
 * Rounding of a binary64 value to an 8-bit format, the conversion the fused
 * epilogue applies to its fp32 result: to the nearest representable value,
 * ties to the one with an even fraction; a magnitude beyond the largest
 * finite value, infinity included, becomes the largest finite value of the
 * same sign (the saturating conversion); NaN becomes the all-ones pattern
 * with the input's sign.  Returns the 8-bit pattern.
 *
 * Steps: the representable values in [2^E, 2^(E+1)) (E >= 1-b) are the
 * multiples of 2^(E-F); below 2^(1-b) they are the multiples of the
 * subnormal spacing 2^(1-b-F).  |x| divided by that spacing is exact; its
 * nearest integer (ties to even: rint in the default rounding mode) times the
 * spacing is the rounded magnitude (at most the largest finite value, to
 * which larger magnitudes were clamped first), which is then encoded.
 */
uint8_t oracle_encode_fp8(double x, int fmt) {
    const int F = fmt == ORACLE_FP8_E4M3 ? 3 : 2;
    const int bias = fmt == ORACLE_FP8_E4M3 ? 7 : 15;
    const double maxfin = fmt == ORACLE_FP8_E4M3 ? 448.0 : 57344.0;
    const uint8_t s = signbit(x) ? 0x80 : 0;
    if (isnan(x)) return s | 0x7f;
    double a = fabs(x);
    if (a > maxfin) a = maxfin;          /* infinity included */
    if (a == 0.0) return s;
    int e2;
    frexp(a, &e2);                       /* a in [2^(e2-1), 2^e2) */
    int E = e2 - 1;
    if (E < 1 - bias) E = 1 - bias;      /* subnormal range: one spacing */
    const double q = ldexp(1.0, E - F);
    const double v = rint(a / q) * q;    /* <= maxfin: the rounding of a value <= maxfin */
    if (v < ldexp(1.0, 1 - bias))        /* zero or subnormal: the code is f */
        return s | (uint8_t)(v / ldexp(1.0, 1 - bias - F));
    frexp(v, &e2);
    E = e2 - 1;                          /* v in [2^E, 2^(E+1)) */
    const int f = (int)(v / ldexp(1.0, E - F)) - (1 << F);
    return s | (uint8_t)(((E + bias) << F) | f);
}

/* Rounds n binary64 values to an 8-bit format (oracle_encode_fp8). */
int oracle_encode_fp8_array(const double* src, int fmt, int64_t n, uint8_t* dst) {
    if ((fmt != ORACLE_FP8_E4M3 && fmt != ORACLE_FP8_E5M2) || n < 0) return -1;
    for (int64_t i = 0; i < n; ++i) dst[i] = oracle_encode_fp8(src[i], fmt);
    return 0;
}

static double decode_one(const void* base, int64_t idx, int dtype) {
    if (dtype == ORACLE_FP8_E4M3 || dtype == ORACLE_FP8_E5M2)
        return oracle_decode_fp8(((const uint8_t*)base)[idx], dtype);
    if (dtype == ORACLE_BINARY32) {
        uint32_t w;
        memcpy(&w, (const char*)base + idx * 4, 4);
        return oracle_decode_binary32(w);
    }
    uint16_t h;
    memcpy(&h, (const char*)base + idx * 2, 2);
    return dtype == ORACLE_BINARY16 ? oracle_decode_binary16(h) : oracle_decode_bfloat16(h);
}

/* Decode n consecutive stored elements of type dtype into binary64. */
int oracle_decode_array(const void* src, int dtype, int64_t n, double* dst) {
    if (dtype < ORACLE_BINARY32 || dtype > ORACLE_FP8_E5M2 || n < 0) return -1;
    for (int64_t i = 0; i < n; ++i) dst[i] = decode_one(src, i, dtype);
    return 0;
}

struct job {
    int64_t nrows, ncols, K;
    const double* Ad;   /* nrows x K, decoded rows of A            */
    const double* Bd;   /* K x ncols, decoded columns of B         */
    double* C;          /* nrows x ncols, leading dimension ldc    */
    int64_t ldc;
    int tid, nthreads;
};

/* Step 2 for the rows r = tid, tid + nthreads, ...: for each row, every
 * requested entry is the sum over k, in increasing k, of a(i,k)*b(k,j).  The
 * k loop is outermost inside a row so that B is walked row by row; each
 * entry still receives its K terms in increasing k. */
static void* run_rows(void* p) {
    struct job* jb = (struct job*)p;
    for (int64_t r = jb->tid; r < jb->nrows; r += jb->nthreads) {
        double* s = jb->C + r * jb->ldc;
        for (int64_t c = 0; c < jb->ncols; ++c) s[c] = 0.0;
        const double* arow = jb->Ad + r * jb->K;
        for (int64_t k = 0; k < jb->K; ++k) {
            const double a = arow[k];
            const double* brow = jb->Bd + k * jb->ncols;
            for (int64_t c = 0; c < jb->ncols; ++c) s[c] += a * brow[c];
        }
    }
    return NULL;
}

/*
 * oracle_gemm: C_out[r][c] = sum_k a(rows[r], k) * b(k, cols[c]) in binary64.
 *
 *   M, N, K      sizes of the product (A: M x K, B: K x N), all >= 0
 *   A, lda       row-major A, leading dimension lda >= K (in elements)
 *   B, ldb       row-major B, leading dimension ldb >= N (in elements)
 *   dtype        element type of A and B (0 binary32, 1 binary16, 2 bfloat16)
 *   rows, nrows  requested row indices of C (NULL: all M rows, nrows ignored)
 *   cols, ncols  requested column indices of C (NULL: all N columns)
 *   C_out, ldc   binary64 output, nrows x ncols, leading dimension ldc >= ncols
 *   nthreads     worker threads (<= 0 means 1)
 *
 * Returns 0, -1 for invalid arguments (nothing written), or -2 when the
 * host is out of memory (nothing written).
 */
int oracle_gemm(int64_t M, int64_t N, int64_t K,
                const void* A, int64_t lda, const void* B, int64_t ldb, int dtype,
                const int64_t* rows, int64_t nrows, const int64_t* cols, int64_t ncols,
                double* C_out, int64_t ldc, int nthreads) {
    if (M < 0 || N < 0 || K < 0) return -1;
    if (dtype < ORACLE_BINARY32 || dtype > ORACLE_BFLOAT16) return -1;
    if (lda < K || ldb < N) return -1;
    if (rows == NULL) nrows = M;
    if (cols == NULL) ncols = N;
    if (nrows < 0 || ncols < 0 || ldc < ncols) return -1;
    for (int64_t r = 0; rows && r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= M) return -1;
    for (int64_t c = 0; cols && c < ncols; ++c)
        if (cols[c] < 0 || cols[c] >= N) return -1;
    if (nrows == 0 || ncols == 0) return 0;
    if (nthreads <= 0) nthreads = 1;
    if (nthreads > nrows) nthreads = (int)nrows;

    /* Step 1: decode. */
    double* Ad = (double*)malloc(sizeof(double) * (size_t)(nrows * (K ? K : 1)));
    double* Bd = (double*)malloc(sizeof(double) * (size_t)((K ? K : 1) * ncols));
    if (!Ad || !Bd) {
        free(Ad);
        free(Bd);
        return -2;
    }
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t i = rows ? rows[r] : r;
        for (int64_t k = 0; k < K; ++k) Ad[r * K + k] = decode_one(A, i * lda + k, dtype);
    }
    for (int64_t k = 0; k < K; ++k)
        for (int64_t c = 0; c < ncols; ++c) {
            const int64_t j = cols ? cols[c] : c;
            Bd[k * ncols + c] = decode_one(B, k * ldb + j, dtype);
        }

    /* Steps 2 and 3. */
    struct job* jobs = (struct job*)calloc((size_t)nthreads, sizeof(struct job));
    pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
    char* started = (char*)calloc((size_t)nthreads, 1);
    int rc = 0;
    if (!jobs || !th || !started) {
        rc = -2;
    } else {
        for (int t = 0; t < nthreads; ++t)
            jobs[t] = (struct job){nrows, ncols, K, Ad, Bd, C_out, ldc, t, nthreads};
        for (int t = 1; t < nthreads; ++t)
            started[t] = pthread_create(&th[t], NULL, run_rows, &jobs[t]) == 0;
        run_rows(&jobs[0]);
        for (int t = 1; t < nthreads; ++t) {
            if (started[t])
                pthread_join(th[t], NULL);
            else
                run_rows(&jobs[t]); /* no thread could be started: do it here */
        }
    }
    free(started);
    free(jobs);
    free(th);
    free(Ad);
    free(Bd);
    return rc;
}

/*
 * The fused epilogue (the operator fusion of page "企业官网建设流程全解析",
 * §6.2: further operators merged into the product's kernel so that the
 * product never makes a round trip through memory).  The pages name no
 * operator; the ones computed here are the usual ones after a matrix
 * product, applied in this order:
 *
 *   D[i][j] = act( alpha * P[i][j] + beta * C_old[i][j] + bias )
 *
 * where P = A x B (oracle_gemm), C_old is the previous content of C (not
 * read at all when beta == 0, so that whatever C holds, NaN included, has no
 * effect), and bias is bias_col[j] (one value per output column, the bias of
 * a linear layer) or bias_row[i] (one per output row), or absent.
 *
 * Activations, in binary64 with the C library's erf, tanh and exp:
 *   0 none       act(x) = x
 *   1 relu       act(x) = x if x > 0, else 0
 *   2 gelu       act(x) = x * Phi(x) = x / 2 * (1 + erf(x / sqrt(2)))
 *                (Gaussian error linear unit, Phi the standard normal CDF)
 *   3 gelu_tanh  act(x) = x / 2 * (1 + tanh(sqrt(2 / pi) * (x + 0.044715 x^3)))
 *                (the tanh approximation of the same function)
 *   4 silu       act(x) = x / (1 + exp(-x))  (x times the logistic function)
 */
#define ORACLE_ACT_NONE 0
#define ORACLE_ACT_RELU 1
#define ORACLE_ACT_GELU 2
#define ORACLE_ACT_GELU_TANH 3
#define ORACLE_ACT_SILU 4

double oracle_activation(double x, int act) {
    switch (act) {
        case ORACLE_ACT_RELU: return x > 0.0 ? x : 0.0;
        case ORACLE_ACT_GELU: return 0.5 * x * (1.0 + erf(x / sqrt(2.0)));
        case ORACLE_ACT_GELU_TANH: {
            const double c = sqrt(2.0 / M_PI);
            return 0.5 * x * (1.0 + tanh(c * (x + 0.044715 * x * x * x)));
        }
        case ORACLE_ACT_SILU: return x / (1.0 + exp(-x));
        default: return x;
    }
}

/*
 * oracle_epilogue: out[r][c] = act(alpha * s[r][c] + beta * c_old[r][c] + bias)
 * for r < nr, c < nc, all binary64.
 *
 *   s, lds            product values (from oracle_gemm), leading dimension lds
 *   alpha, beta       scalars; beta == 0 means c_old is not read (may be NULL)
 *   c_old, ldco       previous values of the same entries of C
 *   bias_row, bias_col  bias per output row (nr values) or per output column
 *                     (nc values); at most one of them non-NULL
 *   act               activation code (0 .. 4 above)
 *   out, ldo          result
 * Returns 0, or -1 for invalid arguments (nothing written).
 */
int oracle_epilogue(int64_t nr, int64_t nc, const double* s, int64_t lds, double alpha, double beta,
                    const double* c_old, int64_t ldco, const double* bias_row, const double* bias_col, int act,
                    double* out, int64_t ldo) {
    if (nr < 0 || nc < 0 || lds < nc || ldo < nc) return -1;
    if (act < ORACLE_ACT_NONE || act > ORACLE_ACT_SILU) return -1;
    if (beta != 0.0 && (c_old == NULL || ldco < nc)) return -1;
    if (bias_row != NULL && bias_col != NULL) return -1;
    for (int64_t r = 0; r < nr; ++r)
        for (int64_t c = 0; c < nc; ++c) {
            double t = alpha * s[r * lds + c];
            if (beta != 0.0) t += beta * c_old[r * ldco + c];
            if (bias_row) t += bias_row[r];
            if (bias_col) t += bias_col[c];
            out[r * ldo + c] = oracle_activation(t, act);
        }
    return 0;
}
