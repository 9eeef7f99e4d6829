/*
 * tgemm.h -- C ABI of the MI355X (gfx950) tiled dense matrix product library
 * libtgemm.so.
 *
 * The operation is the tiled matrix product of page "企业官网建设流程全解析"
 * (a TileLang article despite its title), §3.3: C = A x B with A of size
 * M x K, B of size K x N and C of size M x N; each workgroup owns one output
 * tile, walks K in steps, stages tiles of A and B in on-chip shared memory
 * (LDS here) through a multi-stage software pipeline (§2.3, §4.2 of that
 * page) and accumulates in an fp32 register fragment, which is converted to
 * the output type when it is written back.  Inputs are fp16 (or bf16, or
 * fp32), accumulation is always fp32, as in that page's listing
 * (dtype="float16", accum_dtype="float32").
 *
 * Conventions shared by every entry point:
 *  - All matrices are ROW-MAJOR, the default layout of page "TileLang实战：
 *    用Python DSL自动生成高性能GPU计算内核", §5.1.  Leading dimensions are in
 *    ELEMENTS: A is M x K with lda >= K, B is K x N with ldb >= N, C is M x N
 *    with ldc >= N.  Element (i, j) of A is A[i * lda + j].
 *  - C := A x B.  C is overwritten; there is no alpha/beta.  Elements of C
 *    outside the M x N window (columns N .. ldc-1) are never written.
 *  - A, B and C are DEVICE pointers (memory of the current HIP device), owned
 *    by the caller; the library keeps no reference after the call.  C must
 *    not overlap A or B.  Each pointer is aligned to its element's size
 *    (TGEMM_ERR_ALIGN otherwise); no other alignment is needed: leading
 *    dimensions and base offsets may be any number of elements.
 *  - The call enqueues one kernel on `stream` (a hipStream_t; NULL = the
 *    null stream) and returns without waiting for it.  The library allocates
 *    no memory and keeps no per-call state; concurrent calls are safe.
 *  - K == 0 writes zeros (the empty sum).  M == 0 or N == 0 does nothing and
 *    returns TGEMM_OK.
 *  - Return codes: TGEMM_OK (0); a negative TGEMM_ERR_* for invalid arguments,
 *    detected before anything is enqueued (no side effect); a positive value
 *    is the hipError_t reported by the kernel launch.  gemm_strerror() names
 *    every code.
 */
#ifndef TGEMM_H
#define TGEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types. */
#define TGEMM_F32 0  /* IEEE binary32 */
#define TGEMM_F16 1  /* IEEE binary16 */
#define TGEMM_BF16 2 /* bfloat16 (upper half of a binary32) */
/* 8-bit floating-point outputs (OCP 8-bit floating point formats; output
 * types only):
 *   E4M3: 1 sign, 4 exponent (bias 7), 3 fraction bits; no infinity,
 *         S.1111.111 is NaN; largest finite value 448.
 *   E5M2: 1 sign, 5 exponent (bias 15), 2 fraction bits; IEEE-like
 *         infinities and NaNs; largest finite value 57344.
 * One byte per element; torch's float8_e4m3fn and float8_e5m2 hold the same
 * formats. */
#define TGEMM_FP8_E4M3 3
#define TGEMM_FP8_E5M2 4

/* Supported (in_dtype -> out_dtype) pairs:
 *   F32 -> F32, F16 -> F16, F16 -> F32, BF16 -> BF16, BF16 -> F32,
 *   F16 or BF16 -> FP8_E4M3 or FP8_E5M2.
 * Conversion of the fp32 accumulator to F16 / BF16 rounds to nearest, ties to
 * even; values beyond the output range become +-Inf.  Conversion to an 8-bit
 * format rounds to nearest, ties to even, and saturates: magnitudes beyond
 * the largest finite value, infinities included, become the largest finite
 * value of their sign; NaN stays NaN (the all-ones pattern).  8-bit outputs
 * are written by the fused epilogue's kernels (ring configurations where
 * they apply, the direct kernel otherwise; TGEMM_ERR_DIM where neither
 * does), with the identity epilogue when none is given. */

/* Error codes. */
#define TGEMM_OK 0
#define TGEMM_ERR_DIM (-1)         /* M, N or K negative, or above TGEMM_MAX_DIM */
#define TGEMM_ERR_NULL (-2)        /* NULL pointer for a non-empty operand       */
#define TGEMM_ERR_LD (-3)          /* lda < K, ldb < N or ldc < N                */
#define TGEMM_ERR_DTYPE (-4)       /* unsupported (in_dtype, out_dtype) pair     */
#define TGEMM_ERR_ALIAS (-5)       /* C overlaps A, B or the epilogue's bias     */
#define TGEMM_ERR_CONFIG (-6)      /* gemm_ex / gemm_t: unknown config, wrong
                                      dtype, or a config without a kernel for
                                      column-major operands                  */
#define TGEMM_ERR_LAYOUT (-7)      /* gemm_t: layout not ROW_MAJOR / COL_MAJOR  */
#define TGEMM_ERR_EPILOGUE (-8)    /* gemm_fused: bad activation, bias kind or
                                      bias type, or a bias kind without bias  */
#define TGEMM_ERR_HEAD_DIM (-9)    /* attention_fwd: head_dim not 64 or 128     */
#define TGEMM_ERR_SCRATCH (-10)    /* gemm_fused_noalloc: the call's split-K
                                      workspace exceeds the fixed scratch  */
#define TGEMM_ERR_ALIGN (-11)      /* a pointer not aligned to its element's
                                      size: 2 bytes for F16 / BF16, 4 for F32
                                      (A, B, C, the epilogue's bias;
                                      attention's Q, K, V, O); 8-bit outputs
                                      may start at any byte               */

/* Operand layouts (gemm_t): the row-major default and the column-major option
 * of page "TileLang实战：用Python DSL自动生成高性能GPU计算内核", §5.1. */
#define TGEMM_ROW_MAJOR 0 /* element (i, j) of X at X[i * ld + j] */
#define TGEMM_COL_MAJOR 1 /* element (i, j) of X at X[j * ld + i] */

/* Largest M, N or K accepted (tile indices are 32-bit; element offsets are
 * 64-bit, so matrices may exceed 4 GiB). */
#define TGEMM_MAX_DIM (1LL << 30)

/*
 * gemm: C := A x B (see the conventions above).
 *   M, N, K              sizes; A: M x K, B: K x N, C: M x N
 *   A, lda / B, ldb      device inputs of type in_dtype, leading dims in elements
 *   C, ldc               device output of type out_dtype, leading dim in elements
 *   in_dtype, out_dtype  TGEMM_F32 / TGEMM_F16 / TGEMM_BF16
 *   stream               hipStream_t to enqueue on (NULL: null stream)
 * The tile configuration comes from a per-shape table keyed on the element
 * types, the sizes and the 16-byte alignment of pointers and leading
 * dimensions (gemm_select_config).
 */
int gemm(int64_t M, int64_t N, int64_t K,
         const void* A, int64_t lda, const void* B, int64_t ldb,
         void* C, int64_t ldc, int in_dtype, int out_dtype, void* stream);

/*
 * gemm_ex: as gemm, but forces tile configuration `config_id` (0 ..
 * gemm_num_configs()-1) instead of the table's choice; -1 means "the table's
 * choice".  Any configuration gives a correct result for any shape, layout
 * and alignment of its input type; it is meant for measuring one
 * configuration against another (the tuning method of page
 * "企业官网建设流程全解析", §4.4).  Returns TGEMM_ERR_CONFIG if the id is
 * unknown or the configuration is for another input type.
 */
int gemm_ex(int64_t M, int64_t N, int64_t K,
            const void* A, int64_t lda, const void* B, int64_t ldb,
            void* C, int64_t ldc, int in_dtype, int out_dtype, void* stream,
            int config_id);

/*
 * gemm_t: C := A x B with a layout per matrix (TGEMM_ROW_MAJOR or
 * TGEMM_COL_MAJOR).  A is logically M x K, B K x N, C M x N; a column-major
 * X stores its transpose row by row, so lda >= K for a row-major A and
 * lda >= M for a column-major one (ldb >= N or K, ldc >= N or M likewise).
 * gemm(...) is gemm_t(..., ROW_MAJOR, ..., ROW_MAJOR, ..., ROW_MAJOR, ..., -1).
 * A column-major C is computed as the row-major C^T = B^T x A^T.  Kernels:
 * row-major A and B take every configuration; with a column-major operand
 * the direct-to-LDS ring kernels of configurations 0 and 1 (8 with a
 * row-major A; its other products run configuration 1) and the direct
 * kernels of configurations 6 and 7 (configurations 2 to 5 and 9 return
 * TGEMM_ERR_CONFIG there, and products whose 32-bit buffer offsets would
 * overflow return TGEMM_ERR_DIM).  config_id -1:
 * the table's choice.  Other arguments, ownership and errors as gemm_ex.
 */
int gemm_t(int64_t M, int64_t N, int64_t K,
           const void* A, int64_t lda, int layout_a,
           const void* B, int64_t ldb, int layout_b,
           void* C, int64_t ldc, int layout_c,
           int in_dtype, int out_dtype, void* stream, int config_id);

/*
 * The fused epilogue (gemm_fused): further operators merged into the
 * product's kernel, so that the product makes no round trip through memory
 * (the operator fusion of page "企业官网建设流程全解析", §6.2).  The page names
 * no operator; these are the usual ones after a matrix product:
 *
 *   C := act(alpha * (A x B) + beta * C + bias)
 *
 * evaluated in fp32 on the fp32 accumulator, then rounded to the output type
 * (nearest even; saturating for the 8-bit formats).  beta == 0: C is not read
 * (it may hold anything, NaN included); otherwise C is read in the output
 * type, an 8-bit C too.  bias: one value per row of C (bias_kind TGEMM_BIAS_ROW, M
 * values) or per column (TGEMM_BIAS_COL, N values, the bias of a linear
 * layer), contiguous, of type bias_dtype (TGEMM_F32 / F16 / BF16), device
 * memory owned by the caller, not overlapping C.  Activations:
 *   TGEMM_ACT_RELU       max(x, 0)
 *   TGEMM_ACT_GELU       x * Phi(x) = x/2 (1 + erf(x / sqrt 2))
 *   TGEMM_ACT_GELU_TANH  x/2 (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3)))
 *   TGEMM_ACT_SILU       x / (1 + exp(-x))
 */
#define TGEMM_ACT_NONE 0
#define TGEMM_ACT_RELU 1
#define TGEMM_ACT_GELU 2
#define TGEMM_ACT_GELU_TANH 3
#define TGEMM_ACT_SILU 4
#define TGEMM_BIAS_NONE 0
#define TGEMM_BIAS_ROW 1
#define TGEMM_BIAS_COL 2

typedef struct tgemm_epilogue {
    float alpha;       /* scales A x B (1 for the plain product)        */
    float beta;        /* scales the previous C (0: C not read)         */
    const void* bias;  /* device vector, or NULL with TGEMM_BIAS_NONE   */
    int bias_kind;     /* TGEMM_BIAS_NONE / ROW / COL                   */
    int bias_dtype;    /* TGEMM_F32 / F16 / BF16                        */
    int activation;    /* TGEMM_ACT_*                                   */
} tgemm_epilogue;

/*
 * gemm_fused: gemm_t with the fused epilogue *epilogue (NULL: exactly
 * gemm_t).  The same kernels, tile table and layouts as gemm_t; with a
 * column-major C the bias kinds keep their meaning for C.  Errors as gemm_t,
 * plus TGEMM_ERR_EPILOGUE for bad epilogue arguments and TGEMM_ERR_ALIAS if
 * the bias overlaps C.  M == 0 or N == 0: nothing is read or written;
 * K == 0: C := act(beta * C + bias).
 */
int gemm_fused(int64_t M, int64_t N, int64_t K,
               const void* A, int64_t lda, int layout_a,
               const void* B, int64_t ldb, int layout_b,
               void* C, int64_t ldc, int layout_c,
               int in_dtype, int out_dtype, const tgemm_epilogue* epilogue, void* stream, int config_id);

/*
 * gemm_fused_noalloc: gemm_fused for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  The same plan, kernels and results as gemm_fused with
 * the same arguments, except that a split-K plan (TGEMM_KERNEL_RING_SPLITK)
 * keeps its fp32 partials in the library's own fixed device array of 32 MiB
 * (one per GPU, held until the process ends) rather than in the stream's
 * workspace from the library's pool: the call allocates, frees and records
 * nothing.  Every call on a GPU
 * uses that GPU's one array, so calls that overlap on one GPU (on different
 * streams, or concurrently from several host threads) race; calls on one
 * stream are ordered and safe.  The array keeps the last call's contents
 * (nothing in it needs to start at zero).  Errors as gemm_fused, plus
 * TGEMM_ERR_SCRATCH if the call's workspace would exceed 32 MiB (no split
 * plan of the library's table does: at most 512 partial tiles of 128 x 128).
 */
int gemm_fused_noalloc(int64_t M, int64_t N, int64_t K,
                       const void* A, int64_t lda, int layout_a,
                       const void* B, int64_t ldb, int layout_b,
                       void* C, int64_t ldc, int layout_c,
                       int in_dtype, int out_dtype,
                       const tgemm_epilogue* epilogue, void* stream, int config_id);

/* Human-readable text for a return code of gemm / gemm_ex / gemm_t /
 * gemm_fused (never NULL; the string is static). */
const char* gemm_strerror(int code);

/* Number of tile configurations in the table. */
int gemm_num_configs(void);

/* Description of one tile configuration (the tile-config tuple of page
 * "企业官网建设流程全解析", §3.3: block_M, block_N, block_K, num_stages,
 * threads, plus the gfx950 specifics). */
typedef struct tgemm_config_info {
    int id;
    int in_dtype;       /* TGEMM_F16 configurations also serve TGEMM_BF16 */
    int block_m, block_n, block_k;
    int stages;         /* LDS buffers in the software pipeline (0: none) */
    int threads;        /* workitems per workgroup (64 per wavefront)      */
    int waves_m, waves_n;
    int mfma_m, mfma_n, mfma_k; /* shape of one MFMA instruction           */
    int lds_bytes;      /* LDS per workgroup                               */
    const char* name;   /* static string                                   */
    /* The ring of a row-major A when it differs from B's (block_k, stages):
     * the direct-to-LDS ring kernel stages row-major A in 2 stages of 64 of
     * K, so that every load reads whole 128-byte lines.  Otherwise equal to
     * block_k and stages.  lds_bytes = (a_stages * a_block_k * block_m +
     * stages * block_k * block_n) * element bytes. */
    int a_block_k, a_stages;
} tgemm_config_info;

/* Fills *out for config `id`; returns TGEMM_OK or TGEMM_ERR_CONFIG. */
int gemm_config_info(int id, tgemm_config_info* out);

/* Host-side table lookup only (no GPU call): the configuration id that gemm()
 * would use for these arguments, or a negative TGEMM_ERR_* if gemm() would
 * reject them.  Pointers are only inspected for their alignment. */
int gemm_select_config(int64_t M, int64_t N, int64_t K,
                       const void* A, int64_t lda, const void* B, int64_t ldb,
                       const void* C, int64_t ldc, int in_dtype, int out_dtype);

/* Kernels a call can run (gemm_select_kernel). */
#define TGEMM_KERNEL_GENERAL 0 /* register-staged, every access checked (ragged or unaligned) */
#define TGEMM_KERNEL_TILED 1   /* register-staged, whole tiles, aligned operands              */
#define TGEMM_KERNEL_RING 2    /* direct-to-LDS rings: 16-bit inputs, any M, N, K, layout and
                                  leading dimension (configurations 0, 1 and 8)             */
#define TGEMM_KERNEL_DIRECT 3  /* operands straight from memory to registers, no LDS stage:
                                  small, ragged or unaligned products (configurations 6 and
                                  7)                                                        */
#define TGEMM_KERNEL_RING_SPLITK 4 /* the ring kernel over slices of K (products with too few
                                  output tiles for the CUs and a long K: configuration 8, or
                                  1 for column-major operands), each slice's fp32 partial in
                                  a workspace, then a second kernel that sums the slices in
                                  a fixed order and applies the epilogue; the workspace
                                  (slices x M x N rounded up to 4, fp32) is the stream's own,
                                  kept between calls for the last 8 streams of each device
                                  (from the library's memory pool, held until the process
                                  ends; a call waits on an event of the workspace's previous
                                  call, and calls from several host threads are serialised
                                  around its two launches).  Under stream capture use
                                  gemm_fused_noalloc.  Only the table's choice (config_id -1)
                                  splits; TGEMM_NO_SPLITK=1 in the environment turns it off */

/* Host-side lookup only (no GPU call): which kernel gemm_ex(..., config_id)
 * would launch for these arguments (config_id -1: the table's choice), as a
 * TGEMM_KERNEL_* value, or a negative TGEMM_ERR_* if the call would be
 * rejected.  All kernels of a configuration compute the same tile; this
 * exists so that tests and measurements can tell which one ran.  Pointers
 * are only inspected for their alignment. */
int gemm_select_kernel(int64_t M, int64_t N, int64_t K,
                       const void* A, int64_t lda, const void* B, int64_t ldb,
                       const void* C, int64_t ldc, int in_dtype, int out_dtype, int config_id);

/* gemm_select_kernel for gemm_t's arguments; also stores the configuration
 * that would run in *config_out (if not NULL).  Host-side lookup only. */
int gemm_select_kernel_t(int64_t M, int64_t N, int64_t K,
                         const void* A, int64_t lda, int layout_a,
                         const void* B, int64_t ldb, int layout_b,
                         const void* C, int64_t ldc, int layout_c,
                         int in_dtype, int out_dtype, int config_id, int* config_out);

/* Host-side lookup only (no GPU call): the number of K slices gemm_t with
 * these arguments and the table's choice would run (1: none; see
 * TGEMM_KERNEL_RING_SPLITK), or a negative TGEMM_ERR_* if the call would be
 * rejected. */
int gemm_split_count_t(int64_t M, int64_t N, int64_t K,
                       const void* A, int64_t lda, int layout_a,
                       const void* B, int64_t ldb, int layout_b,
                       const void* C, int64_t ldc, int layout_c,
                       int in_dtype, int out_dtype);

/* Host-side copy of the workgroup -> output-tile map the kernels use (no GPU
 * call), for checking that it is a bijection: workgroup `bid` of a grid of
 * tiles_m x tiles_n tiles, raster groups of `group_m` tile rows, computes
 * tile (*tm, *tn).  Returns TGEMM_OK, or TGEMM_ERR_DIM for out-of-range
 * arguments (nothing written). */
int gemm_tile_map(int bid, int tiles_m, int tiles_n, int group_m, int* tm, int* tn);

/* Library version string (static). */
const char* gemm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TGEMM_H */
