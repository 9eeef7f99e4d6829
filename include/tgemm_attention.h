/*
 * tgemm_attention.h -- attention forward of libtgemm.so.
 *
 * The operation is the attention of page "TileLang实战：用Python DSL自动生成
 * 高性能GPU计算内核", §4.1: O = softmax(Q K^T) V, here with a score scale,
 * O = softmax(scale Q K^T) V, for every (batch, head), computed the way its
 * §4.2 computes it: K and V are walked in blocks and every query keeps a
 * running maximum M and normaliser L of its scores (the online softmax), so
 * that the Nq x Nk score matrix never exists in memory.  Both products run
 * on the matrix cores with fp32 accumulation; the softmax is fp32; the
 * probabilities are rounded to the input type before the second product.
 *
 * Shares the element types, return-code scheme and gemm_strerror() of tgemm.h.
 */
#ifndef TGEMM_ATTENTION_H
#define TGEMM_ATTENTION_H

#include "tgemm.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * attention_fwd: O := softmax(scale Q K^T [+ causal mask]) V.
 *   batch, heads      B, H >= 0 (each at most 65535)
 *   n_q, n_k          query and key counts, 0 <= n_q, n_k <= TGEMM_MAX_DIM;
 *                     n_k >= 1 whenever there is a query (a softmax over no
 *                     key is undefined: TGEMM_ERR_DIM)
 *   head_dim          d, 64 or 128 (else TGEMM_ERR_HEAD_DIM)
 *   Q, K, V           device inputs of type in_dtype: Q is [B, H, n_q, d],
 *                     K and V are [B, H, n_k, d]; element (b, h, i, c) of X
 *                     at X[b * x_stride[0] + h * x_stride[1] + i * x_stride[2]
 *                     + c], strides in ELEMENTS, >= 0, the last dimension
 *                     contiguous.  A NULL stride pointer means the packed
 *                     layout {H n d, n d, d}.  The stride arrays are read on
 *                     the host during the call.  Elements need only be
 *                     aligned to their size (else TGEMM_ERR_ALIGN);
 *                     overlapping inputs are fine.
 *                     The row strides of K and V must keep 64 rows within
 *                     32-bit byte offsets: (64 max(k_stride[2], v_stride[2])
 *                     + d) * 2 < 2^31 (else TGEMM_ERR_LD).
 *   O                 device output [B, H, n_q, d] of type out_dtype, strides
 *                     as above; its elements must not overlap one another
 *                     (TGEMM_ERR_LD) nor Q, K or V (TGEMM_ERR_ALIAS).
 *   in_dtype          TGEMM_F16 or TGEMM_BF16; out_dtype: in_dtype or
 *                     TGEMM_F32 (else TGEMM_ERR_DTYPE)
 *   scale             factor of the scores (finite; 1 is the plain
 *                     softmax(Q K^T) V, 1/sqrt(d) the usual one)
 *   causal            nonzero: key j is hidden from query i when j > i (the
 *                     mask anchored at the top-left corner of the n_q x n_k
 *                     score matrix); every query still sees key 0
 *   stream            hipStream_t (NULL: the null stream)
 * One kernel is enqueued and the call returns without waiting.  Nothing is
 * allocated.  Invalid arguments are reported before anything is enqueued.
 * B H n_q == 0 does nothing and returns TGEMM_OK.
 */
int attention_fwd(int64_t batch, int64_t heads, int64_t n_q, int64_t n_k, int64_t head_dim,
                  const void* Q, const int64_t* q_stride,
                  const void* K, const int64_t* k_stride,
                  const void* V, const int64_t* v_stride,
                  void* O, const int64_t* o_stride,
                  int in_dtype, int out_dtype, float scale, int causal, void* stream);

/*
 * attention_waves: the query tile attention_fwd launches for these sizes, in
 * units of 32 rows: 4 (128 rows, four waves with 32 rows each) or, for
 * head_dim 64 when 128-row tiles would leave some of the 256 CUs without a
 * workgroup, 1 (32 rows, two waves splitting the keys and combining their
 * partial results).  TGEMM_ERR_DIM for sizes outside attention_fwd's range
 * or with nothing to compute, TGEMM_ERR_HEAD_DIM for a head_dim other than
 * 64 and 128.  Host-only; enqueues nothing.
 */
int attention_waves(int64_t batch, int64_t heads, int64_t n_q, int64_t head_dim);

#ifdef __cplusplus
}
#endif

#endif /* TGEMM_ATTENTION_H */
