"""Reference attention forward -- TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may use
it; the GPU library never imports it and it never imports the GPU library.

What it computes (the plain definition, written out): for every batch b and
head h, with Q the Nq x d, K the Nk x d and V the Nk x d matrices of that
head,

    S = scale * Q K^T                      (Nq x Nk scores)
    S[i, j] = -inf where the mask hides key j from query i
    P[i, j] = exp(S[i, j] - max_j S[i, :]) / sum_j exp(S[i, j] - max_j S[i, :])
    O = P V                                (Nq x d)

i.e. O = softmax(scale Q K^T) V, the attention that page "TileLang实战：用
Python DSL自动生成高性能GPU计算内核" §4.1 computes (softmax(QK^T)V; the page
has no scale, which is scale = 1 here) and that its §4.2 computes blockwise
with an online softmax.  The causal mask hides key j from query i when
j > i (the lower-left triangle of the Nq x Nk score matrix, as
torch.nn.functional.scaled_dot_product_attention's is_causal).

Precision: the inputs are the exact values of the stored binary16 / bfloat16 /
binary32 elements (the decoders of oracle_gemm.c), every step in binary64
with numpy.  Rows of Q can be sampled (rows=...), computing only those
rows of O; a row's value does not depend on which other rows are requested.
"""
import numpy as np

from . import decode


def _values(x, dtype):
    """binary64 values of a stored array of any shape."""
    return decode(np.ascontiguousarray(x), dtype)


def attention(q, k, v, dtype, scale=1.0, causal=False, rows=None):
    """O = softmax(scale Q K^T) V per (batch, head), binary64.

    q: [B, H, Nq, d], k and v: [B, H, Nk, d] stored arrays (float16 /
    float32, or uint16 bfloat16 bits).  rows: query indices to compute (None:
    all Nq).  Returns a [B, H, len(rows), d] binary64 array."""
    Q, K, V = _values(q, dtype), _values(k, dtype), _values(v, dtype)
    if Q.ndim != 4 or K.shape != V.shape or Q.shape[:2] != K.shape[:2] or Q.shape[3] != K.shape[3]:
        raise ValueError(f"shapes {q.shape}, {k.shape}, {v.shape}")
    Nq, Nk = Q.shape[2], K.shape[2]
    ri = np.arange(Nq) if rows is None else np.asarray(rows, dtype=np.int64)
    Qr = Q[:, :, ri, :]
    # scores
    S = scale * np.matmul(Qr, np.swapaxes(K, 2, 3))
    if causal:
        hidden = np.arange(Nk)[None, :] > ri[:, None]
        S = np.where(hidden[None, None, :, :], -np.inf, S)
    # softmax over keys
    m = np.max(S, axis=3, keepdims=True)
    E = np.exp(S - m)
    P = E / np.sum(E, axis=3, keepdims=True)
    # weighted values
    return np.matmul(P, V)
