"""Pins of the attention oracle (oracle/attention.py) against facts that do
not come from it: torch.nn.functional.scaled_dot_product_attention in float64
on the CPU (an independent library routine), the block decomposition of the
softmax that the blockwise method of page "TileLang实战：用Python DSL自动生成
高性能GPU计算内核" §4.2 rests on (partial maxima, sums and weighted values per
block of keys, merged associatively), and closed forms.

Each pin takes the attention function to check, so that the same pins run
against the oracle (tests/test_oracle.py) and against copies of it with a
planted mistake (tests/test_oracle_mutants.py), where one must fail.
"""
import numpy as np

import oracle
from tiled_gemm_03_amd import workloads as W


def _qkv(B, H, Nq, Nk, d, dtype, seed):
    rng = np.random.default_rng(seed)
    mk = lambda n: W.to_storage(rng.standard_normal((B, H, n, d)).astype(np.float32), dtype)
    return mk(Nq), mk(Nk), mk(Nk)


def _vals(x, dtype):
    return oracle.decode(np.ascontiguousarray(x), dtype)


def pin_attention_vs_torch(att):
    import torch
    import torch.nn.functional as F
    for (B, H, Nq, Nk, d, dt, scale, causal, seed) in (
            (1, 2, 5, 7, 4, W.F16, 0.5, False, 1), (2, 3, 9, 9, 16, W.BF16, 0.25, True, 2),
            (1, 1, 7, 4, 8, W.F32, 1.0, True, 3), (1, 2, 33, 65, 64, W.F16, 0.125, False, 4),
            (2, 1, 40, 24, 32, W.F16, 1.0 / np.sqrt(32), True, 5)):
        q, k, v = _qkv(B, H, Nq, Nk, d, dt, seed)
        got = att(q, k, v, dt, scale=scale, causal=causal)
        tq, tk, tv = (torch.from_numpy(_vals(x, dt)) for x in (q, k, v))
        want = F.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale).numpy()
        assert np.allclose(got, want, rtol=1e-12, atol=1e-13), (B, H, Nq, Nk, d, causal, np.abs(got - want).max())


def _block_partials(Q, K, V, scale, causal, block):
    """Softmax attention over keys split into blocks, from the identity
    behind the blockwise method of page "TileLang实战：用Python DSL自动生成高性能
    GPU计算内核" §4.2: for any partition of the visible keys of a query into
    blocks, with m_b the block's largest score, s_b = sum exp(score - m_b)
    and u_b = sum exp(score - m_b) v over the block, the attention output is
    sum_b e^(m_b - m) u_b / sum_b e^(m_b - m) s_b for any m.  Each block's
    triple (m_b, s_b, u_b) is formed for all queries at once; the triples are
    merged two at a time in a balanced tree, each merge rescaling both sides
    to the larger of the two maxima; one division at the end."""
    Nq, d = Q.shape
    Nk = K.shape[0]
    parts = []
    for lo in range(0, Nk, block):
        hi = min(lo + block, Nk)
        S = scale * (Q @ K[lo:hi].T)                       # Nq x (hi - lo)
        if causal:
            S = np.where(np.arange(lo, hi)[None, :] > np.arange(Nq)[:, None], -np.inf, S)
        m = S.max(axis=1)                                  # -inf where no key of the block is visible
        safe = np.where(np.isneginf(m), 0.0, m)
        E = np.exp(S - safe[:, None])                      # exp(-inf) = 0 for hidden keys
        parts.append((m, E.sum(axis=1), E @ V[lo:hi]))

    def merge(x, y):
        (mx, sx, ux), (my, sy, uy) = x, y
        m = np.maximum(mx, my)
        safe = np.where(np.isneginf(m), 0.0, m)
        fx = np.where(np.isneginf(mx), 0.0, np.exp(mx - safe))
        fy = np.where(np.isneginf(my), 0.0, np.exp(my - safe))
        return m, fx * sx + fy * sy, fx[:, None] * ux + fy[:, None] * uy

    while len(parts) > 1:
        nxt = [merge(parts[t], parts[t + 1]) for t in range(0, len(parts) - 1, 2)]
        if len(parts) % 2:
            nxt.append(parts[-1])
        parts = nxt
    _, s_all, u_all = parts[0]
    return u_all / s_all[:, None]


def pin_attention_vs_block_partials(att):
    for (Nq, Nk, d, causal, block, seed) in ((6, 11, 8, False, 4, 6), (10, 10, 16, True, 3, 7), (5, 13, 4, True, 5, 8)):
        q, k, v = _qkv(1, 1, Nq, Nk, d, W.F16, seed)
        got = att(q, k, v, W.F16, scale=0.3, causal=causal)[0, 0]
        want = _block_partials(_vals(q, W.F16)[0, 0], _vals(k, W.F16)[0, 0], _vals(v, W.F16)[0, 0], 0.3, causal,
                               block)
        assert np.allclose(got, want, rtol=1e-12, atol=1e-13), (Nq, Nk, causal, np.abs(got - want).max())


def pin_attention_closed_forms(att):
    """Q = 0: every score is 0, so each query averages the values it sees:
    all of V, or (causal) rows 0..i of V.  Two keys e1, e2 and queries c e1:
    weights e^c / (e^c + 1) and 1 / (e^c + 1)."""
    q, k, v = _qkv(1, 2, 6, 9, 8, W.F16, 9)
    q0 = np.zeros_like(q)
    V = _vals(v, W.F16)
    got = att(q0, k, v, W.F16, scale=1.0)
    assert np.allclose(got, np.broadcast_to(V.mean(axis=2, keepdims=True), got.shape), rtol=1e-14, atol=1e-15)
    got = att(q0, k, v, W.F16, scale=1.0, causal=True)
    cum = np.cumsum(V, axis=2)[:, :, :6, :] / np.arange(1, 7)[None, None, :, None]
    assert np.allclose(got, cum, rtol=1e-14, atol=1e-15)
    k2 = np.zeros((1, 1, 2, 4), np.float16)
    k2[0, 0, 0, 0] = 1.0
    k2[0, 0, 1, 1] = 1.0
    v2 = np.array([[[[1, 2, 3, 4], [10, 20, 30, 40]]]], np.float16)
    q2 = np.zeros((1, 1, 3, 4), np.float16)
    q2[0, 0, :, 0] = [0.0, 1.0, 4.0]
    got = att(q2, k2, v2, W.F16, scale=1.0)[0, 0]
    for i, c in enumerate((0.0, 1.0, 4.0)):
        w0 = np.exp(c) / (np.exp(c) + 1.0)
        assert np.allclose(got[i], w0 * np.array([1, 2, 3, 4]) + (1 - w0) * np.array([10, 20, 30, 40]), rtol=1e-14)


def pin_attention_sampled_rows(att):
    q, k, v = _qkv(2, 2, 20, 17, 8, W.BF16, 10)
    full = att(q, k, v, W.BF16, scale=0.5, causal=True)
    rows = np.array([0, 3, 19, 7])
    assert np.array_equal(att(q, k, v, W.BF16, scale=0.5, causal=True, rows=rows), full[:, :, rows, :])


ATTENTION_PINS = [pin_attention_vs_torch, pin_attention_vs_block_partials, pin_attention_closed_forms,
                  pin_attention_sampled_rows]
