"""Pins of the attention oracle (oracle/attention.py) against facts that do
not come from it: torch.nn.functional.scaled_dot_product_attention in float64
on the CPU (an independent library routine), the blockwise online-softmax
algorithm of page "TileLang实战：用Python DSL自动生成高性能GPU计算内核" §4.2
written out here on its own, and closed forms.

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


def _online_blocks(Q, K, V, scale, causal, block):
    """The page's blockwise algorithm: walk K, V in blocks, keep per query the
    running maximum M, normaliser L and normalised output O."""
    Nq, d = Q.shape
    Nk = K.shape[0]
    O = np.zeros((Nq, d))
    L = np.zeros(Nq)
    M = np.full(Nq, -np.inf)
    for s in range(0, Nk, block):
        Kb, Vb = K[s:s + block], V[s:s + block]
        for i in range(Nq):
            sc = scale * (Kb @ Q[i])
            if causal:
                sc = np.where(np.arange(s, s + len(sc)) > i, -np.inf, sc)
            if np.all(np.isneginf(sc)):
                continue
            m_new = max(M[i], np.max(sc))
            l_new = L[i] * np.exp(M[i] - m_new) + np.sum(np.exp(sc - m_new))
            O[i] = (O[i] * L[i] * np.exp(M[i] - m_new) + np.exp(sc - m_new) @ Vb) / l_new
            L[i], M[i] = l_new, m_new
    return O


def pin_attention_vs_online_blocks(att):
    for (Nq, Nk, d, causal, block, seed) in ((6, 11, 8, False, 4, 6), (10, 10, 16, True, 3, 7), (5, 13, 4, True, 5, 8)):
        q, k, v = _qkv(1, 1, Nq, Nk, d, W.F16, seed)
        got = att(q, k, v, W.F16, scale=0.3, causal=causal)[0, 0]
        want = _online_blocks(_vals(q, W.F16)[0, 0], _vals(k, W.F16)[0, 0], _vals(v, W.F16)[0, 0], 0.3, causal, block)
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


ATTENTION_PINS = [pin_attention_vs_torch, pin_attention_vs_online_blocks, pin_attention_closed_forms,
                  pin_attention_sampled_rows]
