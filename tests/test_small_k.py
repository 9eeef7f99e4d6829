"""GPU parity of products whose K is below the ring kernel's step (128): the
ring's K-tail variant then runs its tail alone, steps of 32 of K with the
MFMA fragments loaded straight from global memory (no LDS ring), for every
operand layout, the ring tiles and the table's choice, plain and fused
epilogues and an 8-bit output.

Integer inputs in [-2, 2] make every fp32 sum exact: results must equal the
oracle bit for bit after rounding to the output type.  Operands sit in
NaN-filled buffers with padded rows (G.to_device), so a read past K that is
not masked turns an output into NaN.  Every case prints its shape, layouts
and kernel before it touches the GPU.
"""
import numpy as np
import pytest
import torch

import oracle
import tiled_gemm_03_amd as T
from tiled_gemm_03_amd import workloads as W

import gpu_helpers as G

pytestmark = pytest.mark.gpu

ROW, COL = T.ROW_MAJOR, T.COL_MAJOR
RING = T.KERNEL_RING


def lid(lay):
    return "".join("r" if x == ROW else "c" for x in lay)


def place(x, dt, layout, pad=0):
    if layout == ROW:
        return G.to_device(x, dt, pad_cols=pad)
    return G.to_device(np.ascontiguousarray(x.T), dt, pad_cols=pad).t()


def kernel_of(ad, bd, cd, in_dt, out_dt, cid):
    M, K = ad.shape
    N = bd.shape[1]
    la, lda = T._layout(ad)
    lb, ldb = T._layout(bd)
    lc, ldc = T._layout(cd)
    return T.gemm_select_kernel_t(M, N, K, ad.data_ptr(), lda, la, bd.data_ptr(), ldb, lb, cd.data_ptr(), ldc, lc,
                                  in_dt, out_dt, cid)


# K: one element, less than one 8-element fragment, one step of 32, two, a
# ragged step, one short of the ring's step
KS = [1, 7, 32, 64, 100, 127]


# every layout pair with the 256 x 256 and 128 x 128 rings and the table's
# choice; the 64 x 128 ring reads row-major A only
CASES = [(lay, cid) for lay in [(ROW, ROW), (ROW, COL), (COL, ROW), (COL, COL)] for cid in (0, 1, -1)] + \
        [((ROW, ROW), 8), ((ROW, COL), 8)]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{lid(c[0])}_cfg{c[1]}")
def test_small_k_exact(case):
    """Ragged M and N (one partial tile each way) and every K of KS; fp16,
    bf16 and fp32 outputs in turn."""
    lay, cid = case
    M, N = 300, 260
    for i, K in enumerate(KS):
        in_dt, out_dt = ((W.F16, W.F16), (W.BF16, W.F32), (W.F16, W.F32))[i % 3]
        a, b = W.integer_inputs(M, N, K, in_dt, seed=K + 10 * i)
        ad, bd = place(a, in_dt, lay[0], pad=3), place(b, in_dt, lay[1], pad=5)
        _, cd = G.out_tensor(M, N, out_dt)
        kind, cfg = kernel_of(ad, bd, cd, in_dt, out_dt, cid)
        G.say(f"[case] small K {M}x{N}x{K} lay={lid(lay)} in={in_dt} out={out_dt} cfg{cid} -> kind {kind} cfg{cfg}")
        assert kind == RING, (kind, cfg)
        G.run(ad, bd, cd, cid)
        got = G.values(cd, out_dt)
        want = G.round_to(G.oracle_values(a, b, in_dt), out_dt)
        bad = got != want
        assert not bad.any(), f"K={K}: {int(bad.sum())} entries differ, first at {np.argwhere(bad)[0].tolist()}"


@pytest.mark.parametrize("K", [16, 100])
def test_small_k_fused_and_fp8(K):
    """alpha, beta C, a column bias and relu; then an E4M3 output (the fused
    epilogue's 8-bit conversion), which the direct kernel wrote before the
    ring took these products; exact on integer values."""
    M, N = 1024, 2048
    a, b = W.integer_inputs(M, N, K, W.F16, seed=K)
    ad, bd = G.to_device(a, W.F16), G.to_device(b, W.F16)
    rng = np.random.default_rng(K)
    c_old = rng.integers(-8, 9, size=(M, N)).astype(np.float32)
    bias = rng.integers(-4, 5, size=N).astype(np.float32)
    _, cd = G.out_tensor(M, N, W.F32)
    cd.copy_(torch.from_numpy(c_old).to(G.DEV))
    kind, cfg = kernel_of(ad, bd, cd, W.F16, W.F32, -1)
    G.say(f"[case] small K fused {M}x{N}x{K} -> kind {kind} cfg{cfg}")
    assert kind == RING
    T.gemm_tensors(ad, bd, cd, alpha=2.0, beta=-0.5, bias=torch.from_numpy(bias).to(G.DEV), activation=T.ACT_RELU)
    torch.cuda.synchronize()
    want = oracle.gemm_fused(a, b, W.F16, alpha=2.0, beta=-0.5, c_old=c_old, out_dtype=W.F32, bias=bias,
                             bias_dtype=W.F32, bias_kind=oracle.BIAS_COL, act=oracle.ACT_RELU, nthreads=G.NTHREADS)
    got = G.values(cd, W.F32)
    assert np.array_equal(got, want.astype(np.float32).astype(np.float64)), f"{int((got != want).sum())} differ"
    c8 = torch.zeros((M, N), dtype=torch.float8_e4m3fn, device=G.DEV)
    kind, cfg = kernel_of(ad, bd, c8, W.F16, T.FP8_E4M3, -1)
    G.say(f"[case] small K E4M3 {M}x{N}x{K} -> kind {kind} cfg{cfg}")
    assert kind == RING
    T.gemm_tensors(ad, bd, c8, alpha=1.0 / 8)
    torch.cuda.synchronize()
    got8 = c8.cpu().view(torch.uint8).numpy()
    want8 = oracle.encode_fp8(oracle.gemm(a, b, W.F16, nthreads=G.NTHREADS) / 8, T.FP8_E4M3)
    assert np.array_equal(got8, want8), f"{int((got8 != want8).sum())} entries differ"
