"""GPU test of the allocation-free entry point (gemm_fused_noalloc) through
the C ABI: its results against gemm_fused's on the same arguments (the same
plan, so the same bits) and against the oracle, on two calls in a row, the
second with a smaller product, both split-K plans whose workspace is the
library's fixed scratch; then a plan without slices and one with an
epilogue.  Integer inputs in [-2, 2] keep every sum exact in fp32.  The
device's free memory is the same before and after the allocation-free calls
(after a first pass that loads the library's code objects and its fixed
scratch on the GPU).
"""
import numpy as np
import pytest
import torch

import oracle
import tiled_gemm_03_amd as T
from tiled_gemm_03_amd import workloads as W

import gpu_helpers as G

pytestmark = pytest.mark.gpu

ROW = T.ROW_MAJOR


def call(fn, ad, bd, cd, in_dt, out_dt, ep=None):
    M, K = ad.shape
    N = bd.shape[1]
    stream = torch.cuda.current_stream().cuda_stream
    return fn(M, N, K, ad.data_ptr(), ad.stride(0), ROW, bd.data_ptr(), bd.stride(0), ROW, cd.data_ptr(),
              cd.stride(0), ROW, in_dt, out_dt, ep, stream, -1)


def test_noalloc_matches_gemm_fused_on_two_calls_in_a_row():
    cases = [((512, 512, 16384), True), ((256, 256, 8192), True), ((1024, 1024, 1024), False)]
    prepared = []
    for (M, N, K), split in cases:
        a, b = W.integer_inputs(M, N, K, W.F16, seed=M + K)
        ad, bd = G.to_device(a, W.F16), G.to_device(b, W.F16)
        _, c_ref = G.out_tensor(M, N, W.F16)
        _, c_na = G.out_tensor(M, N, W.F16)
        s = T.gemm_split_count_t(M, N, K, ad.data_ptr(), K, ROW, bd.data_ptr(), N, ROW, c_na.data_ptr(), N, ROW,
                                 W.F16, W.F16)
        assert (s > 1) == split, s
        prepared.append((M, N, K, a, b, ad, bd, c_ref, c_na, s))
    # a first pass loads the library's code objects (and with them the
    # fixed scratch) on this GPU; the measured pass allocates nothing
    for rep in range(2):
        torch.cuda.synchronize()
        free0 = torch.cuda.mem_get_info()[0]
        for M, N, K, a, b, ad, bd, c_ref, c_na, s in prepared:
            G.say(f"[case] gemm_fused_noalloc {M}x{N}x{K} slices {s} pass {rep}")
            c_na.fill_(float("nan"))
            rc = call(T.gemm_fused_noalloc, ad, bd, c_na, W.F16, W.F16)
            assert rc == T.OK, T.gemm_strerror(rc)
            torch.cuda.synchronize()
        free1 = torch.cuda.mem_get_info()[0]
    assert free1 == free0, (free0, free1)
    for M, N, K, a, b, ad, bd, c_ref, c_na, s in prepared:
        G.say(f"[case] gemm_fused {M}x{N}x{K} slices {s}")
        assert call(T.gemm_fused, ad, bd, c_ref, W.F16, W.F16) == T.OK
        torch.cuda.synchronize()
        got, ref = G.values(c_na, W.F16), G.values(c_ref, W.F16)
        assert np.array_equal(got, ref), f"{int((got != ref).sum())} entries differ from gemm_fused"
        want = G.round_to(G.oracle_values(a, b, W.F16), W.F16)
        assert np.array_equal(got, want), f"{int((got != want).sum())} entries differ from the oracle"


def test_noalloc_epilogue_and_errors():
    """A split plan with alpha, beta C, a column bias and relu; the argument
    errors of gemm_fused."""
    M, N, K = 512, 512, 16384
    a, b = W.integer_inputs(M, N, K, W.F16, seed=3)
    ad, bd = G.to_device(a, W.F16), G.to_device(b, W.F16)
    rng = np.random.default_rng(4)
    c_old = rng.integers(-8, 9, size=(M, N)).astype(np.float32)
    bias = rng.integers(-4, 5, size=N).astype(np.float32)
    bd_bias = torch.from_numpy(bias).to(G.DEV)
    _, cd = G.out_tensor(M, N, W.F32)
    cd.copy_(torch.from_numpy(c_old).to(G.DEV))
    ep = T.Epilogue(2.0, -0.5, bd_bias.data_ptr(), T.BIAS_COL, T.F32, T.ACT_RELU)
    G.say(f"[case] gemm_fused_noalloc epilogue {M}x{N}x{K}")
    rc = call(T.gemm_fused_noalloc, ad, bd, cd, W.F16, W.F32, ep)
    assert rc == T.OK, T.gemm_strerror(rc)
    torch.cuda.synchronize()
    want = oracle.gemm_fused(a, b, W.F16, alpha=2.0, beta=-0.5, c_old=c_old, out_dtype=W.F32, bias=bias,
                             bias_dtype=W.F32, bias_kind=oracle.BIAS_COL, act=oracle.ACT_RELU, nthreads=G.NTHREADS)
    assert np.array_equal(G.values(cd, W.F32), want.astype(np.float32).astype(np.float64))
    # argument errors come before any GPU work
    bad = T.Epilogue(1.0, 0.0, None, T.BIAS_NONE, T.F32, 99)
    assert call(T.gemm_fused_noalloc, ad, bd, cd, W.F16, W.F32, bad) == T.ERR_EPILOGUE
    assert T.gemm_fused_noalloc(-1, 4, 4, ad.data_ptr(), 4, ROW, bd.data_ptr(), 4, ROW, cd.data_ptr(), 4, ROW,
                                W.F16, W.F16, None, None, -1) == T.ERR_DIM
