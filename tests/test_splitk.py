"""GPU parity of split-K: products whose ring tiles leave most CUs idle and
whose K is long run the ring kernel over slices of K (fp32 partials in a
workspace from the stream's memory pool), then a kernel that sums the slices
in a fixed order and applies the call's epilogue.

Integer inputs in [-2, 2] keep every partial and every sum exact in fp32, so
the results must equal the oracle bit for bit after the output rounding,
whatever the slicing; random normal inputs are held to the stated tolerance
and the fp32-accumulation bound (which holds for any summation order).  The
plan (kernel kind, configuration, slice count) is asserted for every case,
and each case prints its shape and plan before it touches the GPU.
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
SPLIT = T.KERNEL_RING_SPLITK


def place(x, dt, layout, pad=0):
    if layout == ROW:
        return G.to_device(x, dt, pad_cols=pad)
    return G.to_device(np.ascontiguousarray(x.T), dt, pad_cols=pad).t()


def plan_of(ad, bd, cd, in_dt, out_dt):
    M, K = ad.shape
    N = bd.shape[1]
    la, lda = T._layout(ad)
    lb, ldb = T._layout(bd)
    lc, ldc = T._layout(cd)
    kind, cfg = T.gemm_select_kernel_t(M, N, K, ad.data_ptr(), lda, la, bd.data_ptr(), ldb, lb, cd.data_ptr(), ldc,
                                       lc, in_dt, out_dt)
    s = T.gemm_split_count_t(M, N, K, ad.data_ptr(), lda, la, bd.data_ptr(), ldb, lb, cd.data_ptr(), ldc, lc,
                             in_dt, out_dt)
    return kind, cfg, s


# (M, N, K, pad of A's rows, expected configuration): 64 x 128 tiles in 8
# slices; a K tail in the last slice; 2 slices of 128 tiles; a skinny
# product; 32 slices
SHAPES = [(512, 512, 16384, 0, 8), (256, 256, 8192 + 300, 4, 8), (1024, 1024, 8192, 0, 8), (32, 4096, 4096, 0, 8),
          (200, 304, 6144, 0, 8)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s[:3])))
def test_split_k_exact(shape):
    M, N, K, pad, cfg = shape
    for in_dt, out_dt in ((W.F16, W.F16), (W.BF16, W.F32), (W.F16, W.F32), (W.BF16, W.BF16)):
        a, b = W.integer_inputs(M, N, K, in_dt, seed=M + N + K)
        ad, bd = G.to_device(a, in_dt, pad_cols=pad), G.to_device(b, in_dt)
        flat, cd = G.out_tensor(M, N, out_dt, pad_cols=8)
        kind, c, s = plan_of(ad, bd, cd, in_dt, out_dt)
        G.say(f"[case] split-K {M}x{N}x{K} in={in_dt} out={out_dt} -> kind {kind} cfg{c} slices {s}")
        assert (kind, c) == (SPLIT, cfg) and s > 1
        G.run(ad, bd, cd)
        got = G.values(cd, out_dt)
        want = G.round_to(G.oracle_values(a, b, in_dt), out_dt)
        assert np.array_equal(got, want), f"{int((got != want).sum())} entries differ"
        whole = flat[:M * (N + 8)].view(M, N + 8)
        assert torch.isnan(whole[:, N:].float()).all(), "padding columns written"
        assert torch.isnan(flat[M * (N + 8):].float()).all(), "memory after C written"


def test_split_k_layouts_and_unaligned_c():
    """Column-major A (128 x 128 tiles in slices), a column-major C (the
    flipped product), and C rows not 4-element aligned (the summing kernel's
    element stores)."""
    M, N, K = 512, 512, 16384
    a, b = W.integer_inputs(M, N, K, W.F16, seed=5)
    want = G.round_to(G.oracle_values(a, b, W.F16), W.F16)
    for la, lc, cpad in ((COL, ROW, 0), (ROW, COL, 0), (ROW, ROW, 3)):
        ad, bd = place(a, W.F16, la), place(b, W.F16, ROW)
        if lc == ROW:
            cd = G.out_tensor(M, N, W.F16, pad_cols=cpad)[1]
        else:
            cd = G.out_tensor(N, M, W.F16)[1].t()
        kind, c, s = plan_of(ad, bd, cd, W.F16, W.F16)
        G.say(f"[case] split-K layouts a={la} c={lc} cpad={cpad} -> kind {kind} cfg{c} slices {s}")
        assert kind == SPLIT and s > 1
        G.run(ad, bd, cd)
        got = G.values(cd, W.F16)
        assert np.array_equal(got, want), f"{int((got != want).sum())} entries differ"


def test_split_k_fused_epilogue_and_fp8():
    """alpha, beta C, a column bias and relu applied once, after the sum;
    an 8-bit output; all exact on integer values."""
    M, N, K = 512, 512, 16384
    a, b = W.integer_inputs(M, N, K, W.F16, seed=6)
    ad, bd = G.to_device(a, W.F16), G.to_device(b, W.F16)
    rng = np.random.default_rng(7)
    c_old = rng.integers(-8, 9, size=(M, N)).astype(np.float32)
    bias = rng.integers(-4, 5, size=N).astype(np.float32)
    _, cd = G.out_tensor(M, N, W.F32)
    cd.copy_(torch.from_numpy(c_old).to(G.DEV))
    kind, c, s = plan_of(ad, bd, cd, W.F16, W.F32)
    G.say(f"[case] split-K fused {M}x{N}x{K} -> kind {kind} cfg{c} slices {s}")
    assert kind == SPLIT
    T.gemm_tensors(ad, bd, cd, alpha=2.0, beta=-0.5, bias=torch.from_numpy(bias).to(G.DEV), activation=T.ACT_RELU)
    torch.cuda.synchronize()
    want = oracle.gemm_fused(a, b, W.F16, alpha=2.0, beta=-0.5, c_old=c_old, out_dtype=W.F32, bias=bias,
                             bias_dtype=W.F32, bias_kind=oracle.BIAS_COL, act=oracle.ACT_RELU, nthreads=G.NTHREADS)
    got = G.values(cd, W.F32)
    assert np.array_equal(got, want.astype(np.float32).astype(np.float64)), \
        f"{int((got != want).sum())} entries differ"
    c8 = torch.zeros((M, N), dtype=torch.float8_e4m3fn, device=G.DEV)
    kind, c, s = plan_of(ad, bd, c8, W.F16, T.FP8_E4M3)
    G.say(f"[case] split-K fp8 {M}x{N}x{K} -> kind {kind} cfg{c} slices {s}")
    assert kind == SPLIT
    T.gemm_tensors(ad, bd, c8, alpha=1.0 / 16)
    torch.cuda.synchronize()
    got8 = c8.cpu().view(torch.uint8).numpy()
    want8 = oracle.encode_fp8(oracle.gemm(a, b, W.F16, nthreads=G.NTHREADS) / 16, T.FP8_E4M3)
    assert np.array_equal(got8, want8), f"{int((got8 != want8).sum())} entries differ"


def test_split_k_random_values_and_determinism():
    """Random normal inputs: the tolerance and the fp32-accumulation bound;
    the same call twice gives the same bits (the slices are summed in a
    fixed order)."""
    for (M, N, K), in_dt, out_dt in (((512, 512, 16384), W.F16, W.F16), ((256, 256, 65536), W.BF16, W.F32)):
        a, b = W.random_inputs(M, N, K, in_dt, seed=K)
        ad, bd = G.to_device(a, in_dt), G.to_device(b, in_dt)
        _, cd = G.out_tensor(M, N, out_dt)
        kind, c, s = plan_of(ad, bd, cd, in_dt, out_dt)
        G.say(f"[case] split-K random {M}x{N}x{K} -> kind {kind} cfg{c} slices {s}")
        assert kind == SPLIT and s > 1
        G.run(ad, bd, cd)
        first = G.values(cd, out_dt)
        G.check(first, G.oracle_values(a, b, in_dt), a, b, in_dt, out_dt, K, label="split-K random")
        G.run(ad, bd, cd)
        assert np.array_equal(G.values(cd, out_dt), first)


def test_split_k_other_stream():
    """A call on a stream of its own (the workspace is that stream's) next to
    one on the current stream."""
    M, N, K = 512, 512, 16384
    a, b = W.integer_inputs(M, N, K, W.F16, seed=8)
    ad, bd = G.to_device(a, W.F16), G.to_device(b, W.F16)
    _, c1 = G.out_tensor(M, N, W.F32)
    _, c2 = G.out_tensor(M, N, W.F32)
    other = torch.cuda.Stream()
    torch.cuda.synchronize()
    G.say("[case] split-K on two streams")
    T.gemm_tensors(ad, bd, c1)
    with torch.cuda.stream(other):
        T.gemm_tensors(ad, bd, c2, stream=other.cuda_stream)
    torch.cuda.synchronize()
    want = G.oracle_values(a, b, W.F16)
    assert np.array_equal(G.values(c1, W.F32), want)
    assert np.array_equal(G.values(c2, W.F32), want)


def test_split_k_workspaces_across_many_streams():
    """The library keeps one workspace per stream for its last 8 streams:
    calls on 10 streams in turn, three rounds, take workspaces over from one
    another (the least recently used one, after its last call's kernels) and
    grow them (4, 8, then 16 MiB of partials), with no synchronisation
    between the calls; every result exact."""
    shapes = [(256, 256, 4096), (256, 256, 65536), (512, 512, 16384)]
    rounds = []
    for i, (M, N, K) in enumerate(shapes):
        a, b = W.integer_inputs(M, N, K, W.F16, seed=30 + i)
        ad, bd = G.to_device(a, W.F16), G.to_device(b, W.F16)
        outs = [G.out_tensor(M, N, W.F32)[1] for _ in range(10)]
        kind, cfg, s = plan_of(ad, bd, outs[0], W.F16, W.F32)
        assert kind == SPLIT and s > 1, (M, N, K, kind, s)
        rounds.append((ad, bd, outs, G.oracle_values(a, b, W.F16), s))
    streams = [torch.cuda.Stream() for _ in range(10)]
    torch.cuda.synchronize()  # inputs and NaN-filled outputs in place before any other stream runs
    for ad, bd, outs, _, s in rounds:
        G.say(f"[case] split-K {tuple(ad.shape)} x {tuple(bd.shape)}, {s} slices, on 10 streams")
        for st, c in zip(streams, outs):
            with torch.cuda.stream(st):
                T.gemm_tensors(ad, bd, c, stream=st.cuda_stream)
    torch.cuda.synchronize()
    for _, _, outs, want, _ in rounds:
        for c in outs:
            assert np.array_equal(G.values(c, W.F32), want)
