"""GPU parity: the HIP path (through the C ABI) against the oracle.

Every case prints its name, shape and configuration before it touches the
GPU.  Floating-point cases are held to the two comparisons of gpu_helpers
(the stated tolerance and the rigorous fp32-accumulation bound); cases with
small-integer inputs, whose fp32 sums are exact in any order, must match the
oracle bit for bit after rounding to the output type.
"""
import math

import numpy as np
import pytest
import torch

import tiled_gemm_03_amd as T
from tiled_gemm_03_amd import workloads as W

import gpu_helpers as G

pytestmark = pytest.mark.gpu

NCFG = None


def configs_for(in_dt):
    fam = W.F32 if in_dt == W.F32 else W.F16
    return [i for i in range(T.gemm_num_configs()) if T.gemm_config_info(i)["in_dtype"] == fam]


def run_case(a, b, in_dt, out_dt, config=-1, rows=None, cols=None, label="", pad=(0, 0, 0),
             offset=(0, 0, 0)):
    M, K = a.shape
    N = b.shape[1]
    G.say(f"[case] {label} M={M} N={N} K={K} in={in_dt} out={out_dt} config={config} pad={pad} off={offset}")
    ad = G.to_device(a, in_dt, pad_cols=pad[0], offset_elems=offset[0])
    bd = G.to_device(b, in_dt, pad_cols=pad[1], offset_elems=offset[1])
    flat, cd = G.out_tensor(M, N, out_dt, pad_cols=pad[2], offset_elems=offset[2])
    G.run(ad, bd, cd, config)
    c = G.values(cd, out_dt)
    if rows is not None:
        c = c[rows][:, cols]
    o = G.oracle_values(a, b, in_dt, rows=rows, cols=cols)
    m = G.check(c, o, a, b, in_dt, out_dt, K, rows=rows, cols=cols, label=label)
    G.say(f"    ok {m}")
    return c, o, flat, cd


# ------------------------------------------------------------------ workloads
@pytest.mark.parametrize("w", W.WORKLOADS[:4], ids=lambda w: w.name)
def test_workload_table_config(w):
    a, b = W.make_inputs(w)
    run_case(a, b, w.in_dtype, w.out_dtype, label=w.name)


def test_workload_8192_sampled():
    w = W.WORKLOADS[4]
    a, b = W.make_inputs(w)
    rows = W.sample_indices(w.M, 64, w.seed + 100)
    cols = W.sample_indices(w.N, 64, w.seed + 200)
    run_case(a, b, w.in_dtype, w.out_dtype, rows=rows, cols=cols, label=w.name)


@pytest.mark.parametrize("w", W.WORKLOADS[:4], ids=lambda w: w.name)
def test_workload_every_config(w):
    a, b = W.make_inputs(w)
    for cid in configs_for(w.in_dtype):
        run_case(a, b, w.in_dtype, w.out_dtype, config=cid, label=f"{w.name}/cfg{cid}")


def test_bf16_at_128x256x512():
    w = W.WORKLOADS[1]
    a, b = W.make_inputs(w, in_dtype=W.BF16)
    for out in (W.BF16, W.F32):
        for cid in [-1] + configs_for(W.BF16):
            run_case(a, b, W.BF16, out, config=cid, label=f"bf16->{out}/cfg{cid}")


# --------------------------------------------------------- ragged multi-tile
@pytest.mark.parametrize("cid", range(T.gemm_num_configs()))
def test_ragged_tiles_each_config(cid):
    info = T.gemm_config_info(cid)
    in_dts = [W.F32] if info["in_dtype"] == W.F32 else [W.F16, W.BF16]
    bm, bn, bk = info["block_m"], info["block_n"], info["block_k"]
    shapes = [(2 * bm + 7, 3 * bn - 5, 3 * bk + 9), (bm - 1, bn + 1, bk - 3), (3 * bm, 2 * bn, 2 * bk + 1)]
    if info["stages"] == 0:
        # the direct kernel's register ring holds 8 steps of 32 (4 for 16-bit
        # A read element by element): K below, at and past whole rings
        shapes += [(33, 47, 255), (64, 64, 256), (50, 70, 257), (31, 33, 1000)]
    for in_dt in in_dts:
        outs = [W.F32, in_dt] if in_dt != W.F32 else [W.F32]
        for (M, N, K) in shapes:
            for out in outs:
                a, b = W.random_inputs(M, N, K, in_dt, seed=M * 7 + N * 3 + K)
                run_case(a, b, in_dt, out, config=cid, label=f"ragged cfg{cid}")


# ------------------------------------------------------ exact (bitwise) cases
EXACT_SHAPES = [(128, 128, 128), (128, 256, 512), (127, 255, 512), (1024, 2048, 512), (300, 257, 1000)]


@pytest.mark.parametrize("shape", EXACT_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("pair", [(W.F16, W.F16), (W.F16, W.F32), (W.BF16, W.BF16), (W.BF16, W.F32),
                                  (W.F32, W.F32)], ids=lambda p: f"{p[0]}to{p[1]}")
def test_integer_inputs_bitwise(shape, pair):
    M, N, K = shape
    in_dt, out_dt = pair
    a, b = W.integer_inputs(M, N, K, in_dt, seed=M + N + K)
    want = G.round_to(G.oracle_values(a, b, in_dt), out_dt)
    ad, bd = G.to_device(a, in_dt), G.to_device(b, in_dt)
    for cid in [-1] + configs_for(in_dt):
        G.say(f"[case] integer {shape} {pair} cfg{cid}")
        _, cd = G.out_tensor(M, N, out_dt)
        G.run(ad, bd, cd, cid)
        got = G.values(cd, out_dt)
        assert np.array_equal(got, want), f"cfg{cid}: {int((got != want).sum())} entries differ"


def test_integer_inputs_bitwise_8192_sampled():
    M = N = K = 8192
    a, b = W.integer_inputs(M, N, K, W.F16, seed=8192)
    G.say("[case] integer 8192^3 f16->f16 sampled")
    ad, bd = G.to_device(a, W.F16), G.to_device(b, W.F16)
    _, cd = G.out_tensor(M, N, W.F16)
    G.run(ad, bd, cd)
    rows = W.sample_indices(M, 96, 77)
    cols = W.sample_indices(N, 96, 78)
    want = G.round_to(G.oracle_values(a, b, W.F16, rows=rows, cols=cols), W.F16)
    got = G.values(cd, W.F16)[rows][:, cols]
    assert np.array_equal(got, want)


@pytest.mark.parametrize("shape", [(128, 128, 128), (128, 256, 512), (127, 255, 512), (1024, 2048, 512),
                                   (8192, 8192, 8192)], ids=lambda s: "x".join(map(str, s)))
def test_all_ones_every_shape(shape):
    """Every entry equals K (exact in every output type used here)."""
    M, N, K = shape
    for in_dt, out_dt in ((W.F16, W.F16), (W.F16, W.F32), (W.BF16, W.F32), (W.F32, W.F32)):
        if in_dt == W.F32 and M * N * K > 2 ** 31:
            continue
        G.say(f"[case] ones {shape} {in_dt}->{out_dt}")
        a = torch.ones((M, K), dtype=G.TORCH[in_dt], device=G.DEV)
        b = torch.ones((K, N), dtype=G.TORCH[in_dt], device=G.DEV)
        _, c = G.out_tensor(M, N, out_dt)
        G.run(a, b, c)
        assert bool((c.to(torch.float64) == K).all()), f"ones {shape}: not all entries == {K}"


@pytest.mark.parametrize("n", [128, 512, 8192])
def test_identity(n):
    """I x B == B and A x I == A exactly, in full."""
    a, b = W.random_inputs(n, n, n, W.F16, seed=n)
    G.say(f"[case] identity n={n}")
    eye = torch.eye(n, dtype=torch.float16, device=G.DEV)
    bd = G.to_device(b, W.F16)
    ad = G.to_device(a, W.F16)
    _, c = G.out_tensor(n, n, W.F16)
    G.run(eye, bd, c)
    assert torch.equal(c, bd), "I x B != B"
    _, c2 = G.out_tensor(n, n, W.F32)
    G.run(ad, eye, c2)
    assert torch.equal(c2, ad.to(torch.float32)), "A x I != A"


@pytest.mark.parametrize("out_dt,K,want", [(W.F16, 2049, 2048.0), (W.F16, 2051, 2052.0),
                                           (W.F16, 2053, 2052.0), (W.BF16, 257, 256.0),
                                           (W.BF16, 259, 260.0)])
def test_round_to_nearest_even(out_dt, K, want):
    """All-ones products whose exact value K is a tie in the output type:
    round-to-nearest-even gives `want` (rounding toward zero would give
    2050 for K = 2051 and 258 for K = 259)."""
    in_dt = W.F16 if out_dt == W.F16 else W.BF16
    G.say(f"[case] rne out={out_dt} K={K}")
    for cid in [-1] + configs_for(in_dt):
        a = torch.ones((64, K), dtype=G.TORCH[in_dt], device=G.DEV)
        b = torch.ones((K, 64), dtype=G.TORCH[in_dt], device=G.DEV)
        _, c = G.out_tensor(64, 64, out_dt)
        G.run(a, b, c, cid)
        vals = set(np.unique(G.values(c, out_dt)).tolist())
        assert vals == {want}, f"cfg{cid}: {vals}"


# ------------------------------------------------- coverage and guard bands
@pytest.mark.parametrize("shape", [(127, 255, 512), (300, 200, 100), (1024, 2048, 512), (513, 769, 65)],
                         ids=lambda s: "x".join(map(str, s)))
def test_nan_canary_and_guard_band(shape):
    """C starts as NaN: every entry of the M x N window must be written, and
    the 8 padding columns of every row (ldc = N + 8) plus the tail after the
    last row must keep their sentinel value."""
    M, N, K = shape
    for cid in [-1] + configs_for(W.F16):
        for out_dt in (W.F16, W.F32):
            a, b = W.random_inputs(M, N, K, W.F16, seed=5)
            G.say(f"[case] canary {shape} cfg{cid} out={out_dt}")
            ad, bd = G.to_device(a, W.F16), G.to_device(b, W.F16)
            flat = torch.full((M * (N + 8) + 64,), float("nan"), dtype=G.TORCH[out_dt], device=G.DEV)
            view = flat[:M * (N + 8)].view(M, N + 8)
            view[:, N:] = 12345.0
            flat[M * (N + 8):] = -777.0
            c = view[:, :N]
            G.run(ad, bd, c, cid)
            assert not bool(torch.isnan(c).any()), "some entries of C were not written"
            assert bool((view[:, N:] == 12345.0).all()), "padding columns were written"
            assert bool((flat[M * (N + 8):] == -777.0).all()), "memory after C was written"


def test_k_zero_writes_zeros():
    """K = 0: the empty sum, under the table's choice and every
    configuration; the operands are empty tensors (no memory to read)."""
    for in_dt, out_dt in ((W.F16, W.F16), (W.F32, W.F32), (W.BF16, W.F32)):
        for cid in [-1] + configs_for(in_dt):
            G.say(f"[case] K=0 {in_dt}->{out_dt} cfg{cid}")
            a = torch.empty((37, 0), dtype=G.TORCH[in_dt], device=G.DEV)
            b = torch.empty((0, 45), dtype=G.TORCH[in_dt], device=G.DEV)
            _, c = G.out_tensor(37, 45, out_dt)
            G.run(a, b, c, cid)
            assert bool((c == 0).all())


def test_empty_m_or_n_is_a_noop():
    a = torch.ones((0, 8), dtype=torch.float16, device=G.DEV)
    b = torch.ones((8, 8), dtype=torch.float16, device=G.DEV)
    c = torch.empty((0, 8), dtype=torch.float16, device=G.DEV)
    assert T.gemm_tensors(a, b, c, check=False) == T.OK
    torch.cuda.synchronize()


def test_padded_and_misaligned_operands():
    """Leading dimensions above the width, and base pointers one element off
    16-byte alignment, stay exact under every configuration, whichever kernel
    takes them (the ring where its loads keep every element, else an
    element-wise path)."""
    M, N, K = 200, 300, 150
    for in_dt, out_dt in ((W.F16, W.F32), (W.BF16, W.BF16), (W.F32, W.F32), (W.F16, W.F16)):
        a, b = W.random_inputs(M, N, K, in_dt, seed=9)
        for pad, off in (((8, 8, 8), (0, 0, 0)), ((3, 5, 1), (0, 0, 0)), ((0, 0, 0), (1, 0, 0)),
                         ((0, 0, 0), (0, 1, 0)), ((0, 0, 0), (0, 0, 1)), ((16, 0, 4), (8, 8, 4))):
            for cid in [-1] + configs_for(in_dt):
                run_case(a, b, in_dt, out_dt, config=cid, pad=pad, offset=off, label="pad/offset")


def test_random_shapes_stress():
    """A few hundred seeded random shapes in [1, 300]^3 over every type pair
    (the randomised stress step of the DeepSeek/Ascend toolkit page, §3.3)."""
    rng = np.random.default_rng(2024)
    pairs = [(W.F16, W.F16), (W.F16, W.F32), (W.BF16, W.BF16), (W.BF16, W.F32), (W.F32, W.F32)]
    n_cfg = T.gemm_num_configs()
    for i in range(240):
        M, N, K = (int(x) for x in rng.integers(1, 301, size=3))
        in_dt, out_dt = pairs[i % len(pairs)]
        cands = [-1] + configs_for(in_dt)
        cid = cands[int(rng.integers(0, len(cands)))]
        a, b = W.random_inputs(M, N, K, in_dt, seed=1000 + i)
        run_case(a, b, in_dt, out_dt, config=cid, label=f"stress{i}")
    assert n_cfg > 0


def test_long_k_and_tall_m():
    """Extreme aspect ratios: a 1 x 1 output summing 2^20 terms, and a tall
    matrix of 2^20 rows."""
    a, b = W.random_inputs(1, 1, 1 << 20, W.F16, seed=71)
    run_case(a, b, W.F16, W.F32, label="long K")
    a, b = W.random_inputs(1 << 20, 64, 64, W.F16, seed=72)
    rows = W.sample_indices(1 << 20, 512, 73)
    run_case(a, b, W.F16, W.F16, rows=rows, cols=np.arange(64), label="tall M")


def test_repeat_determinism():
    """No atomics and a fixed summation order: two runs are bitwise equal."""
    for w in (W.WORKLOADS[3], W.WORKLOADS[4]):
        a, b = W.make_inputs(w)
        G.say(f"[case] determinism {w.name}")
        ad, bd = G.to_device(a, w.in_dtype), G.to_device(b, w.in_dtype)
        _, c1 = G.out_tensor(w.M, w.N, w.out_dtype)
        _, c2 = G.out_tensor(w.M, w.N, w.out_dtype)
        G.run(ad, bd, c1)
        G.run(ad, bd, c2)
        assert torch.equal(c1, c2)


def test_invalid_arguments_on_gpu():
    a = torch.ones((4, 4), dtype=torch.float16, device=G.DEV)
    c = torch.ones((4, 4), dtype=torch.float16, device=G.DEV)
    p = a.data_ptr()
    assert T.gemm(4, 4, 4, p, 4, p, 4, p, 4, 1, 1, None) == T.ERR_ALIAS
    assert T.gemm(4, 4, 4, p, 4, p, 4, c.data_ptr(), 4, 1, 2, None) == T.ERR_DTYPE
    assert T.gemm(4, 4, 4, p, 3, p, 4, c.data_ptr(), 4, 1, 1, None) == T.ERR_LD
    torch.cuda.synchronize()


# ------------------------------------------------- the direct-to-LDS ring path
RING_SHAPES = [(256, 256, 128, 0), (256, 256, 256, 0), (512, 768, 384, 0), (256, 512, 640, 0),
               (128, 128, 128, 1), (384, 256, 512, 1), (1024, 2048, 512, 0), (1024, 2048, 512, 1)]


@pytest.mark.parametrize("shape", RING_SHAPES, ids=lambda s: "x".join(map(str, s[:3])) + f"_cfg{s[3]}")
def test_ring_path_against_oracle(shape):
    """Shapes that take the ring kernel (1 to 5 trips of its 4-step loop),
    every 16-bit type pair, against the oracle; the path is asserted."""
    M, N, K, cid = shape
    for in_dt, out_dt in ((W.F16, W.F16), (W.F16, W.F32), (W.BF16, W.BF16), (W.BF16, W.F32)):
        a, b = W.random_inputs(M, N, K, in_dt, seed=M + 3 * N + 7 * K)
        ad, bd = G.to_device(a, in_dt), G.to_device(b, in_dt)
        _, cd = G.out_tensor(M, N, out_dt)
        assert T.gemm_select_kernel(M, N, K, ad.data_ptr(), K, bd.data_ptr(), N, cd.data_ptr(), N, in_dt, out_dt,
                                    cid) == T.KERNEL_RING
        run_case(a, b, in_dt, out_dt, config=cid, label=f"ring {shape}")


# M and N not multiples of the tile (N a multiple of 4): the ring kernel with
# masked edge tiles
RING_RAGGED = [(1000, 1200, 512, 0), (1000, 1200, 512, 1), (777, 1000, 256, 0), (129, 136, 128, 1),
               (255, 264, 384, 0), (1, 8, 128, 0), (300, 1000, 128, 1), (1000, 1200, 640, 0), (513, 264, 1024, 1)]


@pytest.mark.parametrize("shape", RING_RAGGED, ids=lambda s: "x".join(map(str, s[:3])) + f"_cfg{s[3]}")
def test_ring_path_ragged_edges(shape):
    """Ragged M and N through the ring kernel (the path asserted): every
    element inside C against the oracle, the 8 padding columns of every row
    and the memory after C untouched (NaN-prefilled guard)."""
    M, N, K, cid = shape
    for in_dt, out_dt in ((W.F16, W.F16), (W.BF16, W.F32)):
        a, b = W.random_inputs(M, N, K, in_dt, seed=M + 5 * N + 9 * K + cid)
        ad, bd = G.to_device(a, in_dt), G.to_device(b, in_dt)
        flat, cd = G.out_tensor(M, N, out_dt, pad_cols=8)
        assert T.gemm_select_kernel(M, N, K, ad.data_ptr(), K, bd.data_ptr(), N, cd.data_ptr(), N + 8, in_dt,
                                    out_dt, cid) == T.KERNEL_RING
        G.say(f"[case] ring ragged {M}x{N}x{K} cfg{cid} in={in_dt} out={out_dt}")
        G.run(ad, bd, cd, cid)
        c = G.values(cd, out_dt)
        G.check(c, G.oracle_values(a, b, in_dt), a, b, in_dt, out_dt, K, label=f"ring ragged {shape}")
        whole = flat[:M * (N + 8)].view(M, N + 8)
        assert torch.isnan(whole[:, N:].float()).all(), "padding columns written"
        assert torch.isnan(flat[M * (N + 8):].float()).all(), "memory after C written"


@pytest.mark.parametrize("cid", [0, 1])
def test_ring_path_ignores_data_past_k(cid):
    """The ring kernel's loads run up to 4 steps of 32 past the end of K.  A
    and B live in NaN-filled buffers with padded rows (lda = K + 40,
    ldb = N + 24) and NaN after the last row: none of it may reach C, which
    must equal the oracle bit for bit (integer inputs)."""
    M, N, K = (512, 512, 256) if cid == 0 else (256, 384, 384)
    a, b = W.integer_inputs(M, N, K, W.F16, seed=cid + 40)
    lda, ldb = K + 40, N + 24
    fa = torch.full((M * lda + 4096,), float("nan"), dtype=torch.float16, device=G.DEV)
    fb = torch.full((K * ldb + 4096,), float("nan"), dtype=torch.float16, device=G.DEV)
    ad = fa[:M * lda].view(M, lda)[:, :K]
    bd = fb[:K * ldb].view(K, ldb)[:, :N]
    ad.copy_(torch.from_numpy(a).to(G.DEV))
    bd.copy_(torch.from_numpy(b).to(G.DEV))
    for out_dt in (W.F16, W.F32):
        _, cd = G.out_tensor(M, N, out_dt)
        G.say(f"[case] ring past-K {M}x{N}x{K} cfg{cid} out={out_dt}")
        assert T.gemm_select_kernel(M, N, K, ad.data_ptr(), lda, bd.data_ptr(), ldb, cd.data_ptr(), N, W.F16,
                                    out_dt, cid) == T.KERNEL_RING
        G.run(ad, bd, cd, cid)
        got = G.values(cd, out_dt)
        want = G.round_to(G.oracle_values(a, b, W.F16), out_dt)
        assert np.array_equal(got, want), f"{int((got != want).sum())} entries differ"


def test_workload_8192_takes_the_ring_path():
    w = W.WORKLOADS[4]
    a = torch.empty((w.M, w.K), dtype=torch.float16, device=G.DEV)
    b = torch.empty((w.K, w.N), dtype=torch.float16, device=G.DEV)
    c = torch.empty((w.M, w.N), dtype=torch.float16, device=G.DEV)
    assert T.gemm_select_kernel(w.M, w.N, w.K, a.data_ptr(), w.K, b.data_ptr(), w.N, c.data_ptr(), w.N, w.in_dtype,
                                w.out_dtype) == T.KERNEL_RING
