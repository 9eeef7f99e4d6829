"""GPU parity of the fused epilogue (gemm_fused): C := act(alpha AB + beta C +
bias) against the oracle (oracle.gemm_fused), on every kernel family and
layout of C.

Two comparisons:
1. bit for bit where every step is exact: small-integer inputs, alpha and
   beta powers of two, integer C and bias, no activation or relu (every
   value is an integer below 2^24, so fp32 computes it exactly in any order);
   the oracle is rounded to the output type;
2. elsewhere, an element-wise bound that any correct fp32 evaluation meets:
       |z_gpu - z| <= |alpha| B_K + 3 u (|alpha P| + |beta C| + |bias|)
   for z = alpha P + beta C + bias (B_K the fp32-accumulation bound of the
   product, gpu_helpers), then through the activation (slope at most L = 1.2
   for every activation here) plus 16 u of its result and of its argument
   for the fp32 erf / tanh / exp, plus the output rounding.
Every case prints its name and the kernel the library chose before it
touches the GPU.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import tiled_gemm_03_amd as T
from tiled_gemm_03_amd import workloads as W

import gpu_helpers as G

pytestmark = pytest.mark.gpu

ROW, COL = T.ROW_MAJOR, T.COL_MAJOR
KIND = {T.KERNEL_GENERAL: "general", T.KERNEL_TILED: "tiled", T.KERNEL_RING: "ring", T.KERNEL_DIRECT: "direct"}
U32 = 2.0 ** -24
SLOPE = 1.2


def place(x, dt, layout, pad=0):
    if layout == ROW:
        return G.to_device(x, dt, pad_cols=pad)
    return G.to_device(np.ascontiguousarray(x.T), dt, pad_cols=pad).t()


def vec_device(v, dt):
    host = torch.from_numpy(np.ascontiguousarray(v).view(np.int16)).view(torch.bfloat16) if dt == W.BF16 \
        else torch.from_numpy(np.ascontiguousarray(v))
    return host.to(G.DEV)


def run_fused(a, b, in_dt, out_dt, c_old, bias, bias_dt, bias_kind, alpha, beta, act, lay=(ROW, ROW, ROW),
              cid=-1, label=""):
    """Runs the fused product; returns (gpu values, the kernel kind)."""
    M, K = a.shape
    N = b.shape[1]
    ad, bd = place(a, in_dt, lay[0]), place(b, in_dt, lay[1])
    cd = place(c_old, out_dt, lay[2])
    bv = None if bias is None else vec_device(bias, bias_dt)
    la, lda = T._layout(ad)
    lb, ldb = T._layout(bd)
    lc, ldc = T._layout(cd)
    kind, cfg = T.gemm_select_kernel_t(M, N, K, ad.data_ptr(), lda, la, bd.data_ptr(), ldb, lb, cd.data_ptr(), ldc,
                                       lc, in_dt, out_dt, cid)
    G.say(f"[case] {label} {M}x{N}x{K} lay={lay} in={in_dt} out={out_dt} alpha={alpha} beta={beta} "
          f"bias={bias_kind}/{bias_dt} act={act} -> {KIND.get(kind, kind)} cfg{cfg}")
    T.gemm_tensors(ad, bd, cd, config_id=cid, alpha=alpha, beta=beta, bias=bv, bias_kind=bias_kind, activation=act)
    torch.cuda.synchronize()
    return G.values(cd, out_dt), kind


def expected(a, b, in_dt, out_dt, c_old, bias, bias_dt, bias_kind, alpha, beta, act):
    kw = dict(alpha=alpha, beta=beta, c_old=c_old, out_dtype=out_dt, bias=bias, bias_dtype=bias_dt,
              bias_kind=bias_kind if bias is not None else oracle.BIAS_NONE, nthreads=G.NTHREADS)
    o = oracle.gemm_fused(a, b, in_dt, act=act, **kw)
    z = oracle.gemm_fused(a, b, in_dt, act=oracle.ACT_NONE, **kw)
    return o, z


def check_bound(d, o, z, a, b, in_dt, out_dt, c_old, bias, bias_dt, bias_kind, alpha, beta, label):
    K = a.shape[1]
    p = G.oracle_values(a, b, in_dt)
    s = oracle.gemm(G.abs_storage(a, in_dt), G.abs_storage(b, in_dt), in_dt, nthreads=G.NTHREADS)
    ku = K * U32
    bp = (ku / (1 - ku)) * s
    cterm = np.abs(beta * oracle.decode(np.ascontiguousarray(c_old), out_dt)) if beta != 0 else 0.0
    if bias is None:
        bterm = 0.0
    else:
        bvals = oracle.decode(np.ascontiguousarray(bias), bias_dt)
        bterm = np.abs(bvals)[:, None] if bias_kind == oracle.BIAS_ROW else np.abs(bvals)[None, :]
    bz = abs(alpha) * bp + 3 * U32 * (np.abs(alpha * p) + cterm + bterm)
    u_out = G.U_OUT[out_dt]
    half_sub = {W.F32: 2.0 ** -150, W.F16: 2.0 ** -25, W.BF16: 2.0 ** -134}[out_dt]
    bound = (SLOPE * bz + 16 * U32 * (np.abs(o) + np.abs(z))) * (1 + u_out) + u_out * np.abs(o) + half_sub + 1e-30
    assert np.isfinite(d).all(), f"{label}: non-finite outputs"
    diff = np.abs(d - o)
    bad = diff > bound
    assert not bad.any(), (f"{label}: {int(bad.sum())} entries beyond the bound, worst ratio "
                           f"{float((diff / bound).max()):.3f}")
    return float((diff / bound).max())


# shapes and the kernel each takes (-1: the table's choice; a forced
# configuration otherwise, the path asserted): ring 256x256 tiles, ring
# 128x128 tiles, register-staged whole tiles (the 32x32 configuration), direct
SHAPES = [((256, 512, 384), "ring big", 0), ((1024, 2048, 512), "ring mid", 1), ((128, 256, 512), "tiled", 3),
          ((127, 255, 512), "direct", -1), ((33, 47, 255), "direct ragged", -1),
          ((1000, 1200, 512), "ring big ragged", 0), ((777, 1000, 256), "ring mid ragged", 1),
          ((1000, 1208, 1000), "ring big k tail", 0), ((300, 264, 200), "ring mid k tail", 1)]
EPILOGUES = [
    (1.0, 0.0, None, None, oracle.ACT_RELU),
    (0.5, 2.0, W.F32, oracle.BIAS_COL, oracle.ACT_NONE),
    (-1.5, 0.25, W.F16, oracle.BIAS_ROW, oracle.ACT_GELU),
    (2.0, 0.0, W.BF16, oracle.BIAS_COL, oracle.ACT_GELU_TANH),
    (1.0, -1.0, W.F32, oracle.BIAS_ROW, oracle.ACT_SILU),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: s[1].replace(" ", "_"))
@pytest.mark.parametrize("pair", [(W.F16, W.F16), (W.BF16, W.F32)], ids=["f16-f16", "bf16-f32"])
def test_fused_against_oracle(shape, pair):
    (M, N, K), name, cid = shape
    in_dt, out_dt = pair
    a, b = W.random_inputs(M, N, K, in_dt, seed=M + N + K)
    c_old = W.to_storage(np.random.default_rng(8).standard_normal((M, N)).astype(np.float32), out_dt)
    for alpha, beta, bias_dt, bias_kind, act in EPILOGUES:
        bias = None
        if bias_kind is not None:
            n = M if bias_kind == oracle.BIAS_ROW else N
            bias = W.to_storage(np.random.default_rng(9).standard_normal(n).astype(np.float32), bias_dt)
        d, kind = run_fused(a, b, in_dt, out_dt, c_old, bias, bias_dt, bias_kind, alpha, beta, act, cid=cid,
                            label=name)
        if name.startswith("ring"):
            assert kind == T.KERNEL_RING
        if name == "tiled":
            assert kind == T.KERNEL_TILED
        o, z = expected(a, b, in_dt, out_dt, c_old, bias, bias_dt, bias_kind, alpha, beta, act)
        r = check_bound(d, o, z, a, b, in_dt, out_dt, c_old, bias, bias_dt, bias_kind, alpha, beta, name)
        G.say(f"    ok, worst bound ratio {r:.3f}")


@pytest.mark.parametrize("lay", [(ROW, ROW, COL), (COL, ROW, ROW), (ROW, COL, COL), (COL, COL, COL)],
                         ids=lambda l: "".join("rc"[x] for x in l))
@pytest.mark.parametrize("shape", [(256, 512, 384), (127, 255, 512)], ids=["ring", "direct"])
def test_fused_layouts_bitwise(lay, shape):
    """Exact cases in other layouts: a row bias stays a bias per row of C
    when C is column-major (computed as C^T)."""
    M, N, K = shape
    a, b = W.integer_inputs(M, N, K, W.F16, seed=3)
    rng = np.random.default_rng(4)
    c_old = rng.integers(-8, 9, size=(M, N)).astype(np.float32)
    for bias_kind in (oracle.BIAS_ROW, oracle.BIAS_COL):
        bias = rng.integers(-50, 51, size=M if bias_kind == oracle.BIAS_ROW else N).astype(np.float32)
        for act in (oracle.ACT_NONE, oracle.ACT_RELU):
            d, _ = run_fused(a, b, W.F16, W.F32, c_old, bias, W.F32, bias_kind, 2.0, -0.5, act, lay=lay,
                             label="layout exact")
            o, _ = expected(a, b, W.F16, W.F32, c_old, bias, W.F32, bias_kind, 2.0, -0.5, act)
            assert np.array_equal(d, o), f"{int((d != o).sum())} entries differ"


@pytest.mark.parametrize("shape", [((300, 1030, 512), 1), ((1000, 1202, 1000), 0)], ids=["mid", "big_k_tail"])
def test_fused_ring_partial_groups(shape):
    """The fused epilogue on the ring kernel (forced, path asserted) with N %
    4 == 2 (a column-major B keeps the operands aligned) and ldc = N: the
    last group of each row is partial and the C rows are not 4-element
    aligned, in loads of the old C and in stores; exact integer case."""
    (M, N, K), cid = shape
    lay = (ROW, COL, ROW)
    a, b = W.integer_inputs(M, N, K, W.F16, seed=N)
    rng = np.random.default_rng(5)
    c_old = rng.integers(-8, 9, size=(M, N)).astype(np.float32)
    for bias_kind, act in ((oracle.BIAS_COL, oracle.ACT_RELU), (oracle.BIAS_ROW, oracle.ACT_NONE)):
        bias = rng.integers(-50, 51, size=M if bias_kind == oracle.BIAS_ROW else N).astype(np.float32)
        d, kind = run_fused(a, b, W.F16, W.F32, c_old, bias, W.F32, bias_kind, 2.0, -0.5, act, lay=lay, cid=cid,
                            label="ring partial groups")
        assert kind == T.KERNEL_RING
        o, _ = expected(a, b, W.F16, W.F32, c_old, bias, W.F32, bias_kind, 2.0, -0.5, act)
        assert np.array_equal(d, o), f"{int((d != o).sum())} entries differ"


@pytest.mark.parametrize("cid", range(8))
def test_fused_every_configuration_bitwise(cid):
    """Every configuration (forced), exact integer case, fp16 output."""
    info = T.gemm_config_info(cid)
    in_dt = W.F32 if info["in_dtype"] == T.F32 else W.F16
    out_dt = W.F32 if in_dt == W.F32 else W.F16
    for M, N, K in ((256, 256, 256), (200, 136, 72)):
        a, b = W.integer_inputs(M, N, K, in_dt, seed=cid + M)
        rng = np.random.default_rng(cid)
        c_old = W.to_storage(rng.integers(-8, 9, size=(M, N)).astype(np.float32), out_dt)
        bias = rng.integers(-20, 21, size=N).astype(np.float32)
        d, kind = run_fused(a, b, in_dt, out_dt, c_old, bias, W.F32, oracle.BIAS_COL, 1.0, 1.0, oracle.ACT_RELU,
                            cid=cid, label=f"cfg{cid}")
        o, _ = expected(a, b, in_dt, out_dt, c_old, bias, W.F32, oracle.BIAS_COL, 1.0, 1.0, oracle.ACT_RELU)
        want = G.round_to(o, out_dt)
        assert np.array_equal(d, want), f"cfg{cid} {M}x{N}x{K}: {int((d != want).sum())} entries differ"


def test_beta_zero_does_not_read_c():
    """beta = 0: NaN and Inf in C must not reach the result."""
    for M, N, K in ((256, 512, 384), (128, 256, 512), (127, 255, 512)):
        a, b = W.integer_inputs(M, N, K, W.F16, seed=5)
        c_old = np.full((M, N), np.nan, np.float16)
        c_old[::7, ::5] = np.inf
        d, kind = run_fused(a, b, W.F16, W.F16, c_old, None, None, None, 1.0, 0.0, oracle.ACT_RELU,
                            label="beta 0, NaN in C")
        o, _ = expected(a, b, W.F16, W.F16, c_old, None, None, None, 1.0, 0.0, oracle.ACT_RELU)
        assert np.array_equal(d, G.round_to(o, W.F16))


def test_k_zero_fused():
    """K = 0: C := act(beta C + bias)."""
    M, N = 37, 45
    a = torch.empty((M, 0), dtype=torch.float16, device=G.DEV)
    b = torch.empty((0, N), dtype=torch.float16, device=G.DEV)
    c_host = np.arange(M * N, dtype=np.float32).reshape(M, N) - 800
    c = torch.from_numpy(c_host.copy()).to(G.DEV)
    bias = torch.arange(N, dtype=torch.float32, device=G.DEV)
    G.say("[case] K=0 fused")
    T.gemm_tensors(a, b, c, beta=0.5, bias=bias, activation=T.ACT_RELU)
    torch.cuda.synchronize()
    want = np.maximum(0.5 * c_host + np.arange(N, dtype=np.float32)[None, :], 0)
    assert np.array_equal(c.cpu().numpy(), want)


def test_fused_8192_sampled():
    """The 8192^3 workload with a column bias and the tanh gelu (ring kernel,
    256 x 256 tiles), checked on 64 x 64 sampled outputs."""
    w = W.WORKLOADS[4]
    a, b = W.make_inputs(w)
    bias = W.to_storage(np.random.default_rng(10).standard_normal(w.N).astype(np.float32), W.F16)
    ad, bd = G.to_device(a, W.F16), G.to_device(b, W.F16)
    cd = torch.empty((w.M, w.N), dtype=torch.float16, device=G.DEV)
    bv = vec_device(bias, W.F16)
    kind = T.gemm_select_kernel(w.M, w.N, w.K, ad.data_ptr(), w.K, bd.data_ptr(), w.N, cd.data_ptr(), w.N, W.F16,
                                W.F16)
    assert kind == T.KERNEL_RING
    G.say("[case] 8192^3 fused bias + gelu_tanh")
    T.gemm_tensors(ad, bd, cd, bias=bv, activation=T.ACT_GELU_TANH)
    torch.cuda.synchronize()
    rows = W.sample_indices(w.M, 64, w.seed + 500)
    cols = W.sample_indices(w.N, 64, w.seed + 600)
    d = G.values(cd, W.F16)[np.ix_(rows, cols)]
    kw = dict(bias=bias, bias_dtype=W.F16, bias_kind=oracle.BIAS_COL, rows=rows, cols=cols, nthreads=G.NTHREADS)
    o = oracle.gemm_fused(a, b, W.F16, act=oracle.ACT_GELU_TANH, **kw)
    z = oracle.gemm_fused(a, b, W.F16, act=oracle.ACT_NONE, **kw)
    p = oracle.gemm(a, b, W.F16, rows=rows, cols=cols, nthreads=G.NTHREADS)
    s = oracle.gemm(G.abs_storage(a, W.F16), G.abs_storage(b, W.F16), W.F16, rows=rows, cols=cols,
                    nthreads=G.NTHREADS)
    ku = w.K * U32
    bz = (ku / (1 - ku)) * s + 3 * U32 * (np.abs(p) + np.abs(z - p))
    bound = (SLOPE * bz + 16 * U32 * (np.abs(o) + np.abs(z))) * (1 + 2.0 ** -11) + 2.0 ** -11 * np.abs(o) + 2.0 ** -25
    assert (np.abs(d - o) <= bound).all(), float((np.abs(d - o) / bound).max())
