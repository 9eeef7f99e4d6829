"""Pins of the oracle: checks of oracle/ against facts that do not come from
the oracle itself (the bit-level definitions as numpy implements them, exact
rational arithmetic, closed forms, an independent BLAS product and the pages'
own worked example).

Every pin is a plain function `pin_xxx(lib_path)` that raises AssertionError
on failure, so that the same pins can be run against the real oracle
(tests/test_oracle.py) and against copies of it with a planted mistake
(tests/test_oracle_mutants.py), where at least one pin must fail.
"""
import ctypes
import os
from fractions import Fraction

import numpy as np

import oracle
from tiled_gemm_03_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
U = 2.0 ** -53


# ---------------------------------------------------------------- helpers
def np_values(x: np.ndarray, dtype: int) -> np.ndarray:
    """binary64 values of stored elements, computed by numpy (independent of
    the oracle's decoders)."""
    if dtype == W.BF16:
        with np.errstate(invalid="ignore"):
            return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def summation_bound(av: np.ndarray, bv: np.ndarray) -> np.ndarray:
    """Elementwise bound on |s_oracle - s_other| for two binary64 sums of the
    same exact products in different orders: each is within (K-1)*u*sum|terms|
    of the exact value (standard recursive-summation bound)."""
    K = av.shape[1]
    return 2.0 * max(K - 1, 0) * U * (np.abs(av) @ np.abs(bv)) * (1 + 1e-6) + 0.0


def _exact(av, bv):
    """Exact product in rationals (brute force)."""
    M, K = av.shape
    N = bv.shape[1]
    out = [[Fraction(0)] * N for _ in range(M)]
    for i in range(M):
        for j in range(N):
            s = Fraction(0)
            for k in range(K):
                s += Fraction(float(av[i, k])) * Fraction(float(bv[k, j]))
            out[i][j] = s
    return out


# ------------------------------------------------------------ decoder pins
def pin_decode_binary16_exhaustive(lib_path=None):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode(bits, W.F16, lib_path=lib_path)
    want = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan), "binary16 NaN set differs"
    assert np.array_equal(got[~nan], want[~nan]), "binary16 decode differs"
    # signed zeros keep their sign
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def pin_decode_bfloat16_exhaustive(lib_path=None):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode(bits, W.BF16, lib_path=lib_path)
    want = np_values(bits, W.BF16)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan), "bfloat16 NaN set differs"
    assert np.array_equal(got[~nan], want[~nan]), "bfloat16 decode differs"


def pin_decode_binary32_sampled(lib_path=None):
    rng = np.random.default_rng(123)
    bits = rng.integers(0, 2 ** 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    specials = np.array([0, 0x80000000, 1, 0x807FFFFF, 0x00800000, 0x7F7FFFFF,
                         0x7F800000, 0xFF800000, 0x3F800000, 0xBF800000], dtype=np.uint32)
    bits = np.concatenate([bits, specials])
    got = oracle.decode(bits, W.F32, lib_path=lib_path)
    with np.errstate(invalid="ignore"):
        want = bits.view(np.float32).astype(np.float64)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan]), "binary32 decode differs"


# ------------------------------------------------- 8-bit output formats
# The OCP 8-bit formats the fused epilogue can write (E4M3: largest finite
# 448, no infinity; E5M2: largest finite 57344).  torch's float8_e4m3fn and
# float8_e5m2 are the same formats and an independent implementation of
# their decoding and of the nearest-even rounding of in-range values; above
# the largest finite value torch does not saturate (NaN / infinity), which is
# pinned separately against closed forms.
FP8 = ((oracle.FP8_E4M3, "float8_e4m3fn", 448.0, 0x7E), (oracle.FP8_E5M2, "float8_e5m2", 57344.0, 0x7B))


def pin_decode_fp8_exhaustive(lib_path=None):
    import torch
    bits = np.arange(256, dtype=np.uint8)
    for fmt, tname, _, _ in FP8:
        got = oracle.decode(bits, fmt, lib_path=lib_path)
        want = torch.from_numpy(bits).view(getattr(torch, tname)).to(torch.float64).numpy()
        nan = np.isnan(want)
        assert np.array_equal(np.isnan(got), nan), f"{tname}: NaN set differs"
        assert np.array_equal(got[~nan], want[~nan]), f"{tname}: decode differs"
        assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan])), f"{tname}: sign of zero"


def pin_encode_fp8_vs_torch(lib_path=None):
    """Every finite pattern encodes back to itself; every midpoint between
    neighbouring values, the binary32 values just either side of it, and
    random binary32 values within the finite range round as torch rounds."""
    import torch
    bits = np.arange(256, dtype=np.uint8)
    rng = np.random.default_rng(77)
    for fmt, tname, mx, _ in FP8:
        vals = oracle.decode(bits, fmt, lib_path=lib_path)
        fin = np.isfinite(vals)
        back = oracle.encode_fp8(vals[fin], fmt, lib_path=lib_path)
        assert np.array_equal(back, bits[fin]), f"{tname}: a value does not encode to its own pattern"
        pos = np.unique(vals[fin & (vals >= 0)])
        mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)
        x = np.concatenate([mids, np.nextafter(mids, np.float32(np.inf)), np.nextafter(mids, np.float32(0)),
                            rng.uniform(-mx, mx, 4000).astype(np.float32),
                            (rng.standard_normal(2000) * 2.0 ** rng.integers(-20, 8, 2000)).astype(np.float32)])
        x = x[np.abs(x) <= mx]
        x = np.concatenate([x, -x])
        want = torch.from_numpy(x).to(getattr(torch, tname)).view(torch.uint8).numpy()
        got = oracle.encode_fp8(x.astype(np.float64), fmt, lib_path=lib_path)
        bad = got != want
        assert not bad.any(), f"{tname}: {int(bad.sum())} roundings differ, e.g. {x[bad][:4]}"


def pin_encode_fp8_saturation_and_ties(lib_path=None):
    """Closed forms: beyond the largest finite value (infinity included) the
    largest finite value of the sign; NaN the all-ones pattern; ties to the
    even fraction, in the subnormal range too."""
    for fmt, tname, mx, top in FP8:
        enc = lambda v: int(oracle.encode_fp8(np.array([v], dtype=np.float64), fmt, lib_path=lib_path)[0])
        for v in (mx * 1.0001, mx * 1.5, 1e30, np.inf):
            assert enc(v) == top and enc(-v) == 0x80 | top, (tname, v)
        assert enc(np.nan) & 0x7F == 0x7F
        assert enc(0.0) == 0 and enc(-0.0) == 0x80
        # subnormal spacing 2^(1 - bias - F)
        q = 2.0 ** (-9 if fmt == oracle.FP8_E4M3 else -16)
        assert enc(0.5 * q) == 0 and enc(1.5 * q) == 2 and enc(2.5 * q) == 2 and enc(0.5000001 * q) == 1
        # 1 + half a spacing of [1, 2) lies between 1 (even) and the next value
        F = 3 if fmt == oracle.FP8_E4M3 else 2
        one = enc(1.0)
        assert enc(1.0 + 2.0 ** -(F + 1)) == one and enc(1.0 + 3 * 2.0 ** -(F + 1)) == one + 2


# --------------------------------------------------------- product pins
def pin_identity(lib_path=None):
    """I x B == B and A x I == A exactly (closed form), every input type,
    non-square so that a transposed operand cannot hide."""
    for dt in (W.F32, W.F16, W.BF16):
        a, b = W.random_inputs(37, 53, 37, dt, seed=11)
        eye = W.to_storage(np.eye(37, dtype=np.float32), dt)
        got = oracle.gemm(eye, b, dt, lib_path=lib_path)
        assert np.array_equal(got, np_values(b, dt)), f"I x B != B for dtype {dt}"
        eye2 = W.to_storage(np.eye(53, dtype=np.float32), dt)
        a2, _ = W.random_inputs(29, 53, 53, dt, seed=12)
        got = oracle.gemm(a2, eye2, dt, lib_path=lib_path)
        assert np.array_equal(got, np_values(a2, dt)), f"A x I != A for dtype {dt}"


def pin_all_ones(lib_path=None):
    """Every entry of ones(M,K) x ones(K,N) is K (closed form), including the
    empty sum K = 0."""
    for dt in (W.F32, W.F16, W.BF16):
        for (M, N, K) in ((3, 5, 0), (7, 9, 1), (17, 33, 257), (4, 4, 2051)):
            a = W.to_storage(np.ones((M, K), np.float32), dt)
            b = W.to_storage(np.ones((K, N), np.float32), dt)
            got = oracle.gemm(a, b, dt, lib_path=lib_path)
            assert got.shape == (M, N)
            assert np.all(got == K), f"ones product != K at {(M, N, K)}"


def pin_golden_ones_8x8(lib_path=None):
    with open(os.path.join(GOLDEN, "ones_8x8.txt"), encoding="utf-8") as f:
        rows = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    M, N, K = map(int, rows[0])
    want = np.array(rows[1:], dtype=np.float64)
    for dt in (W.F32, W.F16):
        a = W.to_storage(np.ones((M, K), np.float32), dt)
        b = W.to_storage(np.ones((K, N), np.float32), dt)
        assert np.array_equal(oracle.gemm(a, b, dt, lib_path=lib_path), want)


def pin_bruteforce_rational(lib_path=None):
    """Small products against exact rational arithmetic (4x4x4 and a
    non-square 3x5x7), within the binary64 summation bound."""
    for dt in (W.F32, W.F16, W.BF16):
        for (M, N, K, seed) in ((4, 4, 4, 21), (3, 5, 7, 22)):
            a, b = W.random_inputs(M, N, K, dt, seed=seed)
            av, bv = np_values(a, dt), np_values(b, dt)
            ex = _exact(av, bv)
            got = oracle.gemm(a, b, dt, lib_path=lib_path)
            for i in range(M):
                for j in range(N):
                    terms = sum(abs(Fraction(float(av[i, k])) * Fraction(float(bv[k, j])))
                                for k in range(K))
                    err = abs(Fraction(float(got[i, j])) - ex[i][j])
                    assert err <= (K - 1) * Fraction(U) * terms, \
                        f"entry ({i},{j}) off the exact value for dtype {dt}"


def _check_vs_numpy(a, b, dt, lib_path, rows=None, cols=None, nthreads=8):
    av, bv = np_values(a, dt), np_values(b, dt)
    if rows is not None:
        av = av[rows]
    if cols is not None:
        bv = bv[:, cols]
    want = av @ bv
    got = oracle.gemm(a, b, dt, rows=rows, cols=cols, nthreads=nthreads, lib_path=lib_path)
    bound = summation_bound(av, bv)
    bad = np.abs(got - want) > bound
    assert not bad.any(), f"{bad.sum()} entries differ from numpy's binary64 product"


def pin_vs_numpy_unaligned(lib_path=None):
    """127 x 255 x 512 (the non-aligned edge case) against numpy's binary64
    matrix product, an independent BLAS routine."""
    for dt in (W.F16, W.F32, W.BF16):
        a, b = W.random_inputs(127, 255, 512, dt, seed=3, dist="uniform")
        _check_vs_numpy(a, b, dt, lib_path)


def pin_vs_numpy_workloads(lib_path=None):
    """The four smaller workloads in full against numpy's binary64 product."""
    for w in W.WORKLOADS[:4]:
        a, b = W.make_inputs(w)
        _check_vs_numpy(a, b, w.in_dtype, lib_path)


def pin_sampled_equals_full(lib_path=None):
    """Sampled entries are bitwise the full result's entries."""
    a, b = W.random_inputs(127, 255, 64, W.F16, seed=31)
    full = oracle.gemm(a, b, W.F16, lib_path=lib_path)
    rows = np.array([0, 5, 126, 64, 3])
    cols = np.array([254, 0, 7, 100])
    got = oracle.gemm(a, b, W.F16, rows=rows, cols=cols, lib_path=lib_path)
    assert np.array_equal(got, full[rows][:, cols])


def pin_padded_leading_dimension(lib_path=None):
    """Operands whose rows are padded (ld > width) with NaN give the same
    result as tight ones: the padding is never read."""
    a, b = W.random_inputs(45, 70, 33, W.F16, seed=41)
    tight = oracle.gemm(a, b, W.F16, lib_path=lib_path)
    big_a = np.full((45, 40), np.nan, np.float16)
    big_a[:, :33] = a
    big_b = np.full((33, 77), np.nan, np.float16)
    big_b[:, :70] = b
    got = oracle.gemm(big_a[:, :33], big_b[:, :70], W.F16, lib_path=lib_path)
    assert np.array_equal(got, tight)


def pin_threads_invariant(lib_path=None):
    a, b = W.random_inputs(50, 60, 300, W.F16, seed=51)
    one = oracle.gemm(a, b, W.F16, nthreads=1, lib_path=lib_path)
    many = oracle.gemm(a, b, W.F16, nthreads=7, lib_path=lib_path)
    assert np.array_equal(one, many)


def pin_output_overwritten(lib_path=None):
    """An output buffer pre-filled with NaN is fully overwritten, with the
    correct values (small integer inputs make every sum exact)."""
    lib = oracle._load(lib_path)
    a, b = W.integer_inputs(9, 11, 13, W.F16, seed=61)
    want = np_values(a, W.F16) @ np_values(b, W.F16)
    out = np.full((9, 11), np.nan)
    rc = lib.oracle_gemm(9, 11, 13, a.ctypes.data, 13, b.ctypes.data, 11, W.F16,
                         None, 0, None, 0, out.ctypes.data, 11, 2)
    assert rc == 0
    assert np.array_equal(out, want)


def pin_large_sampled(lib_path=None):
    """The 8192^3 workload: 64 seeded rows x 64 seeded columns against numpy
    on the same slices."""
    w = W.WORKLOADS[4]
    a, b = W.make_inputs(w)
    rows = W.sample_indices(w.M, 64, w.seed + 100)
    cols = W.sample_indices(w.N, 64, w.seed + 200)
    _check_vs_numpy(a, b, w.in_dtype, lib_path, rows=rows, cols=cols)


def pin_rejects_bad_arguments(lib_path=None):
    lib = oracle._load(lib_path)
    out = np.zeros(4)
    a = np.zeros(4, np.float16)
    for args in ((-1, 2, 2, 2, 2), (2, 2, 2, 1, 2), (2, 2, 2, 2, 1)):
        M, N, K, lda, ldb = args
        rc = lib.oracle_gemm(M, N, K, a.ctypes.data, lda, a.ctypes.data, ldb, W.F16,
                             None, 0, None, 0, out.ctypes.data, 2, 1)
        assert rc == -1, args
    rc = lib.oracle_gemm(2, 2, 2, a.ctypes.data, 2, a.ctypes.data, 2, 7,
                         None, 0, None, 0, out.ctypes.data, 2, 1)
    assert rc == -1
    bad_rows = np.array([2], dtype=np.int64)
    rc = lib.oracle_gemm(2, 2, 2, a.ctypes.data, 2, a.ctypes.data, 2, W.F16,
                         bad_rows.ctypes.data, 1, None, 0, out.ctypes.data, 2, 1)
    assert rc == -1


# ------------------------------------------------------------ epilogue pins
def pin_activations_vs_torch(lib_path=None):
    """Each activation on a grid of points against torch.nn.functional in
    float64 on the CPU (an independent library implementation)."""
    import torch
    import torch.nn.functional as F
    x = np.concatenate([np.linspace(-8.0, 8.0, 161), [0.0, -0.0, 1e-8, -1e-8, 30.0, -30.0, 3.5, -0.7]])
    t = torch.from_numpy(x)
    refs = {oracle.ACT_NONE: t, oracle.ACT_RELU: F.relu(t), oracle.ACT_GELU: F.gelu(t, approximate="none"),
            oracle.ACT_GELU_TANH: F.gelu(t, approximate="tanh"), oracle.ACT_SILU: F.silu(t)}
    for act, ref in refs.items():
        got = oracle.activation(x, act, lib_path=lib_path)
        want = ref.numpy()
        # the two libraries round their constants and intermediate steps differently
        assert np.allclose(got, want, rtol=1e-13, atol=1e-14), (act, np.max(np.abs(got - want)))


def pin_activation_constants(lib_path=None):
    """Published values: Phi(1) = 0.8413447460685429 (standard normal table),
    so gelu(1) = Phi(1) and gelu(-1) = -(1 - Phi(1)); the logistic function
    at 1 is 1 / (1 + 1/e) = 0.7310585786300049; the tanh form of gelu differs
    from gelu by less than 1e-3 everywhere."""
    act = lambda v, a: float(oracle.activation(np.array([v]), a, lib_path=lib_path)[0])
    assert abs(act(1.0, oracle.ACT_GELU) - 0.8413447460685429) < 1e-15
    assert abs(act(-1.0, oracle.ACT_GELU) + 0.15865525393145707) < 1e-15
    assert abs(act(1.0, oracle.ACT_SILU) - 0.7310585786300049) < 1e-15
    assert abs(act(-1.0, oracle.ACT_SILU) + 0.2689414213699951) < 1e-15
    assert act(-3.0, oracle.ACT_RELU) == 0.0 and act(3.0, oracle.ACT_RELU) == 3.0 and act(-3.0, oracle.ACT_NONE) == -3.0
    xs = np.linspace(-6, 6, 241)
    d = oracle.activation(xs, oracle.ACT_GELU_TANH, lib_path=lib_path) - oracle.activation(xs, oracle.ACT_GELU,
                                                                                        lib_path=lib_path)
    assert np.max(np.abs(d)) < 1e-3 and np.max(np.abs(d)) > 1e-5


def pin_epilogue_worked_example(lib_path=None):
    """A 2 x 2 x 4 all-ones product (every entry 4) through the epilogue,
    with values worked out by hand: alpha = 0.5 -> 2; beta = 3 times
    C_old = [[1, 2], [3, 4]]; a column bias [10, -20] or a row bias
    [10, -20]; relu."""
    ones = np.ones((2, 4), np.float16)
    onesb = np.ones((4, 2), np.float16)
    c_old = np.array([[1, 2], [3, 4]], np.float16)
    bias = np.array([10, -20], np.float16)
    got = oracle.gemm_fused(ones, onesb, W.F16, alpha=0.5, beta=3.0, c_old=c_old, out_dtype=W.F16, bias=bias,
                            bias_dtype=W.F16, bias_kind=oracle.BIAS_COL, act=oracle.ACT_RELU, lib_path=lib_path)
    assert np.array_equal(got, [[15.0, 0.0], [21.0, 0.0]]), got
    got = oracle.gemm_fused(ones, onesb, W.F16, alpha=0.5, beta=3.0, c_old=c_old, out_dtype=W.F16, bias=bias,
                            bias_dtype=W.F16, bias_kind=oracle.BIAS_ROW, act=oracle.ACT_NONE, lib_path=lib_path)
    assert np.array_equal(got, [[15.0, 18.0], [-9.0, -6.0]]), got
    # the activation comes last: relu(2 - 3) = 0, not relu(2) - 3
    got = oracle.gemm_fused(ones, onesb, W.F16, alpha=0.5, bias=np.array([-3, 1], np.float16), bias_dtype=W.F16,
                            bias_kind=oracle.BIAS_COL, act=oracle.ACT_RELU, lib_path=lib_path)
    assert np.array_equal(got, [[0.0, 3.0], [0.0, 3.0]]), got


def pin_epilogue_beta_zero_ignores_c(lib_path=None):
    """beta = 0: C is not read, so NaN or Inf stored there has no effect;
    with alpha = 1, no bias and no activation the epilogue is the product."""
    a, b = W.random_inputs(5, 7, 9, W.F16, seed=11)
    c_old = np.full((5, 7), np.nan, np.float16)
    c_old[0, 0] = np.inf
    p = oracle.gemm(a, b, W.F16, lib_path=lib_path)
    got = oracle.gemm_fused(a, b, W.F16, alpha=1.0, beta=0.0, c_old=c_old, out_dtype=W.F16, lib_path=lib_path)
    assert np.array_equal(got, p)
    got = oracle.gemm_fused(a, b, W.F16, alpha=-2.0, beta=0.0, c_old=c_old, out_dtype=W.F16, lib_path=lib_path)
    assert np.array_equal(got, -2.0 * p)


def pin_epilogue_sampled_equals_full(lib_path=None):
    a, b = W.random_inputs(20, 30, 40, W.BF16, seed=12)
    c_old = W.random_inputs(20, 30, 1, W.F32, seed=13)[0][:, :1].repeat(30, axis=1).astype(np.float32)
    bias = W.random_inputs(1, 30, 1, W.BF16, seed=14)[1].ravel()
    kw = dict(alpha=1.5, beta=-0.25, c_old=c_old, out_dtype=W.F32, bias=bias, bias_dtype=W.BF16,
              bias_kind=oracle.BIAS_COL, act=oracle.ACT_GELU_TANH, lib_path=lib_path)
    full = oracle.gemm_fused(a, b, W.BF16, **kw)
    rows, cols = np.array([0, 7, 19]), np.array([29, 3, 0, 11])
    part = oracle.gemm_fused(a, b, W.BF16, rows=rows, cols=cols, **kw)
    assert np.array_equal(part, full[np.ix_(rows, cols)])


def pin_epilogue_rejects_bad_arguments(lib_path=None):
    lib = oracle._load(lib_path)
    s = np.zeros(4)
    out = np.zeros(4)
    assert lib.oracle_epilogue(2, 2, s.ctypes.data, 2, 1.0, 0.0, None, 2, None, None, 9, out.ctypes.data, 2) == -1
    assert lib.oracle_epilogue(2, 2, s.ctypes.data, 2, 1.0, 1.0, None, 2, None, None, 0, out.ctypes.data, 2) == -1
    assert lib.oracle_epilogue(2, 2, s.ctypes.data, 2, 1.0, 0.0, None, 2, s.ctypes.data, s.ctypes.data, 0,
                               out.ctypes.data, 2) == -1
    assert lib.oracle_epilogue(2, 2, s.ctypes.data, 1, 1.0, 0.0, None, 2, None, None, 0, out.ctypes.data, 2) == -1


# Pins cheap enough to run against every planted mistake.
FAST_PINS = [
    pin_decode_binary16_exhaustive,
    pin_decode_bfloat16_exhaustive,
    pin_decode_binary32_sampled,
    pin_decode_fp8_exhaustive,
    pin_encode_fp8_vs_torch,
    pin_encode_fp8_saturation_and_ties,
    pin_identity,
    pin_all_ones,
    pin_golden_ones_8x8,
    pin_bruteforce_rational,
    pin_vs_numpy_unaligned,
    pin_sampled_equals_full,
    pin_padded_leading_dimension,
    pin_threads_invariant,
    pin_output_overwritten,
    pin_rejects_bad_arguments,
    pin_activations_vs_torch,
    pin_activation_constants,
    pin_epilogue_worked_example,
    pin_epilogue_beta_zero_ignores_c,
    pin_epilogue_sampled_equals_full,
    pin_epilogue_rejects_bad_arguments,
]
ALL_PINS = FAST_PINS + [pin_vs_numpy_workloads, pin_large_sampled]
