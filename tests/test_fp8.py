"""GPU parity of the 8-bit floating-point outputs (TGEMM_FP8_E4M3 /
TGEMM_FP8_E5M2) against the oracle: the output rounding of the fused
epilogue of page "企业官网建设流程全解析" §6.2 taken to the OCP 8-bit formats
(nearest, ties to even; saturating at the largest finite value; NaN stays
NaN).

1. Bit for bit where the fp32 value before the rounding is exact: integer
   inputs in [-2, 2] (every partial sum exact in fp32), alpha a power of two
   (2^-4 puts many results between representable 8-bit values, so the
   rounding decides them), integer C and bias: the GPU pattern must equal
   the oracle's binary64 result rounded by the oracle's own encoder.  Every
   kernel that writes 8-bit outputs (the three ring tiles, the direct
   kernel), the four operand-layout pairs, a column-major C, ragged edges, a
   K tail, partial column groups, both formats; many results of E4M3 are
   beyond 448 and saturate.
2. Elsewhere an element-wise bound: with t the kernel's fp32 value and o the
   exact one, |sat(fp8(t)) - clamp(o)| <= u8 |o| + (1 + u8) |t - o| + eta8
   (u8 = 2^-4 for E4M3, 2^-3 for E5M2: half the spacing relative to the
   value; eta8 half the smallest subnormal; clamp to the largest finite value
   is 1-Lipschitz), |t - o| bounded as in the fused-epilogue tests.
Every case prints its name and the kernel before it touches the GPU.
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
KIND = {T.KERNEL_GENERAL: "general", T.KERNEL_TILED: "tiled", T.KERNEL_RING: "ring", T.KERNEL_DIRECT: "direct"}
FMTS = {T.FP8_E4M3: (torch.float8_e4m3fn, 448.0, 2.0 ** -4, 2.0 ** -10),
        T.FP8_E5M2: (torch.float8_e5m2, 57344.0, 2.0 ** -3, 2.0 ** -17)}
U32 = 2.0 ** -24
SLOPE = 1.2


def place(x, dt, layout):
    if layout == ROW:
        return G.to_device(x, dt)
    return G.to_device(np.ascontiguousarray(x.T), dt).t()


def fp8_tensor(bits, fmt, layout=ROW, pad=0, fill=0x7F):
    """Device 8-bit tensor holding `bits` (M x N), row- or column-major, with
    `pad` extra elements per row (or column) filled with `fill`."""
    tdt = FMTS[fmt][0]
    M, N = bits.shape
    src = bits if layout == ROW else np.ascontiguousarray(bits.T)
    r, c = src.shape
    full = np.full((r, c + pad), fill, np.uint8)
    full[:, :c] = src
    t = torch.from_numpy(full).view(tdt).to(G.DEV)[:, :c]
    return t if layout == ROW else t.t()


def fp8_bits(t):
    """uint8 patterns of a device 8-bit tensor (logical M x N)."""
    return t.detach().cpu().contiguous().view(torch.uint8).numpy()


def vec_device(v, dt):
    host = torch.from_numpy(np.ascontiguousarray(v).view(np.int16)).view(torch.bfloat16) if dt == W.BF16 \
        else torch.from_numpy(np.ascontiguousarray(v))
    return host.to(G.DEV)


def run(a, b, in_dt, fmt, c_old_bits, lay=(ROW, ROW, ROW), cid=-1, label="", **epi):
    M, K = a.shape
    N = b.shape[1]
    ad, bd = place(a, in_dt, lay[0]), place(b, in_dt, lay[1])
    cd = fp8_tensor(c_old_bits, fmt, lay[2])
    la, lda = T._layout(ad)
    lb, ldb = T._layout(bd)
    lc, ldc = T._layout(cd)
    kind, cfg = T.gemm_select_kernel_t(M, N, K, ad.data_ptr(), lda, la, bd.data_ptr(), ldb, lb, cd.data_ptr(), ldc,
                                       lc, in_dt, fmt, cid)
    G.say(f"[case] fp8 {label} {M}x{N}x{K} lay={lay} in={in_dt} fmt={fmt} {epi if epi else ''} "
          f"-> {KIND.get(kind, kind)} cfg{cfg}")
    assert kind >= 0, f"rejected: {T.gemm_strerror(kind)}"
    if "bias" in epi and epi["bias"] is not None:
        epi = dict(epi)
        epi["bias"] = vec_device(epi["bias"], epi.pop("bias_dt"))
    else:
        epi.pop("bias_dt", None)
    T.gemm_tensors(ad, bd, cd, config_id=cid, **epi)
    torch.cuda.synchronize()
    return fp8_bits(cd), kind


# shapes that take each kernel writing 8-bit outputs (forced configuration,
# path asserted): ring 256 x 256, 128 x 128, 64 x 128, direct; ragged edges
# and K tails (partial column groups: test_fp8_plain_product_and_partial_groups)
SHAPES = [((256, 512, 384), 0, "ring big"), ((384, 256, 256), 1, "ring mid"), ((192, 384, 256), 8, "ring small"),
          ((127, 255, 512), 6, "direct"), ((1000, 1200, 512), 0, "ring big ragged"),
          ((300, 520, 1000), 1, "ring mid k tail"), ((200, 384, 296), 8, "ring small ragged k tail"),
          ((33, 47, 255), 6, "direct ragged")]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: s[2].replace(" ", "_"))
@pytest.mark.parametrize("fmt", [T.FP8_E4M3, T.FP8_E5M2], ids=["e4m3", "e5m2"])
def test_fp8_exact(shape, fmt):
    (M, N, K), cid, name = shape
    for in_dt in (W.F16, W.BF16):
        a, b = W.integer_inputs(M, N, K, in_dt, seed=M + K + fmt)
        rng = np.random.default_rng(N)
        c_old = oracle.encode_fp8(rng.integers(-8, 9, size=(M, N)).astype(np.float64), fmt)
        bias = rng.integers(-30, 31, size=N).astype(np.float32)
        for alpha, beta, act in ((0.0625, 0.0, T.ACT_NONE), (1.0, 0.5, T.ACT_RELU)):
            d, kind = run(a, b, in_dt, fmt, c_old, cid=cid, label=name, alpha=alpha, beta=beta, bias=bias,
                          bias_dt=W.F32, activation=act)
            assert kind == (T.KERNEL_DIRECT if cid == 6 else T.KERNEL_RING)
            o = oracle.gemm_fused(a, b, in_dt, alpha=alpha, beta=beta, c_old=c_old, out_dtype=fmt, bias=bias,
                                  bias_dtype=W.F32, bias_kind=oracle.BIAS_COL, act=act, nthreads=G.NTHREADS)
            want = oracle.encode_fp8(o, fmt)
            assert np.array_equal(d, want), f"{name}: {int((d != want).sum())} patterns differ"


@pytest.mark.parametrize("lay", [(ROW, COL, ROW), (COL, ROW, ROW), (COL, COL, COL), (ROW, ROW, COL)],
                         ids=lambda l: "".join("rc"[x] for x in l))
def test_fp8_layouts_exact(lay):
    """Other operand layouts and a column-major C (computed as C^T), on the
    ring (aligned) and the direct kernel (ragged, unaligned rows)."""
    for (M, N, K), cid in (((256, 512, 384), -1), ((130, 250, 200), 6)):
        for fmt in (T.FP8_E4M3, T.FP8_E5M2):
            a, b = W.integer_inputs(M, N, K, W.F16, seed=7 + fmt)
            c_old = np.zeros((M, N), np.uint8)
            d, _ = run(a, b, W.F16, fmt, c_old, lay=lay, cid=cid, label="layouts", alpha=0.125)
            o = oracle.gemm_fused(a, b, W.F16, alpha=0.125, nthreads=G.NTHREADS)
            assert np.array_equal(d, oracle.encode_fp8(o, fmt))


def test_fp8_plain_product_and_partial_groups():
    """gemm_t (no epilogue) with an 8-bit output: the identity epilogue; N %
    4 == 2 with ldc = N (partial last groups, C rows not 4-byte aligned)."""
    for (M, N, K), lay in (((256, 256, 256), (ROW, ROW, ROW)), ((300, 1030, 512), (ROW, COL, ROW)),
                           ((64, 70, 40), (ROW, ROW, ROW))):
        for fmt in (T.FP8_E4M3, T.FP8_E5M2):
            a, b = W.integer_inputs(M, N, K, W.BF16, seed=N)
            d, _ = run(a, b, W.BF16, fmt, np.full((M, N), 0x7F, np.uint8), lay=lay, label="plain")
            o = oracle.gemm(a, b, W.BF16, nthreads=G.NTHREADS)
            assert np.array_equal(d, oracle.encode_fp8(o, fmt))


def test_fp8_unaligned_operands():
    """Operands whose rows are not whole 16-byte chunks (rows of an odd K,
    contiguous) with an 8-bit output, through the ring's fused epilogue: the
    last element of A ending at a 4 KiB page boundary (loaded on its own in
    the K tail), a padded range, one padding element per row.  The
    register-staged tiles the table would take without the ring write no
    8-bit output; that routing (to the direct kernel) is checked on the host
    with an odd address."""
    M, N, K = 1024, 1024, 301   # without the ring: the 64 x 64 register-staged tile
    a, b = W.integer_inputs(M, N, K, W.F16, seed=3)
    o = oracle.gemm_fused(a, b, W.F16, alpha=0.25, nthreads=G.NTHREADS)
    bd = G.to_device(b, W.F16, pad_cols=3)           # ldb = 1027
    n = M * K
    flat = torch.full((n + 4096 + 8,), float("nan"), dtype=torch.float16, device=G.DEV)
    at_page = ((-(flat.data_ptr() + 2 * n)) % 4096) // 2
    placements = [("A ends at a page", flat[at_page:at_page + n].view(M, K), K, T.KERNEL_RING),
                  ("A padded range", flat[at_page + 2:at_page + 2 + n].view(M, K), K, T.KERNEL_RING),
                  ("lda 302", G.to_device(a, W.F16, pad_cols=1), K + 1, T.KERNEL_RING)]
    for label, ad, lda, want_kind in placements:
        if lda == K:
            ad.copy_(torch.from_numpy(a).to(G.DEV))
        cd = fp8_tensor(np.full((M, N), 0x7F, np.uint8), T.FP8_E4M3)
        kind = T.gemm_select_kernel_t(M, N, K, ad.data_ptr(), lda, ROW, bd.data_ptr(), N + 3, ROW,
                                      cd.data_ptr(), N, ROW, W.F16, T.FP8_E4M3, -1)[0]
        G.say(f"[case] fp8 unaligned operands, {label} -> {KIND.get(kind, kind)}")
        assert kind == want_kind
        T.gemm_tensors(ad, bd, cd, alpha=0.25)
        torch.cuda.synchronize()
        assert np.array_equal(fp8_bits(cd), oracle.encode_fp8(o, T.FP8_E4M3))


@pytest.mark.parametrize("shape", [(256, 512, 256, -1), (100, 72, 40, 6)], ids=["ring", "direct"])
def test_fp8_nan_and_infinity(shape):
    """A NaN in row 0 of A makes row 0 of C NaN: an 8-bit NaN pattern (E4M3
    S.1111.111, E5M2 exponent 31 with a nonzero fraction; the sign of a NaN
    the arithmetic makes is not defined).  An infinity in row 1 of A, times
    a row of B that is all ones, makes row 1 +infinity: the largest finite
    value (saturating).  The other rows against the oracle, exactly."""
    M, N, K, cid = shape
    a, b = W.integer_inputs(M, N, K, W.F16, seed=21)
    a[0, 3] = np.float16(np.nan)
    a[1, 0] = np.float16(np.inf)
    b[0, :] = np.float16(1.0)
    ad, bd = G.to_device(a, W.F16), G.to_device(b, W.F16)
    rest = np.ascontiguousarray(a[2:])
    o = oracle.gemm_fused(rest, b, W.F16, alpha=0.5, nthreads=G.NTHREADS)
    for fmt, top in ((T.FP8_E4M3, 0x7E), (T.FP8_E5M2, 0x7B)):
        cd = fp8_tensor(np.zeros((M, N), np.uint8), fmt)
        kind = T.gemm_select_kernel(M, N, K, ad.data_ptr(), K, bd.data_ptr(), N, cd.data_ptr(), N, W.F16, fmt, cid)
        G.say(f"[case] fp8 NaN / infinity {M}x{N}x{K} fmt={fmt} -> {KIND.get(kind, kind)}")
        T.gemm_tensors(ad, bd, cd, config_id=cid, alpha=0.5)
        torch.cuda.synchronize()
        got = fp8_bits(cd)
        mag = got[0] & 0x7F
        if fmt == T.FP8_E4M3:
            assert (mag == 0x7F).all(), np.unique(got[0])
        else:
            assert ((mag >> 2) == 0x1F).all() and ((mag & 3) != 0).all(), np.unique(got[0])
        assert (got[1] == top).all(), np.unique(got[1])
        assert np.array_equal(got[2:], oracle.encode_fp8(o, fmt))


@pytest.mark.parametrize("cid", [1, 6], ids=["ring", "direct"])
def test_fp8_every_half_value(cid):
    """Every fp16 bit pattern through the output conversion: C = alpha A B
    with A's column 0 holding all 65536 patterns (the other columns zero) and
    B's row 0 all ones, so each row of C is alpha times one fp16 value,
    exact in fp32 (alpha 1, 2^-8, 3; -0 sums to +0).  Each 8-bit pattern
    must equal the oracle's rounding of that value (nearest even,
    saturating), NaN inputs an 8-bit NaN; both formats, a ring and the
    direct kernel."""
    M, N, K = 65536, 16, 128
    col = np.arange(65536, dtype=np.uint16).view(np.float16)
    a = np.zeros((M, K), np.float16)
    a[:, 0] = col
    b = np.zeros((K, N), np.float16)
    b[0, :] = 1.0
    ad, bd = G.to_device(a, W.F16), G.to_device(b, W.F16)
    nan = np.isnan(col.astype(np.float64))
    for fmt in (T.FP8_E4M3, T.FP8_E5M2):
        for alpha in (1.0, 2.0 ** -8, 3.0):
            cd = fp8_tensor(np.zeros((M, N), np.uint8), fmt)
            kind = T.gemm_select_kernel(M, N, K, ad.data_ptr(), K, bd.data_ptr(), N, cd.data_ptr(), N, W.F16, fmt,
                                        cid)
            G.say(f"[case] fp8 every fp16 value fmt={fmt} alpha={alpha} cfg{cid} -> {KIND.get(kind, kind)}")
            T.gemm_tensors(ad, bd, cd, config_id=cid, alpha=alpha)
            torch.cuda.synchronize()
            got = fp8_bits(cd)
            assert (got == got[:, :1]).all()
            # the product's value: alpha (a_i0 * 1 + the zero products): +0 for -0
            vals = np.where(nan, 0.0, col.astype(np.float64))
            want = oracle.encode_fp8(vals * alpha + 0.0, fmt)
            g0 = got[:, 0]
            assert np.array_equal(g0[~nan], want[~nan]), f"{int((g0[~nan] != want[~nan]).sum())} patterns differ"
            mag = g0[nan] & 0x7F
            if fmt == T.FP8_E4M3:
                assert (mag == 0x7F).all()
            else:
                assert ((mag >> 2) == 0x1F).all() and ((mag & 3) != 0).all()


def test_fp8_guard_band_and_k_zero():
    """Padding bytes after each row of C are untouched; K = 0 writes +0."""
    M, N, K = 200, 264, 256
    a, b = W.integer_inputs(M, N, K, W.F16, seed=9)
    ad, bd = G.to_device(a, W.F16), G.to_device(b, W.F16)
    full = torch.from_numpy(np.full((M, N + 8), 0x55, np.uint8)).view(torch.float8_e4m3fn).to(G.DEV)
    cd = full[:, :N]
    G.say("[case] fp8 guard band")
    T.gemm_tensors(ad, bd, cd, alpha=0.5)
    torch.cuda.synchronize()
    fb = fp8_bits(full)
    assert (fb[:, N:] == 0x55).all(), "padding written"
    o = oracle.gemm_fused(a, b, W.F16, alpha=0.5, nthreads=G.NTHREADS)
    assert np.array_equal(fb[:, :N], oracle.encode_fp8(o, T.FP8_E4M3))
    a0 = torch.empty((37, 0), dtype=torch.float16, device=G.DEV)
    b0 = torch.empty((0, 45), dtype=torch.float16, device=G.DEV)
    c0 = fp8_tensor(np.full((37, 45), 0x7F, np.uint8), T.FP8_E5M2)
    G.say("[case] fp8 K = 0")
    T.gemm_tensors(a0, b0, c0)
    torch.cuda.synchronize()
    assert (fp8_bits(c0) == 0).all()


def _bound_check(d_bits, o, z, p, s, alpha, cterm, bterm, fmt, K, label):
    tdt, mx, u8, eta8 = FMTS[fmt]
    d = oracle.decode(d_bits, fmt)
    assert np.isfinite(d).all(), f"{label}: non-finite outputs"
    ku = K * U32
    bz = abs(alpha) * (ku / (1 - ku)) * s + 3 * U32 * (np.abs(alpha * p) + cterm + bterm)
    dt = SLOPE * bz + 16 * U32 * (np.abs(o) + np.abs(z))     # |t - o|
    bound = u8 * np.abs(o) + (1 + u8) * dt + eta8
    diff = np.abs(d - np.clip(o, -mx, mx))
    assert (diff <= bound).all(), f"{label}: worst ratio {float((diff / bound).max()):.3f}"
    return float((diff / bound).max())


@pytest.mark.parametrize("fmt", [T.FP8_E4M3, T.FP8_E5M2], ids=["e4m3", "e5m2"])
@pytest.mark.parametrize("shape", [((256, 512, 384), 0), ((1024, 2048, 512), 8), ((127, 255, 512), 6)],
                         ids=["ring_big", "ring_small", "direct"])
def test_fp8_random_bound(fmt, shape):
    (M, N, K), cid = shape
    a, b = W.random_inputs(M, N, K, W.F16, seed=M + fmt)
    bias = W.to_storage(np.random.default_rng(3).standard_normal(N).astype(np.float32), W.F16)
    c_old = np.zeros((M, N), np.uint8)
    for alpha, act in ((0.5, T.ACT_GELU_TANH), (4.0, T.ACT_SILU)):
        d, _ = run(a, b, W.F16, fmt, c_old, cid=cid, label="random", alpha=alpha, bias=bias, bias_dt=W.F16,
                   activation=act)
        kw = dict(alpha=alpha, bias=bias, bias_dtype=W.F16, bias_kind=oracle.BIAS_COL, nthreads=G.NTHREADS)
        o = oracle.gemm_fused(a, b, W.F16, act=act, **kw)
        z = oracle.gemm_fused(a, b, W.F16, act=oracle.ACT_NONE, **kw)
        p = oracle.gemm(a, b, W.F16, nthreads=G.NTHREADS)
        s = oracle.gemm(G.abs_storage(a, W.F16), G.abs_storage(b, W.F16), W.F16, nthreads=G.NTHREADS)
        bterm = np.abs(oracle.decode(bias, W.F16))[None, :]
        r = _bound_check(d, o, z, p, s, alpha, 0.0, bterm, fmt, K, f"{M}x{N}x{K} fmt {fmt}")
        G.say(f"    ok, worst bound ratio {r:.3f}")


def test_fp8_8192_sampled():
    """The 8192^3 workload to E4M3 with a column bias and the tanh gelu at
    alpha = 1/64 (results mostly inside the finite range), 64 x 64 sampled."""
    w = W.WORKLOADS[4]
    a, b = W.make_inputs(w)
    bias = W.to_storage(np.random.default_rng(10).standard_normal(w.N).astype(np.float32), W.F16)
    ad, bd = G.to_device(a, W.F16), G.to_device(b, W.F16)
    cd = torch.empty((w.M, w.N), dtype=torch.float8_e4m3fn, device=G.DEV)
    kind = T.gemm_select_kernel(w.M, w.N, w.K, ad.data_ptr(), w.K, bd.data_ptr(), w.N, cd.data_ptr(), w.N, W.F16,
                                T.FP8_E4M3)
    G.say(f"[case] fp8 8192^3 bias + gelu_tanh -> {KIND.get(kind, kind)}")
    assert kind == T.KERNEL_RING
    alpha = 1.0 / 64
    T.gemm_tensors(ad, bd, cd, alpha=alpha, bias=vec_device(bias, W.F16), activation=T.ACT_GELU_TANH)
    torch.cuda.synchronize()
    rows = W.sample_indices(w.M, 64, w.seed + 700)
    cols = W.sample_indices(w.N, 64, w.seed + 800)
    d = fp8_bits(cd)[np.ix_(rows, cols)]
    kw = dict(alpha=alpha, bias=bias, bias_dtype=W.F16, bias_kind=oracle.BIAS_COL, rows=rows, cols=cols,
              nthreads=G.NTHREADS)
    o = oracle.gemm_fused(a, b, W.F16, act=oracle.ACT_GELU_TANH, **kw)
    z = oracle.gemm_fused(a, b, W.F16, act=oracle.ACT_NONE, **kw)
    p = oracle.gemm(a, b, W.F16, rows=rows, cols=cols, nthreads=G.NTHREADS)
    s = oracle.gemm(G.abs_storage(a, W.F16), G.abs_storage(b, W.F16), W.F16, rows=rows, cols=cols,
                    nthreads=G.NTHREADS)
    bterm = np.abs(oracle.decode(bias, W.F16))[cols][None, :]
    _bound_check(d, o, z, p, s, alpha, 0.0, bterm, T.FP8_E4M3, w.K, "8192^3 e4m3")
