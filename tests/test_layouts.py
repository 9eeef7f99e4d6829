"""GPU parity of the column-major layouts (gemm_t): every combination of
row-major and column-major A, B and C against the oracle.

A column-major operand is stored transposed on the device and handed over as
a transposed view (stride 1 down its columns); the binding reads the layout
off the strides.  The same host values feed the oracle, so a case passes only
if the kernels read each layout as the matrix it stands for (the two layouts
of page "TileLang实战：用Python DSL自动生成高性能GPU计算内核", §5.1).  Every
case prints its name, shape, layouts and the kernel the library chose before
it touches the GPU.
"""
import itertools

import numpy as np
import pytest
import torch

import tiled_gemm_03_amd as T
from tiled_gemm_03_amd import workloads as W

import gpu_helpers as G

pytestmark = pytest.mark.gpu

ROW, COL = T.ROW_MAJOR, T.COL_MAJOR
LAYOUTS = list(itertools.product((ROW, COL), repeat=3))
KIND = {T.KERNEL_GENERAL: "general", T.KERNEL_TILED: "tiled", T.KERNEL_RING: "ring", T.KERNEL_DIRECT: "direct"}


def lid(lay):
    return "".join("r" if x == ROW else "c" for x in lay)


def place(x, dt, layout, pad=0, offset=0):
    """Host values (rows x cols) -> device view of the same matrix in the
    given layout; the padding extends the leading dimension."""
    if layout == ROW:
        return G.to_device(x, dt, pad_cols=pad, offset_elems=offset)
    return G.to_device(np.ascontiguousarray(x.T), dt, pad_cols=pad, offset_elems=offset).t()


def out_place(M, N, dt, layout, pad=0, offset=0):
    if layout == ROW:
        return G.out_tensor(M, N, dt, pad_cols=pad, offset_elems=offset)[1]
    return G.out_tensor(N, M, dt, pad_cols=pad, offset_elems=offset)[1].t()


def kernel_of(ad, bd, cd, in_dt, out_dt, cid=-1):
    la, lda = T._layout(ad)
    lb, ldb = T._layout(bd)
    lc, ldc = T._layout(cd)
    M, K = ad.shape
    N = bd.shape[1]
    return T.gemm_select_kernel_t(M, N, K, ad.data_ptr(), lda, la, bd.data_ptr(), ldb, lb, cd.data_ptr(), ldc, lc,
                                  in_dt, out_dt, cid)


def effective_row_row(lay):
    """Whether the call reduces to row-major A and B (a column-major C is
    computed as C^T = B^T A^T, which flips both operands' layouts)."""
    la, lb, lc = lay
    if lc == COL:
        la, lb = lb ^ 1, la ^ 1
    return la == ROW and lb == ROW


def run_layout(a, b, in_dt, out_dt, lay, cid=-1, pads=(0, 0, 0), offs=(0, 0, 0), rows=None, cols=None, label=""):
    M, K = a.shape
    N = b.shape[1]
    ad = place(a, in_dt, lay[0], pads[0], offs[0])
    bd = place(b, in_dt, lay[1], pads[1], offs[1])
    cd = out_place(M, N, out_dt, lay[2], pads[2], offs[2])
    kind, cfg = kernel_of(ad, bd, cd, in_dt, out_dt, cid)
    G.say(f"[case] {label} {M}x{N}x{K} layouts={lid(lay)} in={in_dt} out={out_dt} pads={pads} offs={offs} "
          f"-> {KIND.get(kind, kind)} cfg{cfg}")
    G.run(ad, bd, cd, cid)
    c = G.values(cd, out_dt)
    if rows is not None:
        c = c[rows][:, cols]
    o = G.oracle_values(a, b, in_dt, rows=rows, cols=cols)
    return c, o, kind


SHAPES = [(256, 256, 128), (512, 768, 384), (1024, 2048, 512), (127, 255, 512), (33, 47, 255), (300, 257, 1000),
          (1, 1, 1), (64, 64, 40), (128, 384, 100)]


@pytest.mark.parametrize("lay", LAYOUTS, ids=lid)
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_layouts_against_oracle(lay, shape):
    """Random inputs; whole tiles with K a multiple of 128 take the ring
    kernel whenever the call does not reduce to row-major operands, other
    shapes the ring or the direct kernel."""
    M, N, K = shape
    for in_dt, out_dt in ((W.F16, W.F16), (W.BF16, W.F32)):
        a, b = W.random_inputs(M, N, K, in_dt, seed=M + 5 * N + 11 * K + 3 * lay[0] + 7 * lay[1] + 13 * lay[2])
        c, o, kind = run_layout(a, b, in_dt, out_dt, lay, label="layout")
        G.check(c, o, a, b, in_dt, out_dt, K, label=f"{lid(lay)} {shape}")
        if not effective_row_row(lay) and M % 128 == 0 and N % 128 == 0 and K % 128 == 0:
            assert kind == T.KERNEL_RING
        if not effective_row_row(lay):
            # column-major operands run the ring kernel where it applies
            # (alignment, K % 8, N % 4: pinned in test_abi) and else direct
            assert kind in (T.KERNEL_RING, T.KERNEL_DIRECT)


@pytest.mark.parametrize("lay", LAYOUTS, ids=lid)
@pytest.mark.parametrize("cid", [0, 1])
def test_layouts_ring_k_tail(lay, cid):
    """K not a multiple of 128: the ring kernel walks the largest multiple
    and adds the rest in 32-wide steps from registers (forced, path
    asserted).  Tails of 1, 72, 127 and 104 elements, K odd and K % 8 != 0;
    leading dimensions padded to 16-byte rows with NaN, so a k-contiguous
    operand has NaN right after its K-th element: it must be masked, not
    multiplied by zero."""
    cases = (((1001, 1004, 129), W.F16, W.F16), ((260, 516, 200), W.BF16, W.F32),
             ((513, 260, 1023), W.F16, W.F32), ((256, 256, 1000), W.BF16, W.BF16))
    pad = lambda e, mult: (-e) % mult or mult
    for (M, N, K), in_dt, out_dt in cases:
        if lay[2] == COL:
            M, N = N, M  # keep the odd size in the role of M of the product the call runs
        ext = {"a": (K, M), "b": (N, K), "c": (N, M)}
        pads = (pad(ext["a"][lay[0]], 8), pad(ext["b"][lay[1]], 8), pad(ext["c"][lay[2]], 4))
        a, b = W.random_inputs(M, N, K, in_dt, seed=K + cid + 3 * lay[0] + 5 * lay[1] + 7 * lay[2])
        c, o, kind = run_layout(a, b, in_dt, out_dt, lay, cid=cid, pads=pads, label="ring k tail")
        assert kind == T.KERNEL_RING, kind
        G.check(c, o, a, b, in_dt, out_dt, K, label=f"ring k tail {M}x{N}x{K} {lid(lay)} cfg{cid}")


@pytest.mark.parametrize("lay", [(ROW, ROW, ROW), (COL, ROW, ROW), (ROW, COL, ROW)], ids=lid)
def test_ring_k_tail_large_sampled(lay):
    """8192 x 8192 x 8000 fp16 (a K tail of 64 after 62 ring trips of 128),
    the launch configuration of the large products, checked on 64 x 64
    sampled outputs."""
    M, N, K = 8192, 8192, 8000
    a, b = W.random_inputs(M, N, K, W.F16, seed=8000)
    rows = W.sample_indices(M, 64, 8001)
    cols = W.sample_indices(N, 64, 8002)
    c, o, kind = run_layout(a, b, W.F16, W.F16, lay, rows=rows, cols=cols, label="ring k tail 8192^2x8000")
    assert kind == T.KERNEL_RING
    G.check(c, o, a, b, W.F16, W.F16, K, rows=rows, cols=cols, label=f"8192^2x8000 {lid(lay)}")


@pytest.mark.parametrize("lay", LAYOUTS, ids=lid)
def test_layouts_integer_bitwise(lay):
    """Small-integer inputs: every sum is exact in fp32 whatever its order,
    so C must equal the oracle rounded to the output type bit for bit, for
    every 16-bit type pair, through the ring and the direct kernel."""
    for M, N, K in ((256, 512, 640), (512, 256, 256), (127, 255, 512), (300, 257, 1000)):
        for in_dt, out_dt in ((W.F16, W.F16), (W.F16, W.F32), (W.BF16, W.BF16), (W.BF16, W.F32)):
            a, b = W.integer_inputs(M, N, K, in_dt, seed=M + N + K + 17 * lay[2])
            c, o, _ = run_layout(a, b, in_dt, out_dt, lay, label="layout bitwise")
            want = G.round_to(o, out_dt)
            assert np.array_equal(c, want), f"{int((c != want).sum())} entries differ"


@pytest.mark.parametrize("lay", LAYOUTS, ids=lid)
def test_layouts_fp32_inputs(lay):
    for M, N, K in ((127, 255, 512), (64, 128, 96), (300, 200, 33)):
        a, b = W.random_inputs(M, N, K, W.F32, seed=M * N + K)
        c, o, kind = run_layout(a, b, W.F32, W.F32, lay, label="layout fp32")
        G.check(c, o, a, b, W.F32, W.F32, K, label=f"{lid(lay)} fp32")
        if not effective_row_row(lay):
            assert kind == T.KERNEL_DIRECT


@pytest.mark.parametrize("lay", [l for l in LAYOUTS if not effective_row_row(l)], ids=lid)
def test_layouts_padded_and_misaligned(lay):
    """Padded leading dimensions and operand bases off 16-byte alignment stay
    on the ring kernel (even sizes: its loads keep every element); a C whose
    rows are not 4-element aligned moves this small product to the direct
    kernel; both must be exact (integer inputs)."""
    M, N, K = 256, 512, 384
    a, b = W.integer_inputs(M, N, K, W.F16, seed=77)
    for pads, offs, ring in (((8, 16, 8), (0, 0, 0), True), ((3, 5, 0), (0, 0, 0), True),
                             ((3, 5, 1), (0, 0, 0), False), ((0, 0, 0), (1, 0, 0), True),
                             ((0, 0, 0), (0, 1, 0), True), ((0, 0, 0), (0, 0, 1), False)):
        for out_dt in (W.F16, W.F32):
            c, o, kind = run_layout(a, b, W.F16, out_dt, lay, pads=pads, offs=offs, label="layout pad/offset")
            assert (kind == T.KERNEL_RING) == ring
            want = G.round_to(o, out_dt)
            assert np.array_equal(c, want), f"{int((c != want).sum())} entries differ"


@pytest.mark.parametrize("lay", LAYOUTS, ids=lid)
def test_layouts_write_only_c(lay):
    """C starts as NaN inside padded storage whose padding holds a sentinel:
    every entry of C is written and nothing else."""
    M, N, K = 200, 136, 72
    a, b = W.random_inputs(M, N, K, W.F16, seed=3)
    ad, bd = place(a, W.F16, lay[0]), place(b, W.F16, lay[1])
    rows, cols = (M, N) if lay[2] == ROW else (N, M)
    flat = torch.full((rows * (cols + 8) + 64,), float("nan"), dtype=torch.float16, device=G.DEV)
    store = flat[:rows * (cols + 8)].view(rows, cols + 8)
    store[:, cols:] = 12345.0
    flat[rows * (cols + 8):] = -777.0
    c = store[:, :cols] if lay[2] == ROW else store[:, :cols].t()
    G.say(f"[case] layout canary {M}x{N}x{K} {lid(lay)}")
    G.run(ad, bd, c)
    assert not bool(torch.isnan(c).any()), "some entries of C were not written"
    assert bool((store[:, cols:] == 12345.0).all()), "padding was written"
    assert bool((flat[rows * (cols + 8):] == -777.0).all()), "memory after C was written"
    G.check(G.values(c, W.F16), G.oracle_values(a, b, W.F16), a, b, W.F16, W.F16, K, label="canary")


@pytest.mark.parametrize("lay", LAYOUTS, ids=lid)
@pytest.mark.parametrize("cid", [0, 1])
def test_layouts_ring_partial_groups_unaligned_c(lay, cid):
    """The ring kernel (forced, path asserted) with M and N both 2 mod 4 and
    C rows 3 elements longer than C (ldc odd: no 4-element aligned store),
    operands padded to 16-byte rows: the last column group of every row is
    partial and every store unaligned, through the fused epilogue's stores
    with the identity epilogue.  C starts as NaN, its padding and the memory
    after it hold sentinels: every entry of C is written and nothing else,
    and with small-integer inputs the values are exact."""
    M, N, K = 302, 1030, 384 if cid == 1 else 520
    pad = lambda e, mult: (-e) % mult or mult
    stored = {"a": (K, M), "b": (N, K)}  # stored row length for (row-major, column-major)
    for in_dt, out_dt in ((W.F16, W.F16), (W.BF16, W.F32)):
        a, b = W.integer_inputs(M, N, K, in_dt, seed=cid + 3 * lay[0] + 5 * lay[1] + 7 * lay[2])
        ad = place(a, in_dt, lay[0], pad(stored["a"][lay[0]], 8))
        bd = place(b, in_dt, lay[1], pad(stored["b"][lay[1]], 8))
        rows, cols = (M, N) if lay[2] == ROW else (N, M)
        tdt = G.TORCH[out_dt]
        flat = torch.full((rows * (cols + 3) + 64,), float("nan"), dtype=tdt, device=G.DEV)
        store = flat[:rows * (cols + 3)].view(rows, cols + 3)
        store[:, cols:] = 12345.0
        flat[rows * (cols + 3):] = -777.0
        c = store[:, :cols] if lay[2] == ROW else store[:, :cols].t()
        kind, _ = kernel_of(ad, bd, c, in_dt, out_dt, cid)
        G.say(f"[case] ring partial groups {M}x{N}x{K} {lid(lay)} cfg{cid} in={in_dt} out={out_dt} kind={kind}")
        assert kind == T.KERNEL_RING, kind
        G.run(ad, bd, c, config=cid)
        assert not bool(torch.isnan(c).any()), "some entries of C were not written"
        assert bool((store[:, cols:] == 12345.0).all()), "padding was written"
        assert bool((flat[rows * (cols + 3):] == -777.0).all()), "memory after C was written"
        got = G.values(c, out_dt)
        want = G.round_to(G.oracle_values(a, b, in_dt), out_dt)
        assert np.array_equal(got, want), f"{int((got != want).sum())} entries differ"


def test_layouts_k_zero():
    for lay in LAYOUTS:
        G.say(f"[case] layout K=0 {lid(lay)}")
        a = place(np.zeros((37, 0), np.float16), W.F16, lay[0])
        b = place(np.zeros((0, 45), np.float16), W.F16, lay[1])
        c = out_place(37, 45, W.F32, lay[2])
        G.run(a, b, c)
        assert bool((c == 0).all())


@pytest.mark.parametrize("lay", [(ROW, COL, ROW), (COL, ROW, ROW), (COL, COL, ROW)], ids=lid)
def test_layouts_8192_sampled(lay):
    """The 8192^3 fp16 product with transposed operands (ring kernel, 256 x
    256 tiles), checked on 64 x 64 sampled outputs."""
    w = W.WORKLOADS[4]
    a, b = W.make_inputs(w)
    rows = W.sample_indices(w.M, 64, w.seed + 300)
    cols = W.sample_indices(w.N, 64, w.seed + 400)
    c, o, kind = run_layout(a, b, w.in_dtype, w.out_dtype, lay, rows=rows, cols=cols, label=w.name)
    assert kind == T.KERNEL_RING
    G.check(c, o, a, b, w.in_dtype, w.out_dtype, w.K, rows=rows, cols=cols, label=f"{w.name} {lid(lay)}")


@pytest.mark.parametrize("lay", LAYOUTS, ids=lid)
@pytest.mark.parametrize("cid", [0, 1])
def test_layouts_ring_odd_edges(lay, cid):
    """The ring kernel (forced, path asserted) on an odd M and N a multiple
    of 4 but not of 8: leading dimensions padded to the alignment the ring
    needs, the padding NaN (it reaches only outputs past M or N, never
    stored; a k-strided A's last element must not be lost to the dword that
    straddles the end of its range)."""
    # an odd size in the role of M of the row-major product the call runs
    # (a column-major C swaps M and N); its N a multiple of 4, not of 8
    M, N, K = (1001, 1004, 512) if lay[2] == ROW else (1004, 1001, 512)
    ext = {"a": (K, M), "b": (N, K), "c": (N, M)}  # stored row length for (row-major, column-major)
    pad = lambda e, mult: (-e) % mult or mult
    pads = (pad(ext["a"][lay[0]], 8), pad(ext["b"][lay[1]], 8), pad(ext["c"][lay[2]], 4))
    for in_dt, out_dt in ((W.F16, W.F16), (W.BF16, W.F32)):
        a, b = W.random_inputs(M, N, K, in_dt, seed=17 + cid + 3 * lay[0] + 5 * lay[1] + 7 * lay[2])
        c, o, kind = run_layout(a, b, in_dt, out_dt, lay, cid=cid, pads=pads, label="ring odd")
        assert kind == T.KERNEL_RING, kind
        G.check(c, o, a, b, in_dt, out_dt, K, label=f"ring odd {lid(lay)} cfg{cid}")
