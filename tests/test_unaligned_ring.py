"""GPU parity of the ring kernel on operands whose rows are not whole 16-byte
chunks: leading dimensions of every residue mod 8 and bases at any even
address, for every operand-layout pair, against the oracle.

The ring's 16-byte loads then start at 2-byte-aligned addresses; their range
check keeps a 4-byte part only if it ends inside the operand's range, which
ends at the dword boundary after the operand's last element, or 2 bytes
further where the last element starts a part at an address of 2 mod 4 (those
bytes are then read, so they must lie in the element's page).  Where they
would start a new 4 KiB page (the rule restated in `last_fix` below) the
kernel loads that element on its own in its K tail, leaving a k-strided
operand's last k-row to the tail; those placements are run for each operand
and layout.  Every even-address operand runs the ring.

Every operand sits in a NaN-filled buffer (NaN in the row padding, in the
elements before the base and after the last element), so a read past K that
is not masked, or a part kept past the operand's end, turns an output into
NaN.  Integer inputs in [-2, 2] make every fp32 sum exact: the results must
equal the oracle bit for bit after rounding to the output type.  Every case
prints its shape, layouts, offsets and the kernel before it touches the GPU.
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


def lid(lay):
    return "".join("r" if x == ROW else "c" for x in lay)


def last_fix(base, ld, kcontig, outer, K):
    """Whether the ring loads the operand's last element on its own: that
    element starts a 4-byte part of its 16-byte load (an odd element count
    along the row from the row's first loaded element) at an address of
    2 mod 4, and the 2 bytes after it start a new 4 KiB page (else the range
    is padded by them)."""
    rows, cols = (outer, K) if kcontig else (K, outer)
    last = base + 2 * ((rows - 1) * ld + cols - 1)
    return cols % 2 == 1 and last % 4 == 2 and (last + 2) % 4096 == 0


def place_ending_at_page(x, dt, layout=ROW):
    """Device copy of x (rows x cols) stored row- or column-major with no
    padding, whose last stored element ends exactly at a 4 KiB page
    boundary, in a NaN-filled buffer."""
    s = np.ascontiguousarray(x if layout == ROW else x.T)
    rows, cols = s.shape
    n = rows * cols
    flat = torch.full((n + 4096,), float("nan"), dtype=G.TORCH[dt], device=G.DEV)
    off = ((-(flat.data_ptr() + 2 * n)) % 4096) // 2
    view = flat[off:off + n].view(rows, cols)
    host = torch.from_numpy(s.view(np.int16)).view(torch.bfloat16) if dt == W.BF16 else torch.from_numpy(s)
    view.copy_(host.to(G.DEV))
    assert (view.data_ptr() + 2 * n) % 4096 == 0
    return view if layout == ROW else view.t()


def place(x, dt, layout, pad, offset):
    if layout == ROW:
        return G.to_device(x, dt, pad_cols=pad, offset_elems=offset)
    return G.to_device(np.ascontiguousarray(x.T), dt, pad_cols=pad, offset_elems=offset).t()


def run_exact(M, N, K, in_dt, out_dt, lay, pads, offs, cid, seed, at_page=(False, False)):
    """Integer inputs through gemm_t (an operand flagged in at_page is placed
    with its last element ending at a page boundary instead of by pad and
    offset); asserts the ring and bit-exact results; returns whether an
    operand's last element was loaded on its own."""
    a, b = W.integer_inputs(M, N, K, in_dt, seed=seed)
    ad = place_ending_at_page(a, in_dt, lay[0]) if at_page[0] else place(a, in_dt, lay[0], pads[0], offs[0])
    bd = place_ending_at_page(b, in_dt, lay[1]) if at_page[1] else place(b, in_dt, lay[1], pads[1], offs[1])
    _, cd = G.out_tensor(M, N, out_dt)
    la, lda = T._layout(ad)
    lb, ldb = T._layout(bd)
    kind, cfg = T.gemm_select_kernel_t(M, N, K, ad.data_ptr(), lda, la, bd.data_ptr(), ldb, lb, cd.data_ptr(), N,
                                       ROW, in_dt, out_dt, cid)
    fix = (last_fix(ad.data_ptr(), lda, la == ROW, M, K), last_fix(bd.data_ptr(), ldb, lb == COL, N, K))
    G.say(f"[case] unaligned {M}x{N}x{K} lay={lid(lay)} in={in_dt} out={out_dt} lda={lda} ldb={ldb} "
          f"offs={offs} at_page={at_page} last_fix={fix} cfg{cid} -> {KIND.get(kind, kind)} cfg{cfg}")
    assert kind == T.KERNEL_RING, kind
    G.run(ad, bd, cd, cid)
    got = G.values(cd, out_dt)
    want = G.round_to(G.oracle_values(a, b, in_dt), out_dt)
    bad = got != want
    assert not bad.any(), f"{int(bad.sum())} entries differ, first at {np.argwhere(bad)[0].tolist()}"
    return any(fix)


# (M, N, K, configuration): odd and even sizes, K tails of odd length, one
# trip of the ring's loop or several
SHAPES = [(509, 515, 517, 1), (256, 264, 383, 1), (130, 1001, 300, 0), (777, 250, 1024, 0), (200, 384, 297, 8)]
# (pad A, pad B, offset A, offset B) in elements
PLACEMENTS = [(1, 3, 0, 0), (0, 0, 1, 0), (0, 0, 0, 3), (5, 2, 7, 1), (3, 7, 2, 6), (1, 1, 1, 1), (0, 0, 5, 5)]


@pytest.mark.parametrize("lay", [(ROW, ROW), (ROW, COL), (COL, ROW), (COL, COL)], ids=lambda l: lid(l))
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s[:3])) + f"_cfg{s[3]}")
def test_unaligned_operands_exact(shape, lay):
    M, N, K, cid = shape
    if cid == 8 and lay[0] == COL:
        cid = 1  # the 64 x 128 ring reads row-major A only
    for i, (pa, pb, oa, ob) in enumerate(PLACEMENTS):
        in_dt, out_dt = ((W.F16, W.F16), (W.BF16, W.F32), (W.F16, W.F32), (W.BF16, W.BF16))[i % 4]
        run_exact(M, N, K, in_dt, out_dt, lay, (pa, pb), (oa, ob), cid, seed=M + N + K + 11 * i)


# (M, N, K, layouts, A / B at a page, configuration): the last element of a
# k-contiguous operand (odd K: it is in the K tail) and of a k-strided one
# (odd M or N; K a multiple of the ring's step, so the tail exists only for
# the operand's last k-row), of A, of B, of both, in the 128 x 128, 256 x 256
# and 64 x 128 rings and the table's choice
AT_PAGE = [(511, 512, 513, (ROW, ROW), (True, False), 1), (511, 512, 512, (COL, ROW), (True, False), 1),
           (512, 509, 512, (ROW, ROW), (False, True), 1), (512, 512, 513, (ROW, COL), (False, True), 1),
           (511, 509, 512, (COL, ROW), (True, True), 1), (1023, 1024, 1024, (COL, COL), (True, False), 0),
           (1024, 1021, 2048, (ROW, ROW), (False, True), 0), (300, 512, 1025, (ROW, COL), (True, True), 8),
           (2048, 2048, 2047, (ROW, ROW), (True, False), -1), (2048, 1024, 1536, (COL, ROW), (True, False), -1)]


@pytest.mark.parametrize("case", AT_PAGE, ids=lambda c: "x".join(map(str, c[:3])) + "_" + lid(c[3]) +
                         "".join("ab"[i] for i in (0, 1) if c[4][i]) + f"_cfg{c[5]}")
def test_unaligned_last_element_at_page_boundary(case):
    """An operand whose last element starts a 4-byte part at 2 mod 4 and
    ends at a 4 KiB page boundary (its range cannot be padded): the kernel
    loads that element on its own.  NaN fills the buffer before the operand
    and the page after it; exact on integer values, with two of the input
    and output types."""
    M, N, K, lay, at_page, cid = case
    for i, (in_dt, out_dt) in enumerate(((W.F16, W.F16), (W.BF16, W.F32))):
        fixed = run_exact(M, N, K, in_dt, out_dt, lay, (0, 0), (0, 0), cid, seed=M + N + K + i, at_page=at_page)
        # an odd extent along the contiguous dimension at a page end puts
        # the last element at 2 mod 4: the element loaded on its own
        contig = (K if lay[0] == ROW else M, K if lay[1] == COL else N)
        assert fixed == any(at_page[j] and contig[j] % 2 == 1 for j in (0, 1)), (fixed, at_page, contig)


def test_unaligned_operands_random_values():
    """Random normal fp16 / bf16 inputs with odd leading dimensions and
    shifted bases through the ring: the stated tolerance and the
    fp32-accumulation bound."""
    for (M, N, K), in_dt, out_dt, pads, offs in (((1023, 1021, 1025), W.F16, W.F16, (0, 0), (0, 0)),
                                                 ((1000, 1003, 999), W.BF16, W.F32, (1, 2), (2, 2)),
                                                 ((1280, 1040, 777), W.F16, W.F32, (3, 5), (2, 4))):
        a, b = W.random_inputs(M, N, K, in_dt, seed=M + K)
        ad = G.to_device(a, in_dt, pad_cols=pads[0], offset_elems=offs[0])
        bd = G.to_device(b, in_dt, pad_cols=pads[1], offset_elems=offs[1])
        _, cd = G.out_tensor(M, N, out_dt)
        kind = T.gemm_select_kernel(M, N, K, ad.data_ptr(), K + pads[0], bd.data_ptr(), N + pads[1], cd.data_ptr(),
                                    N, in_dt, out_dt)
        G.say(f"[case] unaligned random {M}x{N}x{K} in={in_dt} out={out_dt} pads={pads} offs={offs} "
              f"-> {KIND.get(kind, kind)}")
        assert kind == T.KERNEL_RING
        G.run(ad, bd, cd)
        G.check(G.values(cd, out_dt), G.oracle_values(a, b, in_dt), a, b, in_dt, out_dt, K, label="unaligned")


def test_unaligned_operands_fused_and_fp8():
    """The fused epilogue (alpha, beta, bias, relu) and an 8-bit output on
    unaligned operands through the ring, exact on integer values."""
    M, N, K = 509, 515, 517
    a, b = W.integer_inputs(M, N, K, W.F16, seed=77)
    ad = G.to_device(a, W.F16, pad_cols=1, offset_elems=2)
    bd = G.to_device(b, W.F16, pad_cols=3, offset_elems=2)
    rng = np.random.default_rng(78)
    c_old = rng.integers(-8, 9, size=(M, N)).astype(np.float32)
    bias = rng.integers(-4, 5, size=N).astype(np.float32)
    flat, cd = G.out_tensor(M, N, W.F32)
    cd.copy_(torch.from_numpy(c_old).to(G.DEV))
    # the 128 x 128 ring, forced (the table runs this small product direct)
    kind = T.gemm_select_kernel(M, N, K, ad.data_ptr(), K + 1, bd.data_ptr(), N + 3, cd.data_ptr(), N, W.F16, W.F32,
                                1)
    G.say(f"[case] unaligned fused {M}x{N}x{K} -> {KIND.get(kind, kind)}")
    assert kind == T.KERNEL_RING
    T.gemm_tensors(ad, bd, cd, config_id=1, alpha=2.0, beta=-0.5, bias=torch.from_numpy(bias).to(G.DEV),
                   activation=T.ACT_RELU)
    torch.cuda.synchronize()
    want = oracle.gemm_fused(a, b, W.F16, alpha=2.0, beta=-0.5, c_old=c_old, out_dtype=W.F32, bias=bias,
                             bias_dtype=W.F32, bias_kind=oracle.BIAS_COL, act=oracle.ACT_RELU)
    got = G.values(cd, W.F32)
    assert np.array_equal(got, want.astype(np.float32).astype(np.float64)), \
        f"{int((got != want).sum())} entries differ"
    # 8-bit output (E4M3, alpha 1/16: many results between 8-bit values)
    c8 = torch.zeros((M, N), dtype=torch.float8_e4m3fn, device=G.DEV)
    G.say(f"[case] unaligned fp8 {M}x{N}x{K}")
    assert T.gemm_select_kernel(M, N, K, ad.data_ptr(), K + 1, bd.data_ptr(), N + 3, c8.data_ptr(), N, W.F16,
                                T.FP8_E4M3, 1) == T.KERNEL_RING
    T.gemm_tensors(ad, bd, c8, config_id=1, alpha=1.0 / 16)
    torch.cuda.synchronize()
    got8 = c8.cpu().view(torch.uint8).numpy()
    want8 = oracle.encode_fp8(oracle.gemm(a, b, W.F16, nthreads=G.NTHREADS) / 16, T.FP8_E4M3)
    assert np.array_equal(got8, want8), f"{int((got8 != want8).sum())} entries differ"


@pytest.mark.parametrize("n", [8191, 4095])
def test_odd_square_sampled(n):
    """n x n x n fp16 with contiguous rows of odd length (every base aligned):
    the ring (asserted), sampled rows and columns against the oracle."""
    a, b = W.random_inputs(n, n, n, W.F16, seed=n)
    ad, bd = G.to_device(a, W.F16), G.to_device(b, W.F16)
    _, cd = G.out_tensor(n, n, W.F16)
    kind = T.gemm_select_kernel(n, n, n, ad.data_ptr(), n, bd.data_ptr(), n, cd.data_ptr(), n, W.F16, W.F16)
    G.say(f"[case] odd square {n}^3 -> {KIND.get(kind, kind)}")
    assert kind == T.KERNEL_RING
    G.run(ad, bd, cd)
    rows = np.unique(np.concatenate([W.sample_indices(n, 48, seed=1), [0, n - 1]]))
    cols = np.unique(np.concatenate([W.sample_indices(n, 48, seed=2), [0, n - 1]]))
    c = G.values(cd, W.F16)[rows][:, cols]
    G.check(c, G.oracle_values(a, b, W.F16, rows=rows, cols=cols), a, b, W.F16, W.F16, n, rows=rows, cols=cols,
            label=f"odd square {n}")
