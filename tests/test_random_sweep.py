"""GPU parity over a seeded random sweep of calls.  Each case draws the sizes
(1 to 1100, tile multiples and their neighbours, and long-K products
that split K), the layouts of A, B and C, padded leading dimensions, the input
and output types (8-bit outputs included), the configuration (the table's
choice or any configuration of the input family that takes the layouts)
and the fused epilogue (alpha and beta powers of two, a row or column bias
of any bias type, relu).

Integer inputs in [-2, 2], small-integer C and bias: every value on both
sides is exact until the output rounding, so each output must equal the
oracle's value rounded to the output type bit for bit.  Operands and C sit
in NaN-filled buffers, so a read past an operand's extent turns outputs into
NaN and a write past C's shows in its padding.  Each case prints its draw
before it touches the GPU.
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
E4M3, E5M2 = T.FP8_E4M3, T.FP8_E5M2
FP8_TORCH = {E4M3: torch.float8_e4m3fn, E5M2: torch.float8_e5m2}
OUTS = {W.F32: [W.F32], W.F16: [W.F16, W.F32, E4M3, E5M2], W.BF16: [W.BF16, W.F32, E4M3, E5M2]}
NAMES = {W.F32: "f32", W.F16: "f16", W.BF16: "bf16", E4M3: "e4m3", E5M2: "e5m2"}
FP8_NAN = 0x7F  # a NaN in both 8-bit formats


def draw_dim(rng):
    r = rng.random()
    if r < 0.15:
        return int(rng.integers(1, 17))
    if r < 0.6:
        return int(rng.integers(17, 1101))
    return max(1, int(rng.choice([32, 64, 128, 256])) * int(rng.integers(1, 4)) + int(rng.integers(-1, 2)))


def draw(seed):
    rng = np.random.default_rng(1000 + seed)
    d = {"in": int(rng.choice([W.F16, W.BF16, W.F32], p=[0.4, 0.35, 0.25]))}
    d["out"] = int(rng.choice(OUTS[d["in"]]))
    if d["in"] != W.F32 and rng.random() < 0.2:  # few tiles, long K: split-K
        d["M"], d["N"], d["K"] = int(rng.integers(1, 301)), int(rng.integers(1, 301)), int(rng.integers(4096, 6501))
        if rng.random() < 0.7:  # whole groups of 4 columns, which split-K needs
            d["N"] = 4 * int(rng.integers(1, 76))
    else:
        d["M"], d["N"], d["K"] = draw_dim(rng), draw_dim(rng), draw_dim(rng)
    d["lay"] = tuple(int(x) for x in rng.choice([ROW, COL], size=3))
    d["pad"] = tuple(int(x) for x in rng.choice([0, 0, 0, 8, 1, 3], size=3))
    fam_dt = W.F32 if d["in"] == W.F32 else W.F16  # the 16-bit configurations take both 16-bit types
    fam = [i for i in range(T.gemm_num_configs()) if T.gemm_config_info(i)["in_dtype"] == fam_dt]
    d["cfg"] = -1 if rng.random() < 0.5 else int(rng.choice(fam))
    fp8 = d["out"] in (E4M3, E5M2)
    d["fused"] = fp8 or rng.random() < 0.5
    # alpha keeps |alpha * sum| <= 4 K |alpha| within E4M3's 448 with C and the bias
    d["alpha"] = 2.0 ** -int(np.ceil(np.log2(4 * d["K"] / 400))) if fp8 else float(rng.choice([1, 2, 0.5, -1]))
    d["beta"] = float(rng.choice([0, 1, -0.5, 2])) if d["fused"] else 0.0
    d["bias"] = int(rng.choice([oracle.BIAS_NONE, oracle.BIAS_ROW, oracle.BIAS_COL])) if d["fused"] else 0
    d["bias_dt"] = int(rng.choice([W.F32, W.F16, W.BF16]))
    d["act"] = int(rng.choice([oracle.ACT_NONE, oracle.ACT_RELU])) if d["fused"] else 0
    return d


def describe(d):
    lay = "".join("r" if x == ROW else "c" for x in d["lay"])
    s = f"{d['M']}x{d['N']}x{d['K']} {NAMES[d['in']]}->{NAMES[d['out']]} lay={lay} pad={d['pad']} cfg{d['cfg']}"
    if d["fused"]:
        s += f" alpha={d['alpha']} beta={d['beta']} bias={d['bias']}/{NAMES[d['bias_dt']]} act={d['act']}"
    return s


def place(x, dt, layout, pad):
    if layout == ROW:
        return G.to_device(x, dt, pad_cols=pad)
    return G.to_device(np.ascontiguousarray(x.T), dt, pad_cols=pad).t()


def device_vector(values, dt):
    st = W.to_storage(values.astype(np.float32), dt)
    t = torch.from_numpy(st.view(np.int16)).view(torch.bfloat16) if dt == W.BF16 else torch.from_numpy(st)
    return st, t.to(G.DEV)


def output_buffer(M, N, dt, layout, pad):
    """(flat buffer, C view, rows, stored width, ld) with the padding filled
    with NaN; a column-major C is the transpose of an N x M row-major one."""
    rows, width = (M, N) if layout == ROW else (N, M)
    ld = width + pad
    size = rows * ld + 64
    if dt in FP8_TORCH:
        flat = torch.full((size,), FP8_NAN, dtype=torch.uint8, device=G.DEV).view(FP8_TORCH[dt])
    else:
        flat = torch.full((size,), float("nan"), dtype=G.TORCH[dt], device=G.DEV)
    view = flat[:rows * ld].view(rows, ld)[:, :width]
    return flat, (view if layout == ROW else view.t()), rows, width, ld


def stored_c(values, dt):
    """Stored bits (the oracle's c_old) and a device copy of small-integer C
    values (of 8-bit outputs: their bytes)."""
    if dt in FP8_TORCH:
        bits = oracle.encode_fp8(values, dt)
        return bits, torch.from_numpy(bits).to(G.DEV)
    st = W.to_storage(values.astype(np.float32), dt)
    t = torch.from_numpy(st.view(np.int16)).view(torch.bfloat16) if dt == W.BF16 else torch.from_numpy(st)
    return st, t.to(G.DEV)


def padding_untouched(flat, rows, width, ld, dt):
    if dt in FP8_TORCH:
        raw = flat.view(torch.uint8)
        whole = raw[:rows * ld].view(rows, ld)
        return bool((whole[:, width:] == FP8_NAN).all()) and bool((raw[rows * ld:] == FP8_NAN).all())
    whole = flat[:rows * ld].view(rows, ld)
    return bool(torch.isnan(whole[:, width:].float()).all()) and bool(torch.isnan(flat[rows * ld:].float()).all())


@pytest.mark.parametrize("seed", range(96))
def test_random_call(seed):
    d = draw(seed)
    M, N, K, in_dt, out_dt = d["M"], d["N"], d["K"], d["in"], d["out"]
    a, b = W.integer_inputs(M, N, K, in_dt, seed=seed)
    ad, bd = place(a, in_dt, d["lay"][0], d["pad"][0]), place(b, in_dt, d["lay"][1], d["pad"][1])
    flat, cd, rows, width, ld = output_buffer(M, N, out_dt, d["lay"][2], d["pad"][2])
    la, lda = T._layout(ad)
    lb, ldb = T._layout(bd)
    lc, ldc = T._layout(cd)
    kind, cfg = T.gemm_select_kernel_t(M, N, K, ad.data_ptr(), lda, la, bd.data_ptr(), ldb, lb, cd.data_ptr(), ldc,
                                       lc, in_dt, out_dt, d["cfg"])
    if kind < 0:  # the drawn configuration does not take these layouts
        assert kind == T.ERR_CONFIG, (kind, describe(d))
        d["cfg"] = -1
        kind, cfg = T.gemm_select_kernel_t(M, N, K, ad.data_ptr(), lda, la, bd.data_ptr(), ldb, lb, cd.data_ptr(),
                                           ldc, lc, in_dt, out_dt, -1)
    G.say(f"[case] sweep {seed}: {describe(d)} -> kind {kind} cfg{cfg}")
    assert kind >= 0, kind
    rng = np.random.default_rng(seed)
    if not d["fused"]:
        G.run(ad, bd, cd, d["cfg"])
        got = G.values(cd, out_dt)
        want = G.round_to(G.oracle_values(a, b, in_dt), out_dt)
        assert np.array_equal(got, want), f"{int((got != want).sum())} entries differ"
    else:
        c_bits = None
        if d["beta"] != 0.0:
            c_bits, c_dev = stored_c(rng.integers(-8, 9, size=(M, N)).astype(np.float64), out_dt)
            (cd.view(torch.uint8) if out_dt in FP8_TORCH else cd).copy_(c_dev)
        bias_st, bias_dev = None, None
        if d["bias"] != oracle.BIAS_NONE:
            n = M if d["bias"] == oracle.BIAS_ROW else N
            bias_st, bias_dev = device_vector(rng.integers(-4, 5, size=n).astype(np.float64), d["bias_dt"])
        rc = T.gemm_tensors(ad, bd, cd, config_id=d["cfg"], check=False, alpha=d["alpha"], beta=d["beta"],
                            bias=bias_dev, bias_kind=d["bias"] if d["bias"] else None, activation=d["act"])
        assert rc == T.OK, f"gemm_fused returned {rc}: {T.gemm_strerror(rc)}"
        torch.cuda.synchronize()
        want = oracle.gemm_fused(a, b, in_dt, alpha=d["alpha"], beta=d["beta"], c_old=c_bits, out_dtype=out_dt,
                                 bias=bias_st, bias_dtype=d["bias_dt"], bias_kind=d["bias"], act=d["act"],
                                 nthreads=G.NTHREADS)
        if out_dt in FP8_TORCH:
            got = cd.view(torch.uint8).cpu().numpy()
            exp = oracle.encode_fp8(want, out_dt)
        else:
            got, exp = G.values(cd, out_dt), G.round_to(want, out_dt)
        assert np.array_equal(got, exp), f"{int((got != exp).sum())} entries differ"
    assert padding_untouched(flat, rows, width, ld, out_dt), "C's padding written"
