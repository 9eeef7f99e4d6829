"""Attention forward through the C ABI (attention_fwd) against the oracle.

CPU tests: argument checks (every invalid call is rejected before anything is
enqueued, so they need no GPU).

GPU tests: element-wise parity with oracle.attention (binary64) on the same
seeded inputs, every output held to the bound that any implementation of the
method with these precisions meets (fp32 scores and softmax, probabilities
rounded to the input type before the product with V, fp32 accumulation,
output rounded once):

    |o - r| <= u_out |r| + (1 + u_out) ((2 u_in / (1 - u_in) + 2 rho) (P|V|) + 2 n_k eta_in max_j |v_j|)

with r the oracle's output, P|V| the oracle's attention of |V| (the same
weights applied to the absolute values), u_in / u_out the unit roundoffs of
the input / output types (2^-11 fp16, 2^-8 bf16, 0 fp32; a weight p_j / L
with p_j rounded to the input type and L the sum of the rounded or of the
unrounded p is off by at most 2 u_in / (1 - u_in) relative), eta_in half the
smallest subnormal spacing of the input type (probabilities below the normal
range lose relative precision: 2^-25 fp16, negligible for bf16), and rho the
fp32 part: the relative error of each weight from the rounded scores
(scale gamma_{d+4} max_j sum_c |q_c k_jc|, doubled since a weight is a ratio
of two exponentials, through exp), of the fp32 sums of the normaliser and of
the product (gamma_{n_k} each), of one rescale per key block and of a few
roundings (exp2, division, scaling).
"""
import math

import numpy as np
import pytest

import oracle
import tiled_gemm_03_amd as T
from oracle.attention import attention as oracle_attention
from tiled_gemm_03_amd import workloads as W

FAKE = 1 << 40  # a pointer value that is never dereferenced (rejected calls)
U = {W.F32: 0.0, W.F16: 2.0 ** -11, W.BF16: 2.0 ** -8}
ETA = {W.F16: 2.0 ** -25, W.BF16: 0.0}


def _call(B=1, H=1, nq=4, nk=4, d=64, q=FAKE, qs=None, k=FAKE + (1 << 30), ks=None, v=FAKE + (2 << 30), vs=None,
          o=FAKE + (3 << 30), os_=None, i=W.F16, out=W.F16, scale=1.0, causal=0):
    return T.attention_fwd(B, H, nq, nk, d, q, qs, k, ks, v, vs, o, os_, i, out, scale, causal, None)


@pytest.mark.parametrize("kw,code", [
    (dict(B=-1), T.ERR_DIM),
    (dict(H=70000), T.ERR_DIM),
    (dict(nk=0), T.ERR_DIM),
    (dict(nq=-3), T.ERR_DIM),
    (dict(scale=float("inf")), T.ERR_DIM),
    (dict(scale=float("nan")), T.ERR_DIM),
    (dict(d=32), T.ERR_HEAD_DIM),
    (dict(d=96), T.ERR_HEAD_DIM),
    (dict(i=W.F32, out=W.F32), T.ERR_DTYPE),
    (dict(i=W.F16, out=W.BF16), T.ERR_DTYPE),
    (dict(i=W.BF16, out=W.F16), T.ERR_DTYPE),
    (dict(q=None), T.ERR_NULL),
    (dict(v=None), T.ERR_NULL),
    (dict(o=None), T.ERR_NULL),
    (dict(qs=(256, 256, -64)), T.ERR_LD),
    (dict(os_=(256, 256, 32)), T.ERR_LD),            # output rows overlap
    (dict(ks=(1 << 26, 1 << 26, 1 << 24)), T.ERR_LD),  # 64 K rows beyond 32-bit byte offsets
    (dict(vs=(1 << 26, 1 << 26, 1 << 24)), T.ERR_LD),  # the same for V
    (dict(ks=(1 << 26, 1 << 26, (1 << 24) - 1)), T.ERR_LD),  # 64 rows + d elements just reach 2^31 bytes
    (dict(H=2, os_=(512, 32, 128)), T.ERR_LD),       # head 1 starts inside a row of head 0
    (dict(o=FAKE + 100), T.ERR_ALIAS),                # output overlaps Q
    (dict(o=FAKE + (2 << 30) + 510), T.ERR_ALIAS),   # output overlaps the end of V
    (dict(q=FAKE + 1), T.ERR_ALIGN),                  # elements not aligned to their size
    (dict(k=FAKE + (1 << 30) + 3), T.ERR_ALIGN),
    (dict(o=FAKE + (3 << 30) + 2, out=W.F32), T.ERR_ALIGN),
])
def test_attention_arguments_are_checked(kw, code):
    assert _call(**kw) == code
    assert T.gemm_strerror(code) != "unknown error code"


def test_attention_interleaved_heads_are_not_an_overlap():
    # heads interleaved with rows (head h at offset 64 h, rows 128 apart) do
    # not overlap; the call would launch, so only the check itself is run:
    # the same layout with the output on top of Q is rejected as an alias,
    # which is tested after the layout check
    assert _call(H=2, os_=(512, 64, 128), o=FAKE + 8) == T.ERR_ALIAS


def test_attention_workgroup_shape():
    # 128-row tiles while that gives every CU a workgroup, else (head dim
    # 64) 32-row tiles with the keys split over two waves
    assert T.attention_waves(4, 16, 4096, 128) == 4
    assert T.attention_waves(1, 256, 1, 64) == 4
    assert T.attention_waves(1, 255, 128, 64) == 1
    assert T.attention_waves(1, 12, 1024, 64) == 1
    assert T.attention_waves(1, 1, 1, 64) == 1
    assert T.attention_waves(1, 1, 1, 128) == 4   # head_dim 128: always 4
    assert T.attention_waves(0, 1, 1, 64) == T.ERR_DIM
    assert T.attention_waves(1, 1 << 20, 1, 64) == T.ERR_DIM
    assert T.attention_waves(1, 1, 1, 96) == T.ERR_HEAD_DIM


def test_attention_empty_problems_are_noops():
    # nothing to compute: success, even with NULL pointers and no keys
    assert _call(nq=0, nk=0, q=None, k=None, v=None, o=None) == T.OK
    assert _call(B=0, q=None, k=None, v=None, o=None) == T.OK
    assert _call(H=0, q=None, k=None, v=None, o=None) == T.OK


# ----------------------------------------------------------------- GPU parity
def _dev(x, dtype):
    import torch
    from gpu_helpers import TORCH
    if dtype == W.BF16:
        h = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
    else:
        h = torch.from_numpy(np.ascontiguousarray(x))
    return h.to("cuda:0")


def _abs_stored(x, dtype):
    """|x| of a stored array, exactly (clear the sign)."""
    if dtype == W.BF16:
        return x & np.uint16(0x7FFF)
    return np.abs(x)


def _bound(q, k, v, ref, dtype, out, scale, causal, rows=None):
    """The element-wise tolerance of the module docstring (binary64)."""
    Qv, Kv = oracle.decode(np.ascontiguousarray(q), dtype), oracle.decode(np.ascontiguousarray(k), dtype)
    if rows is not None:
        Qv = Qv[:, :, rows, :]
    nk, d = Kv.shape[2], Kv.shape[3]
    u = 2.0 ** -24
    g = lambda n: n * u / (1 - n * u)
    qk = np.matmul(np.abs(Qv), np.swapaxes(np.abs(Kv), 2, 3))  # sum_c |q_c k_jc|
    ds = abs(scale) * g(d + 4) * qk.max(axis=3, keepdims=True)
    nb = math.ceil(nk / 64)
    rho = math.e ** (2 * ds) - 1 + 2 * g(nk) + 2 * nb * u + 16 * u
    pv = oracle_attention(q, k, _abs_stored(v, dtype), dtype, scale=scale, causal=causal, rows=rows)
    vmax = np.abs(oracle.decode(np.ascontiguousarray(v), dtype)).max(axis=2, keepdims=True)
    uo = U[out]
    ui = U[dtype]
    return uo * np.abs(ref) + (1 + uo) * ((2 * ui / (1 - ui) + 2 * rho) * pv + 2 * nk * ETA[dtype] * vmax)


def _run(q, k, v, dtype, out, scale, causal, layout="bhnd", tail=0):
    """Device copies in the given layout (bhnd packed; bhnd_odd: rows d + 1
    elements apart, the extra element NaN; bnhd: [B, n, H, d] memory seen
    through a permuted view), `tail` NaN rows after every head's n_q / n_k
    rows, a NaN-filled output; returns (o, untouched-guard ok)."""
    import torch
    from gpu_helpers import TORCH
    B, H, nq, d = q.shape
    nk = k.shape[2]

    def place(x, n, dt, fill=float("nan")):
        if layout == "bhnd":
            buf = torch.full((B, H, n + tail, d), fill, dtype=TORCH[dt], device="cuda:0")
            view = buf[:, :, :n, :]
        elif layout == "bhnd_odd":  # rows d + 1 elements apart: odd strides, rows 2-byte aligned
            buf = torch.full((B, H, n + tail, d + 1), fill, dtype=TORCH[dt], device="cuda:0")
            view = buf[:, :, :n, :d]
        else:
            buf = torch.full((B, n + tail, H, d), fill, dtype=TORCH[dt], device="cuda:0")
            view = buf[:, :n, :, :].permute(0, 2, 1, 3)
        if x is not None:
            view.copy_(_dev(x, dt))
        return buf, view

    _, qd = place(q, nq, dtype)
    _, kd = place(k, nk, dtype)
    _, vd = place(v, nk, dtype)
    obuf, od = place(None, nq, out, fill=12345.0)
    T.attention_tensors(qd, kd, vd, od, scale=scale, causal=causal)
    torch.cuda.synchronize()
    # the tail rows of the output buffer are never written
    if layout == "bhnd":
        guard = obuf[:, :, nq:, :]
    elif layout == "bhnd_odd":
        guard = torch.cat([obuf[:, :, nq:, :].flatten(), obuf[:, :, :nq, d:].flatten()])
    else:
        guard = obuf[:, nq:, :, :]
    untouched = bool(torch.all(guard == 12345.0).item()) if guard.numel() else True
    return od.to("cpu").to(torch.float64).numpy(), untouched


def _check(o, ref, bound, label):
    assert np.all(np.isfinite(o)), f"{label}: non-finite output"
    err = np.abs(o - ref)
    worst = np.unravel_index(np.argmax(err - bound), err.shape)
    assert np.all(err <= bound), (f"{label}: |o - r| = {err[worst]:.3e} > bound {bound[worst]:.3e} at {worst} "
                                  f"(o {o[worst]!r}, r {ref[worst]!r})")
    from gpu_helpers import say
    say(f"[attention] {label}: max |o - r| {err.max():.3e}, max |o - r| / bound {(err / bound).max():.3f}")


CASES = [
    # B, H, n_q, n_k, d, in, out, scale, causal, layout, tail, tile rows / 32 (1: keys split over waves)
    (1, 2, 200, 300, 64, W.F16, W.F16, 0.125, False, "bhnd", 0, 1),
    (2, 1, 130, 130, 128, W.BF16, W.F32, 128 ** -0.5, True, "bhnd", 3, 4),
    (1, 1, 64, 64, 64, W.F16, W.F32, 1.0, True, "bhnd", 0, 1),
    (1, 3, 1, 1, 64, W.F16, W.F16, 1.0, False, "bhnd", 5, 1),
    (1, 2, 100, 40, 128, W.F16, W.F32, 0.1, True, "bnhd", 7, 4),     # more queries than keys, causal
    (1, 2, 40, 200, 64, W.BF16, W.BF16, 0.125, True, "bnhd", 0, 1),  # fewer queries than keys, causal
    (2, 2, 65, 1, 64, W.BF16, W.F32, 2.0, False, "bhnd", 64, 1),     # one key: o = v_0
    (1, 1, 257, 513, 128, W.F16, W.F16, 128 ** -0.5, False, "bnhd", 1, 4),
    (1, 4, 192, 192, 64, W.BF16, W.F32, 1.0, False, "bhnd", 0, 1),   # the pages' unscaled softmax(QK^T)V
    (1, 4, 130, 140, 64, W.F16, W.F32, -0.3, False, "bhnd", 0, 1),   # negative scale
    (1, 130, 100, 77, 128, W.F16, W.F16, 0.2, True, "bhnd", 0, 4),   # head_dim 128: always 4 waves
    (1, 130, 100, 77, 64, W.F16, W.F16, 0.2, True, "bhnd", 0, 1),
    (2, 65, 100, 300, 64, W.BF16, W.BF16, 0.125, False, "bnhd", 1, 1),
    (1, 256, 65, 70, 64, W.F16, W.F16, 0.125, True, "bhnd", 0, 4),
    (2, 128, 130, 129, 128, W.BF16, W.F32, 128 ** -0.5, False, "bnhd", 2, 4),
    (1, 3, 100, 77, 64, W.F16, W.F32, 0.0, False, "bhnd", 0, 1),     # scale 0: the mean of V
    (1, 3, 100, 77, 64, W.F16, W.F32, 0.0, True, "bhnd", 0, 1),      # scale 0, causal: running means
    (2, 2, 300, 300, 128, W.BF16, W.BF16, 128 ** -0.5, True, "bnhd", 3, 4),
    (1, 2, 97, 449, 64, W.F16, W.F16, 0.125, False, "bhnd", 2, 1),   # 8 key blocks split over two waves
    (1, 2, 300, 300, 64, W.BF16, W.F32, 0.125, True, "bnhd", 0, 1),  # split, causal, tiles along the diagonal
    (1, 2, 130, 140, 64, W.F16, W.F16, 0.125, False, "bhnd_odd", 1, 1),         # odd row strides (65)
    (1, 3, 200, 333, 128, W.BF16, W.F32, 128 ** -0.5, True, "bhnd_odd", 2, 4),  # odd row strides (129)
    # causal, 64 tiles in 8 XCD runs of 2 whole heads: longest tiles first
    # across the heads of a run
    (2, 8, 512, 512, 128, W.F16, W.F16, 128 ** -0.5, True, "bhnd", 0, 4),
]


@pytest.mark.gpu
@pytest.mark.parametrize("case", CASES, ids=lambda c: "b%d_h%d_q%d_k%d_d%d_in%d_out%d_%s%s_w%d" % (
    c[0], c[1], c[2], c[3], c[4], c[5], c[6], "causal" if c[8] else "full", "_" + c[9], c[11]))
def test_attention_parity_full(case):
    from gpu_helpers import say
    B, H, nq, nk, d, dt, out, scale, causal, layout, tail, waves = case
    assert T.attention_waves(B, H, nq, d) == waves  # the case runs the tile shape it is meant to cover
    say(f"[attention] case {case}")
    q, k, v = W.attention_inputs(B, H, nq, nk, d, dt, seed=1000 + nq + nk + d)
    o, untouched = _run(q, k, v, dt, out, scale, causal, layout, tail)
    assert untouched, "rows past n_q were written"
    ref = oracle_attention(q, k, v, dt, scale=scale, causal=causal)
    _check(o, ref, _bound(q, k, v, ref, dt, out, scale, causal), str(case))
    if nk == 1:  # closed form: the only key gets weight 1
        vv = oracle.decode(np.ascontiguousarray(v), dt)
        assert np.all(np.abs(o - vv) <= U[out] * np.abs(vv))


@pytest.mark.gpu
@pytest.mark.parametrize("w", W.ATTN_WORKLOADS, ids=lambda w: w.name)
def test_attention_parity_workloads_sampled(w):
    """The benchmark's workloads at full size (the kernel bench.py times),
    checked on sampled query rows of every (batch, head), the first and last
    row included."""
    import torch
    from gpu_helpers import say
    say(f"[attention] workload {w.name}")
    q, k, v = W.attention_inputs(w.B, w.H, w.N, w.N, w.d, w.dtype, seed=77)
    qd, kd, vd = _dev(q, w.dtype), _dev(k, w.dtype), _dev(v, w.dtype)
    od = torch.empty_like(qd)
    T.attention_tensors(qd, kd, vd, od, scale=w.scale, causal=w.causal)
    torch.cuda.synchronize()
    rows = W.sample_indices(w.N, 12, seed=5)
    o = od[:, :, torch.from_numpy(rows).to("cuda:0"), :].to("cpu").to(torch.float64).numpy()
    ref = oracle_attention(q, k, v, w.dtype, scale=w.scale, causal=w.causal, rows=rows)
    _check(o, ref, _bound(q, k, v, ref, w.dtype, w.dtype, w.scale, w.causal, rows=rows), w.name)


@pytest.mark.gpu
def test_attention_causal_first_row_is_first_value():
    """Causal: query 0 sees only key 0, so its output is v_0 rounded once."""
    import torch
    q, k, v = W.attention_inputs(1, 2, 70, 70, 64, W.F16, seed=9)
    o, _ = _run(q, k, v, W.F16, W.F32, 0.3, True)
    vv = oracle.decode(np.ascontiguousarray(v), W.F16)
    assert np.array_equal(o[:, :, 0, :], vv[:, :, 0, :])


@pytest.mark.gpu
def test_attention_rejects_before_launch_on_device_tensors():
    import torch
    q = torch.zeros(1, 1, 8, 64, dtype=torch.float16, device="cuda:0")
    o = torch.zeros(1, 1, 8, 64, dtype=torch.float16, device="cuda:0")
    rc = T.attention_tensors(q, q, q, q, check=False)  # output is the input
    assert rc == T.ERR_ALIAS
    q32 = torch.zeros(1, 1, 8, 32, dtype=torch.float16, device="cuda:0")
    o32 = torch.zeros(1, 1, 8, 32, dtype=torch.float16, device="cuda:0")
    assert T.attention_tensors(q32, q32, q32, o32, check=False) == T.ERR_HEAD_DIM
    assert torch.all(o == 0).item()


def _random_case(seed):
    """One seeded draw of every argument the kernel takes: head size, types,
    batch and heads, ragged query and key counts, scale and its sign, the
    causal mask, the memory layout and the rows after each head's."""
    rng = np.random.default_rng(5000 + seed)
    d = int(rng.choice([64, 128]))
    dt = int(rng.choice([W.F16, W.BF16]))
    out = int(rng.choice([dt, W.F32]))
    B, H = int(rng.integers(1, 3)), int(rng.integers(1, 7))
    nq, nk = int(rng.integers(1, 400)), int(rng.integers(1, 400))
    scale = float(rng.choice([d ** -0.5, 0.125, 1.0, -0.25]))
    causal = bool(rng.random() < 0.5)
    layout = str(rng.choice(["bhnd", "bnhd", "bhnd_odd"]))
    tail = int(rng.choice([0, 1, 5]))
    return B, H, nq, nk, d, dt, out, scale, causal, layout, tail


@pytest.mark.gpu
@pytest.mark.parametrize("seed", range(32))
def test_attention_random_sweep(seed):
    """Seeded random calls, each held to the bound of the full-parity cases,
    with the rows past each head's queries left unwritten."""
    from gpu_helpers import say
    case = _random_case(seed)
    B, H, nq, nk, d, dt, out, scale, causal, layout, tail = case
    say(f"[attention] sweep {seed}: {case}")
    q, k, v = W.attention_inputs(B, H, nq, nk, d, dt, seed=seed)
    o, untouched = _run(q, k, v, dt, out, scale, causal, layout, tail)
    assert untouched, "rows past n_q were written"
    ref = oracle_attention(q, k, v, dt, scale=scale, causal=causal)
    _check(o, ref, _bound(q, k, v, ref, dt, out, scale, causal), str(case))
