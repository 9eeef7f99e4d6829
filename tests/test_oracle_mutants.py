"""Planted mistakes: copies of the oracle source, each with one plausible
mistake, are compiled and run against the pins in a child process; every
copy must fail at least one pin.  The mistakes live only in temporary copies
on the CPU; the oracle itself is unchanged."""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path.insert(0, ROOT)
from oracle import build as obuild  # noqa: E402

# (name, text in oracle_gemm.c, replacement)
MUTANTS = [
    ("dropped_first_term", "for (int64_t k = 0; k < jb->K; ++k) {", "for (int64_t k = 1; k < jb->K; ++k) {"),
    ("dropped_last_term", "for (int64_t k = 0; k < jb->K; ++k) {", "for (int64_t k = 0; k + 1 < jb->K; ++k) {"),
    ("transposed_b", "decode_one(B, k * ldb + j, dtype)", "decode_one(B, j * ldb + k, dtype)"),
    ("a_stride_ignores_lda", "decode_one(A, i * lda + k, dtype)", "decode_one(A, i * K + k, dtype)"),
    ("b_stride_uses_n", "decode_one(B, k * ldb + j, dtype)", "decode_one(B, k * ncols + j, dtype)"),
    ("wrong_sign", "s[c] += a * brow[c];", "s[c] -= a * brow[c];"),
    ("no_zero_init", "for (int64_t c = 0; c < jb->ncols; ++c) s[c] = 0.0;", ""),
    ("f16_subnormal_scale", "v = ldexp((double)f, -24);", "v = ldexp((double)f, -25);"),
    ("f16_bias", "v = ldexp((double)(1024 + f), e - 25);", "v = ldexp((double)(1024 + f), e - 24);"),
    ("f16_inf_as_nan", "v = f ? NAN : INFINITY;\n    else\n        v = ldexp((double)(1024", "v = NAN;\n    else\n        v = ldexp((double)(1024"),
    ("bf16_exponent_field", "int e = (h >> 7) & 0xff;", "int e = (h >> 8) & 0xff;"),
    ("bf16_subnormal_scale", "v = ldexp((double)f, -133);", "v = ldexp((double)f, -134);"),
    ("f32_bias", "v = ldexp((double)(8388608u + f), e - 150);", "v = ldexp((double)(8388608u + f), e - 149);"),
    ("sampled_rows_ignored", "const int64_t i = rows ? rows[r] : r;", "const int64_t i = r;"),
    ("sampled_cols_ignored", "const int64_t j = cols ? cols[c] : c;", "const int64_t j = c;"),
    ("a_times_a", "s[c] += a * brow[c];", "s[c] += a * a;"),
    ("skips_last_row", "for (int64_t r = jb->tid; r < jb->nrows; r += jb->nthreads) {",
     "for (int64_t r = jb->tid; r + 1 < jb->nrows; r += jb->nthreads) {"),
    # the fused epilogue
    ("alpha_ignored", "double t = alpha * s[r * lds + c];", "double t = s[r * lds + c];"),
    ("beta_sign", "t += beta * c_old[r * ldco + c];", "t -= beta * c_old[r * ldco + c];"),
    ("c_read_when_beta_zero", "if (beta != 0.0) t += beta", "t += beta"),
    ("bias_row_indexed_by_column", "if (bias_row) t += bias_row[r];", "if (bias_row) t += bias_row[c];"),
    ("activation_before_bias", "out[r * ldo + c] = oracle_activation(t, act);",
     "out[r * ldo + c] = oracle_activation(t - (bias_row ? bias_row[r] : bias_col ? bias_col[c] : 0.0), act) + (bias_row ? bias_row[r] : bias_col ? bias_col[c] : 0.0);"),
    ("gelu_wrong_scale", "erf(x / sqrt(2.0))", "erf(x * sqrt(2.0))"),
    ("gelu_tanh_cubic_term", "0.044715 * x * x * x", "0.044715 * x * x"),
    ("silu_sign", "return x / (1.0 + exp(-x));", "return x / (1.0 + exp(x));"),
    ("relu_inverted", "return x > 0.0 ? x : 0.0;", "return x < 0.0 ? x : 0.0;"),
    # the 8-bit output formats
    ("fp8_e4m3_bias", "const int bias = fmt == ORACLE_FP8_E4M3 ? 7 : 15;",
     "const int bias = fmt == ORACLE_FP8_E4M3 ? 8 : 15;"),
    ("fp8_e4m3_nan_as_number", "else if (fmt == ORACLE_FP8_E4M3 && e == 15 && f == 7)\n        v = NAN;", ""),
    ("fp8_subnormal_scale", "v = ldexp((double)f, 1 - bias - F);", "v = ldexp((double)f, -bias - F);"),
    ("fp8_truncates", "const double v = rint(a / q) * q;", "const double v = floor(a / q) * q;"),
    ("fp8_ties_away", "const double v = rint(a / q) * q;", "const double v = round(a / q) * q;"),
    ("fp8_no_saturation", "if (a > maxfin) a = maxfin;", ""),
    ("fp8_sign_dropped", "const uint8_t s = signbit(x) ? 0x80 : 0;", "const uint8_t s = 0;"),
    ("fp8_e5m2_fraction_bits", "const int F = fmt == ORACLE_FP8_E4M3 ? 3 : 2;\n    const int bias = fmt == ORACLE_FP8_E4M3 ? 7 : 15;\n    const double maxfin",
     "const int F = fmt == ORACLE_FP8_E4M3 ? 3 : 3;\n    const int bias = fmt == ORACLE_FP8_E4M3 ? 7 : 15;\n    const double maxfin"),
]

RUNNER = r"""
import sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
import oracle_pins as P
failed = []
for pin in P.FAST_PINS:
    try:
        pin({lib!r})
    except Exception as e:
        failed.append(pin.__name__)
print("FAILED:", ",".join(failed))
sys.exit(1 if failed else 0)
"""


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(name, old, new, tmp_path):
    src = open(obuild.SRC, encoding="utf-8").read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    mutated = src.replace(old, new, 1)
    cpath = tmp_path / "oracle_mut.c"
    cpath.write_text(mutated, encoding="utf-8")
    lib = str(tmp_path / "liboracle_mut.so")
    obuild.build(str(cpath), lib)
    code = RUNNER.format(root=ROOT, tests=HERE, lib=lib)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"mutant {name} passed every pin:\n{r.stdout}\n{r.stderr}"


def test_unmutated_copy_passes(tmp_path):
    """Control: the same harness on an untouched copy passes every pin."""
    lib = str(tmp_path / "liboracle_copy.so")
    obuild.build(obuild.SRC, lib)
    code = RUNNER.format(root=ROOT, tests=HERE, lib=lib)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr


# Planted mistakes in the attention oracle (oracle/attention.py): a mutated
# copy is loaded as a module of its own and must fail one of the attention
# pins.
ATTENTION_MUTANTS = [
    ("scores_use_v", "np.swapaxes(K, 2, 3)", "np.swapaxes(V, 2, 3)"),
    ("scale_dropped", "S = scale * np.matmul", "S = np.matmul"),
    ("causal_hides_diagonal", "np.arange(Nk)[None, :] > ri[:, None]", "np.arange(Nk)[None, :] >= ri[:, None]"),
    ("causal_upper_triangle", "np.arange(Nk)[None, :] > ri[:, None]", "np.arange(Nk)[None, :] < ri[:, None]"),
    ("max_over_queries", "m = np.max(S, axis=3, keepdims=True)", "m = np.max(S, axis=2, keepdims=True)"),
    ("normalised_over_queries", "np.sum(E, axis=3, keepdims=True)", "np.sum(E, axis=2, keepdims=True)"),
    ("weights_times_k", "return np.matmul(P, V)", "return np.matmul(P, K)"),
    ("sampled_rows_ignored", "Qr = Q[:, :, ri, :]", "Qr = Q[:, :, :len(ri), :]"),
]


@pytest.mark.parametrize("name,old,new", ATTENTION_MUTANTS, ids=[m[0] for m in ATTENTION_MUTANTS])
def test_planted_attention_mistake_is_caught(name, old, new, tmp_path):
    import importlib.util
    import attention_pins as AP
    import oracle.attention as OA
    src = open(OA.__file__, encoding="utf-8").read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    path = tmp_path / "attention_mut.py"
    path.write_text(src.replace(old, new, 1).replace("from . import decode", "from oracle import decode"),
                    encoding="utf-8")
    spec = importlib.util.spec_from_file_location("attention_mut", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    failed = []
    for pin in AP.ATTENTION_PINS:
        try:
            pin(mod.attention)
        except Exception:
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every attention pin"
