"""Reference (oracle) matrix product for the tests -- TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and the cpu_baseline leg of bench.py may
import this package.  The GPU library (tiled_gemm_03_amd) never imports it and
it never imports the GPU library.

`gemm(a, b, dtype)` returns the binary64 product C[i, j] = sum_k a(i,k) b(k,j)
of the exact stored values of a and b (see oracle_gemm.c for the definition,
the decoders and the summation order).  `decode(bits, dtype)` exposes the
decoders so that they can be pinned on their own.  `epilogue(...)` and
`gemm_fused(...)` add the fused epilogue act(alpha P + beta C_old + bias)
(oracle_gemm.c, oracle_epilogue).
"""
import ctypes
import os

import numpy as np

from . import build as _build

BINARY32, BINARY16, BFLOAT16, FP8_E4M3, FP8_E5M2 = 0, 1, 2, 3, 4
ACT_NONE, ACT_RELU, ACT_GELU, ACT_GELU_TANH, ACT_SILU = 0, 1, 2, 3, 4
BIAS_NONE, BIAS_ROW, BIAS_COL = 0, 1, 2
_NAMES = {"f32": BINARY32, "f16": BINARY16, "bf16": BFLOAT16, "e4m3": FP8_E4M3, "e5m2": FP8_E5M2}

_lib = None


def _load(path=None):
    global _lib
    if path is not None:
        lib = ctypes.CDLL(path)
    else:
        if _lib is not None:
            return _lib
        if not os.path.exists(_build.LIB):
            _build.build()
        lib = ctypes.CDLL(_build.LIB)
    i64, p = ctypes.c_int64, ctypes.c_void_p
    lib.oracle_gemm.restype = ctypes.c_int
    lib.oracle_gemm.argtypes = [i64, i64, i64, p, i64, p, i64, ctypes.c_int,
                                p, i64, p, i64, p, i64, ctypes.c_int]
    lib.oracle_decode_array.restype = ctypes.c_int
    lib.oracle_decode_array.argtypes = [p, ctypes.c_int, i64, p]
    lib.oracle_encode_fp8_array.restype = ctypes.c_int
    lib.oracle_encode_fp8_array.argtypes = [p, ctypes.c_int, i64, p]
    d = ctypes.c_double
    lib.oracle_activation.restype = d
    lib.oracle_activation.argtypes = [d, ctypes.c_int]
    lib.oracle_epilogue.restype = ctypes.c_int
    lib.oracle_epilogue.argtypes = [i64, i64, p, i64, d, d, p, i64, p, p, ctypes.c_int, p, i64]
    if path is None:
        _lib = lib
    return lib


def dtype_code(dtype) -> int:
    if isinstance(dtype, int):
        return dtype
    return _NAMES[dtype]


def _operand(x: np.ndarray, code: int):
    """Pointer and leading dimension (in elements) of a row-major 2-D array
    whose rows may be padded (row stride >= width)."""
    want = np.uint32 if code == BINARY32 else np.uint16
    if x.dtype.itemsize != np.dtype(want).itemsize:
        raise TypeError(f"operand of itemsize {x.dtype.itemsize} for dtype code {code}")
    if x.ndim == 2 and x.size == 0:
        return x.ctypes.data, x.shape[1]
    if x.ndim != 2 or x.strides[1] != x.itemsize or x.strides[0] % x.itemsize:
        raise ValueError("operand must be a 2-D array with unit column stride")
    ld = x.strides[0] // x.itemsize if x.shape[0] > 1 else x.shape[1]
    return x.ctypes.data, max(ld, x.shape[1])


def gemm(a: np.ndarray, b: np.ndarray, dtype, rows=None, cols=None,
         nthreads: int = 1, lib_path=None) -> np.ndarray:
    """C[r, c] = sum_k a(rows[r], k) * b(k, cols[c]) in binary64.

    a: M x K and b: K x N arrays holding the STORED bits of the inputs
    (float16 / float32 arrays, or uint16 arrays of bfloat16 bits).  Rows may be
    padded (leading dimension larger than the width).  rows / cols select a
    subset of output entries (None: all).
    """
    code = dtype_code(dtype)
    lib = _load(lib_path)
    M, K = a.shape
    K2, N = b.shape
    if K2 != K:
        raise ValueError(f"inner sizes differ: {a.shape} x {b.shape}")
    pa, lda = _operand(a, code)
    pb, ldb = _operand(b, code)
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    c = None if cols is None else np.ascontiguousarray(cols, dtype=np.int64)
    nr = M if r is None else r.size
    nc = N if c is None else c.size
    out = np.empty((nr, nc), dtype=np.float64)
    rc = lib.oracle_gemm(M, N, K, pa, lda, pb, ldb, code,
                         None if r is None else r.ctypes.data, nr,
                         None if c is None else c.ctypes.data, nc,
                         out.ctypes.data, max(nc, 1), int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_gemm rejected its arguments (code {rc})")
    return out


def decode(bits: np.ndarray, dtype, lib_path=None) -> np.ndarray:
    """binary64 values of stored elements (uint16 bits for binary16 and
    bfloat16, uint32 bits or float32 for binary32, uint8 bits for the 8-bit
    formats FP8_E4M3 and FP8_E5M2)."""
    code = dtype_code(dtype)
    lib = _load(lib_path)
    x = np.ascontiguousarray(bits)
    out = np.empty(x.size, dtype=np.float64)
    if lib.oracle_decode_array(x.ctypes.data, code, x.size, out.ctypes.data) != 0:
        raise ValueError("bad dtype")
    return out.reshape(x.shape)


def encode_fp8(values, fmt, lib_path=None) -> np.ndarray:
    """uint8 patterns of binary64 values rounded to FP8_E4M3 or FP8_E5M2
    (nearest, ties to even; beyond the largest finite value, infinities
    included, the largest finite value of the sign; NaN stays NaN)."""
    code = dtype_code(fmt)
    lib = _load(lib_path)
    x = np.ascontiguousarray(values, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint8)
    if lib.oracle_encode_fp8_array(x.ctypes.data, code, x.size, out.ctypes.data) != 0:
        raise ValueError("bad 8-bit format")
    return out


def activation(x, act: int, lib_path=None) -> np.ndarray:
    """act(x) in binary64 for an array of values (oracle_activation)."""
    lib = _load(lib_path)
    x = np.asarray(x, dtype=np.float64)
    out = np.array([lib.oracle_activation(float(v), int(act)) for v in x.ravel()], dtype=np.float64)
    return out.reshape(x.shape)


def epilogue(s: np.ndarray, alpha=1.0, beta=0.0, c_old=None, bias=None, bias_kind=BIAS_NONE, act=ACT_NONE,
             lib_path=None) -> np.ndarray:
    """act(alpha * s + beta * c_old + bias) in binary64 (oracle_epilogue).

    s: binary64 product values (nr x nc); c_old: binary64 values of the same
    entries of C (read only when beta != 0); bias: binary64 vector, one value
    per row of s (bias_kind BIAS_ROW) or per column (BIAS_COL)."""
    lib = _load(lib_path)
    s = np.ascontiguousarray(s, dtype=np.float64)
    nr, nc = s.shape
    out = np.empty((nr, nc), dtype=np.float64)
    co = None if c_old is None else np.ascontiguousarray(c_old, dtype=np.float64)
    if co is not None and co.shape != s.shape:
        raise ValueError("c_old must have the shape of s")
    bv = None if bias is None or bias_kind == BIAS_NONE else np.ascontiguousarray(bias, dtype=np.float64)
    if bv is not None and bv.size != (nr if bias_kind == BIAS_ROW else nc):
        raise ValueError("bias length does not match its kind")
    brow = bv.ctypes.data if bv is not None and bias_kind == BIAS_ROW else None
    bcol = bv.ctypes.data if bv is not None and bias_kind == BIAS_COL else None
    rc = lib.oracle_epilogue(nr, nc, s.ctypes.data, max(nc, 1), float(alpha), float(beta),
                             None if co is None else co.ctypes.data, max(nc, 1), brow, bcol, int(act),
                             out.ctypes.data, max(nc, 1))
    if rc != 0:
        raise ValueError(f"oracle_epilogue rejected its arguments (code {rc})")
    return out


def gemm_fused(a, b, dtype, alpha=1.0, beta=0.0, c_old=None, out_dtype=None, bias=None, bias_dtype=None,
               bias_kind=BIAS_NONE, act=ACT_NONE, rows=None, cols=None, nthreads: int = 1, lib_path=None):
    """act(alpha * (a x b) + beta * c_old + bias) in binary64 on the requested
    entries.  c_old: the STORED bits of the whole M x N output (of out_dtype),
    read only when beta != 0; bias: stored bits of a vector of bias_dtype, M
    values (BIAS_ROW) or N values (BIAS_COL)."""
    s = gemm(a, b, dtype, rows=rows, cols=cols, nthreads=nthreads, lib_path=lib_path)
    M, N = a.shape[0], b.shape[1]
    ri = np.arange(M) if rows is None else np.asarray(rows)
    ci = np.arange(N) if cols is None else np.asarray(cols)
    co = None
    if beta != 0.0:
        co = decode(np.ascontiguousarray(c_old), out_dtype, lib_path=lib_path)[np.ix_(ri, ci)]
    bv = None
    if bias_kind != BIAS_NONE:
        full = decode(np.ascontiguousarray(bias).ravel(), bias_dtype, lib_path=lib_path)
        bv = full[ri] if bias_kind == BIAS_ROW else full[ci]
    return epilogue(s, alpha, beta, co, bv, bias_kind, act, lib_path=lib_path)
