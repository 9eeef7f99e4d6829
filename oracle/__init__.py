"""Reference (oracle) matrix product for the tests -- TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and the cpu_baseline leg of bench.py may
import this package.  The GPU library (tiled_gemm_03_amd) never imports it and
it never imports the GPU library.

`gemm(a, b, dtype)` returns the binary64 product C[i, j] = sum_k a(i,k) b(k,j)
of the exact stored values of a and b (see oracle_gemm.c for the definition,
the decoders and the summation order).  `decode(bits, dtype)` exposes the
decoders so that they can be pinned on their own.
"""
import ctypes
import os

import numpy as np

from . import build as _build

BINARY32, BINARY16, BFLOAT16 = 0, 1, 2
_NAMES = {"f32": BINARY32, "f16": BINARY16, "bf16": BFLOAT16}

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
    bfloat16, uint32 bits or float32 for binary32)."""
    code = dtype_code(dtype)
    lib = _load(lib_path)
    x = np.ascontiguousarray(bits)
    out = np.empty(x.size, dtype=np.float64)
    if lib.oracle_decode_array(x.ctypes.data, code, x.size, out.ctypes.data) != 0:
        raise ValueError("bad dtype")
    return out.reshape(x.shape)
