"""Python binding of libtgemm.so, the gfx950 tiled matrix-product library.

Argument marshalling only: every function here forwards to the C entry point
of the same name declared in include/tgemm.h; all computation happens in the
library's HIP kernels.  There is no fallback: if the library has not been
built, loading fails with an error that says so.

    gemm(M, N, K, A, lda, B, ldb, C, ldc, in_dtype, out_dtype, stream)
    gemm_ex(..., config_id)
    gemm_strerror(code), gemm_num_configs(), gemm_config_info(id),
    gemm_select_config(...), gemm_tile_map(...), gemm_version()
    attention_fwd(B, H, n_q, n_k, d, Q, q_stride, K, k_stride, V, v_stride,
                  O, o_stride, in_dtype, out_dtype, scale, causal, stream)
        (include/tgemm_attention.h)

`gemm_tensors(a, b, c)` and `attention_tensors(q, k, v, o)` take torch device
tensors and pass their pointers, strides and the current HIP stream; torch
provides only the memory and the stream.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libtgemm.so")

F32, F16, BF16, FP8_E4M3, FP8_E5M2 = 0, 1, 2, 3, 4
OK = 0
ERR_DIM, ERR_NULL, ERR_LD, ERR_DTYPE, ERR_ALIAS, ERR_CONFIG, ERR_LAYOUT, ERR_EPILOGUE = -1, -2, -3, -4, -5, -6, -7, -8
ERR_HEAD_DIM = -9
ERR_SCRATCH = -10
ERR_ALIGN = -11

EXPORTED = ["gemm", "gemm_ex", "gemm_t", "gemm_fused", "gemm_fused_noalloc", "gemm_strerror", "gemm_num_configs",
            "gemm_config_info",
            "gemm_select_config", "gemm_select_kernel", "gemm_select_kernel_t", "gemm_split_count_t",
            "gemm_tile_map", "gemm_version",
            "attention_fwd", "attention_waves"]

# operand layouts (gemm_t)
ROW_MAJOR, COL_MAJOR = 0, 1

# fused epilogue (gemm_fused): activations and bias kinds
ACT_NONE, ACT_RELU, ACT_GELU, ACT_GELU_TANH, ACT_SILU = 0, 1, 2, 3, 4
BIAS_NONE, BIAS_ROW, BIAS_COL = 0, 1, 2

# gemm_select_kernel results
KERNEL_GENERAL, KERNEL_TILED, KERNEL_RING, KERNEL_DIRECT, KERNEL_RING_SPLITK = 0, 1, 2, 3, 4


class ConfigInfo(ctypes.Structure):
    _fields_ = [("id", ctypes.c_int), ("in_dtype", ctypes.c_int),
                ("block_m", ctypes.c_int), ("block_n", ctypes.c_int), ("block_k", ctypes.c_int),
                ("stages", ctypes.c_int), ("threads", ctypes.c_int),
                ("waves_m", ctypes.c_int), ("waves_n", ctypes.c_int),
                ("mfma_m", ctypes.c_int), ("mfma_n", ctypes.c_int), ("mfma_k", ctypes.c_int),
                ("lds_bytes", ctypes.c_int), ("name", ctypes.c_char_p),
                ("a_block_k", ctypes.c_int), ("a_stages", ctypes.c_int)]

    def as_dict(self):
        d = {f: getattr(self, f) for f, _ in self._fields_}
        d["name"] = d["name"].decode()
        return d


class Epilogue(ctypes.Structure):
    """tgemm_epilogue: C := act(alpha * AB + beta * C + bias)."""
    _fields_ = [("alpha", ctypes.c_float), ("beta", ctypes.c_float), ("bias", ctypes.c_void_p),
                ("bias_kind", ctypes.c_int), ("bias_dtype", ctypes.c_int), ("activation", ctypes.c_int)]


class TgemmError(RuntimeError):
    def __init__(self, code):
        super().__init__(f"tgemm error {code}: {gemm_strerror(code)}")
        self.code = code


_lib = None


def lib():
    """The loaded libtgemm.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                          "(there is no fallback path)")
    L = ctypes.CDLL(LIB_PATH)
    i64, p, i = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    L.gemm.restype = i
    L.gemm.argtypes = [i64, i64, i64, p, i64, p, i64, p, i64, i, i, p]
    L.gemm_ex.restype = i
    L.gemm_ex.argtypes = [i64, i64, i64, p, i64, p, i64, p, i64, i, i, p, i]
    L.gemm_strerror.restype = ctypes.c_char_p
    L.gemm_strerror.argtypes = [i]
    L.gemm_num_configs.restype = i
    L.gemm_num_configs.argtypes = []
    L.gemm_config_info.restype = i
    L.gemm_config_info.argtypes = [i, ctypes.POINTER(ConfigInfo)]
    L.gemm_select_config.restype = i
    L.gemm_select_config.argtypes = [i64, i64, i64, p, i64, p, i64, p, i64, i, i]
    L.gemm_t.restype = i
    L.gemm_t.argtypes = [i64, i64, i64, p, i64, i, p, i64, i, p, i64, i, i, i, p, i]
    L.gemm_fused_noalloc.restype = i
    L.gemm_fused_noalloc.argtypes = [i64, i64, i64, p, i64, i, p, i64, i, p, i64, i, i, i, ctypes.POINTER(Epilogue), p,
                                     i]
    L.gemm_fused.restype = i
    L.gemm_fused.argtypes = [i64, i64, i64, p, i64, i, p, i64, i, p, i64, i, i, i, ctypes.POINTER(Epilogue), p, i]
    L.gemm_select_kernel_t.restype = i
    L.gemm_select_kernel_t.argtypes = [i64, i64, i64, p, i64, i, p, i64, i, p, i64, i, i, i, i, ctypes.POINTER(i)]
    L.gemm_split_count_t.restype = i
    L.gemm_split_count_t.argtypes = [i64, i64, i64, p, i64, i, p, i64, i, p, i64, i, i, i]
    L.gemm_select_kernel.restype = i
    L.gemm_select_kernel.argtypes = [i64, i64, i64, p, i64, p, i64, p, i64, i, i, i]
    L.gemm_tile_map.restype = i
    L.gemm_tile_map.argtypes = [i, i, i, i, ctypes.POINTER(i), ctypes.POINTER(i)]
    L.gemm_version.restype = ctypes.c_char_p
    L.gemm_version.argtypes = []
    s3 = ctypes.POINTER(i64)
    L.attention_fwd.restype = i
    L.attention_fwd.argtypes = [i64, i64, i64, i64, i64, p, s3, p, s3, p, s3, p, s3, i, i, ctypes.c_float, i, p]
    L.attention_waves.restype = i
    L.attention_waves.argtypes = [i64, i64, i64, i64]
    _lib = L
    return L


def gemm(M, N, K, A, lda, B, ldb, C, ldc, in_dtype, out_dtype, stream=None):
    return lib().gemm(M, N, K, A, lda, B, ldb, C, ldc, in_dtype, out_dtype, stream)


def gemm_ex(M, N, K, A, lda, B, ldb, C, ldc, in_dtype, out_dtype, stream=None, config_id=-1):
    return lib().gemm_ex(M, N, K, A, lda, B, ldb, C, ldc, in_dtype, out_dtype, stream, config_id)


def gemm_strerror(code):
    return lib().gemm_strerror(code).decode()


def gemm_num_configs():
    return lib().gemm_num_configs()


def gemm_config_info(config_id):
    info = ConfigInfo()
    rc = lib().gemm_config_info(config_id, ctypes.byref(info))
    if rc != OK:
        raise TgemmError(rc)
    return info.as_dict()


def gemm_select_config(M, N, K, A, lda, B, ldb, C, ldc, in_dtype, out_dtype):
    return lib().gemm_select_config(M, N, K, A, lda, B, ldb, C, ldc, in_dtype, out_dtype)


def gemm_t(M, N, K, A, lda, layout_a, B, ldb, layout_b, C, ldc, layout_c, in_dtype, out_dtype, stream=None,
           config_id=-1):
    return lib().gemm_t(M, N, K, A, lda, layout_a, B, ldb, layout_b, C, ldc, layout_c, in_dtype, out_dtype, stream,
                        config_id)


def gemm_fused(M, N, K, A, lda, layout_a, B, ldb, layout_b, C, ldc, layout_c, in_dtype, out_dtype, epilogue=None,
               stream=None, config_id=-1):
    """gemm_t with the fused epilogue (an Epilogue, or None for none)."""
    ep = ctypes.byref(epilogue) if epilogue is not None else None
    return lib().gemm_fused(M, N, K, A, lda, layout_a, B, ldb, layout_b, C, ldc, layout_c, in_dtype, out_dtype, ep,
                            stream, config_id)


def gemm_fused_noalloc(M, N, K, A, lda, layout_a, B, ldb, layout_b, C, ldc, layout_c, in_dtype, out_dtype,
                       epilogue=None, stream=None, config_id=-1):
    """gemm_fused that allocates nothing (the split-K workspace in the
    library's fixed scratch; calls overlapping on one GPU race)."""
    ep = ctypes.byref(epilogue) if epilogue is not None else None
    return lib().gemm_fused_noalloc(M, N, K, A, lda, layout_a, B, ldb, layout_b, C, ldc, layout_c, in_dtype,
                                    out_dtype, ep, stream, config_id)


def gemm_select_kernel_t(M, N, K, A, lda, layout_a, B, ldb, layout_b, C, ldc, layout_c, in_dtype, out_dtype,
                         config_id=-1):
    """(kernel kind or negative error, configuration that would run)."""
    cfg = ctypes.c_int(-1)
    k = lib().gemm_select_kernel_t(M, N, K, A, lda, layout_a, B, ldb, layout_b, C, ldc, layout_c, in_dtype,
                                   out_dtype, config_id, ctypes.byref(cfg))
    return k, cfg.value


def gemm_split_count_t(M, N, K, A, lda, layout_a, B, ldb, layout_b, C, ldc, layout_c, in_dtype, out_dtype):
    """K slices the table's choice would run (1: none), or a negative error."""
    return lib().gemm_split_count_t(M, N, K, A, lda, layout_a, B, ldb, layout_b, C, ldc, layout_c, in_dtype,
                                    out_dtype)


def gemm_select_kernel(M, N, K, A, lda, B, ldb, C, ldc, in_dtype, out_dtype, config_id=-1):
    return lib().gemm_select_kernel(M, N, K, A, lda, B, ldb, C, ldc, in_dtype, out_dtype, config_id)


def gemm_tile_map(bid, tiles_m, tiles_n, group_m):
    tm, tn = ctypes.c_int(-1), ctypes.c_int(-1)
    rc = lib().gemm_tile_map(bid, tiles_m, tiles_n, group_m, ctypes.byref(tm), ctypes.byref(tn))
    if rc != OK:
        raise TgemmError(rc)
    return tm.value, tn.value


def gemm_version():
    return lib().gemm_version().decode()


def _strides(st):
    """A host array of three int64 strides (batch, head, row), or None."""
    if st is None:
        return None
    return (ctypes.c_int64 * 3)(*[int(x) for x in st])


def attention_fwd(B, H, n_q, n_k, d, Q, q_stride, K, k_stride, V, v_stride, O, o_stride, in_dtype, out_dtype,
                  scale, causal, stream=None):
    """O := softmax(scale Q K^T [causal]) V; strides are 3-sequences or None
    (packed)."""
    return lib().attention_fwd(B, H, n_q, n_k, d, Q, _strides(q_stride), K, _strides(k_stride), V,
                               _strides(v_stride), O, _strides(o_stride), in_dtype, out_dtype, float(scale),
                               int(bool(causal)), stream)


def attention_waves(B, H, n_q, d):
    """Query rows per workgroup that attention_fwd launches, in units of 32:
    4, or 1 (two waves splitting the keys of 32 rows)."""
    return lib().attention_waves(B, H, n_q, d)


# ------------------------------------------------------------ torch marshalling
def dtype_code(t):
    import torch
    codes = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16,
             torch.float8_e4m3fn: FP8_E4M3, torch.float8_e5m2: FP8_E5M2}
    if t.dtype not in codes:
        raise TypeError(f"unsupported tensor dtype {t.dtype}")
    return codes[t.dtype]


def _ld(t):
    if t.dim() != 2:
        raise ValueError("expected a 2-D tensor")
    if t.shape[0] > 0 and t.shape[1] > 0 and t.stride(1) != 1:
        raise ValueError("tensor rows must be contiguous (unit column stride)")
    return max(t.stride(0) if t.shape[0] > 1 else t.shape[1], t.shape[1])


def _layout(t):
    """(layout, leading dimension) of a 2-D tensor: row-major when its rows
    are contiguous, column-major when its columns are (a transposed view)."""
    if t.dim() != 2:
        raise ValueError("expected a 2-D tensor")
    r, c = t.shape
    if r == 0 or c == 0 or t.stride(1) == 1:
        return ROW_MAJOR, max(t.stride(0) if r > 1 else c, c, 1)
    if t.stride(0) == 1:
        return COL_MAJOR, max(t.stride(1) if c > 1 else r, r, 1)
    raise ValueError("tensor needs contiguous rows or contiguous columns")


def gemm_tensors(a, b, c, config_id=-1, stream=None, check=True, alpha=None, beta=None, bias=None,
                 bias_kind=None, activation=ACT_NONE):
    """c := a @ b on the device, through the C ABI.  a: M x K, b: K x N,
    c: M x N torch tensors on the GPU, each with contiguous rows (row-major,
    rows may be padded) or contiguous columns (column-major, e.g. a
    transposed view).  With any of alpha, beta, bias or activation given, the
    fused epilogue c := act(alpha * a @ b + beta * c + bias) runs
    (gemm_fused); bias is a contiguous 1-D tensor of M values (one per row of
    c, bias_kind BIAS_ROW) or N values (per column, BIAS_COL, the default for
    a bias of N values).  Returns the library's return code (raises
    TgemmError on failure if check)."""
    import torch
    M, K = a.shape
    K2, N = b.shape
    if K2 != K or tuple(c.shape) != (M, N):
        raise ValueError(f"shape mismatch {tuple(a.shape)} x {tuple(b.shape)} -> {tuple(c.shape)}")
    if a.dtype != b.dtype:
        raise TypeError("a and b must have one dtype")
    if stream is None:
        stream = torch.cuda.current_stream(a.device).cuda_stream
    la, lda = _layout(a)
    lb, ldb = _layout(b)
    lc, ldc = _layout(c)
    fused = alpha is not None or beta is not None or bias is not None or activation != ACT_NONE
    if not fused:
        rc = gemm_t(M, N, K, a.data_ptr(), lda, la, b.data_ptr(), ldb, lb, c.data_ptr(), ldc, lc,
                    dtype_code(a), dtype_code(c), stream, config_id)
    else:
        ep = Epilogue(1.0 if alpha is None else float(alpha), 0.0 if beta is None else float(beta), None,
                      BIAS_NONE, F32, int(activation))
        if bias is not None:
            if bias.dim() != 1 or not bias.is_contiguous():
                raise ValueError("bias must be a contiguous 1-D tensor")
            kind = bias_kind if bias_kind is not None else (BIAS_COL if bias.numel() == N else BIAS_ROW)
            if bias.numel() != (M if kind == BIAS_ROW else N):
                raise ValueError("bias length does not match its kind")
            ep.bias, ep.bias_kind, ep.bias_dtype = bias.data_ptr(), kind, dtype_code(bias)
        rc = gemm_fused(M, N, K, a.data_ptr(), lda, la, b.data_ptr(), ldb, lb, c.data_ptr(), ldc, lc,
                        dtype_code(a), dtype_code(c), ep, stream, config_id)
    if check and rc != OK:
        raise TgemmError(rc)
    return rc


def _bhnd(t, name):
    if t.dim() != 4:
        raise ValueError(f"{name} must be a 4-D [batch, heads, n, d] tensor")
    if t.numel() > 0 and t.stride(3) != 1:
        raise ValueError(f"{name}: the last dimension must be contiguous")
    return (t.stride(0), t.stride(1), t.stride(2))


def attention_tensors(q, k, v, o, scale=1.0, causal=False, stream=None, check=True):
    """o := softmax(scale q k^T) v on the device, through the C ABI.  q, o:
    [B, H, n_q, d]; k, v: [B, H, n_k, d] torch tensors on the GPU (any
    strides with a contiguous last dimension).  Returns the return code
    (raises TgemmError on failure if check)."""
    import torch
    B, H, nq, d = q.shape
    if k.shape != v.shape or k.shape[:2] != (B, H) or k.shape[3] != d or tuple(o.shape) != (B, H, nq, d):
        raise ValueError(f"shape mismatch q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}, "
                         f"o {tuple(o.shape)}")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k and v must have one dtype")
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    rc = attention_fwd(B, H, nq, k.shape[2], d, q.data_ptr(), _bhnd(q, "q"), k.data_ptr(), _bhnd(k, "k"),
                       v.data_ptr(), _bhnd(v, "v"), o.data_ptr(), _bhnd(o, "o"), dtype_code(q), dtype_code(o),
                       scale, causal, stream)
    if check and rc != OK:
        raise TgemmError(rc)
    return rc
