"""Seeded synthetic inputs for the five GEMM workloads and the attention forward.

This module draws random matrices and stores them in the input element type;
it holds none of the matrix-product or attention arithmetic.  Both the GPU tests and the
oracle tests take their inputs from here, so the two sides see the same bits.

The workloads are the pages' own kind of input: random dense matrices drawn
with a fixed seed (page "企业官网建设流程全解析", §3.4, times a GEMM on
torch.randn fp16 matrices; page "TileLang实战：用Python DSL自动生成高性能GPU计算
内核", §3.2, checks a float32 128x128x128 product on np.random.randn inputs; the
DeepSeek/Ascend TileLang toolkit page, §3.3, verifies matmul at m=128, n=256,
k=512 and at the non-aligned M=127, N=255, and insists on fixed seeds).
"""
from dataclasses import dataclass

import numpy as np

F32, F16, BF16 = 0, 1, 2
DTYPE_NAMES = {F32: "f32", F16: "f16", BF16: "bf16"}


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    in_dtype: int
    out_dtype: int
    dist: str      # "normal", "uniform" or "normal_scaled" (N(0,1)/sqrt(K))
    seed: int


WORKLOADS = [
    Workload("f32_128x128x128", 128, 128, 128, F32, F32, "normal", 1),
    Workload("f16_128x256x512", 128, 256, 512, F16, F16, "normal", 2),
    Workload("f16_127x255x512_unaligned", 127, 255, 512, F16, F32, "uniform", 3),
    Workload("f16_1024x2048x512", 1024, 2048, 512, F16, F32, "normal_scaled", 4),
    Workload("f16_8192x8192x8192", 8192, 8192, 8192, F16, F16, "normal", 5),
]
BY_NAME = {w.name: w for w in WORKLOADS}


def float32_to_bfloat16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even) and return the
    16-bit patterns as uint16.  NaN stays NaN."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = rounded.astype(np.uint16)
    nan = np.isnan(x)
    out[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return out


def _draw(rng: np.random.Generator, shape, dist: str, K: int) -> np.ndarray:
    if dist == "normal":
        return rng.standard_normal(shape, dtype=np.float32)
    if dist == "uniform":
        return rng.uniform(-1.0, 1.0, shape).astype(np.float32)
    if dist == "normal_scaled":
        return (rng.standard_normal(shape, dtype=np.float32) / np.float32(np.sqrt(K))).astype(np.float32)
    raise ValueError(dist)


def to_storage(x32: np.ndarray, dtype: int) -> np.ndarray:
    """float32 values -> stored element array (float32, float16, or uint16
    bfloat16 bit patterns), rounding to nearest-even."""
    if dtype == F32:
        return np.ascontiguousarray(x32, dtype=np.float32)
    if dtype == F16:
        return np.ascontiguousarray(x32.astype(np.float16))
    if dtype == BF16:
        return float32_to_bfloat16_bits(x32)
    raise ValueError(dtype)


def make_inputs(w: Workload, in_dtype=None):
    """(A, B) stored arrays for workload w: A is M x K, B is K x N, drawn in
    that order from numpy.random.default_rng(w.seed)."""
    dt = w.in_dtype if in_dtype is None else in_dtype
    rng = np.random.default_rng(w.seed)
    a = to_storage(_draw(rng, (w.M, w.K), w.dist, w.K), dt)
    b = to_storage(_draw(rng, (w.K, w.N), w.dist, w.K), dt)
    return a, b


def random_inputs(M, N, K, dtype, seed, dist="normal"):
    """(A, B) of any shape, same recipe as make_inputs."""
    rng = np.random.default_rng(seed)
    return (to_storage(_draw(rng, (M, K), dist, max(K, 1)), dtype),
            to_storage(_draw(rng, (K, N), dist, max(K, 1)), dtype))


def integer_inputs(M, N, K, dtype, seed, lo=-2, hi=2):
    """(A, B) with integer entries in [lo, hi]: every partial sum of the
    product is an integer of magnitude <= max(|lo|,|hi|)^2 * K (<= 32768 for
    the default range at K = 8192), below 2^24, so an fp32 accumulator holds
    every partial sum exactly in any order of summation."""
    rng = np.random.default_rng(seed)
    a = rng.integers(lo, hi + 1, size=(M, K)).astype(np.float32)
    b = rng.integers(lo, hi + 1, size=(K, N)).astype(np.float32)
    return to_storage(a, dtype), to_storage(b, dtype)


def sample_indices(n: int, count: int, seed: int) -> np.ndarray:
    """`count` distinct sorted indices in [0, n) from default_rng(seed), always
    holding 0 and n-1 so that the first and the last tile are covered."""
    if count >= n:
        return np.arange(n, dtype=np.int64)
    rng = np.random.default_rng(seed)
    inner = rng.choice(np.arange(1, n - 1), size=count - 2, replace=False)
    return np.sort(np.concatenate([[0, n - 1], inner]).astype(np.int64))


# ------------------------------------------------------------------ attention
# Q, K, V for the attention forward: N(0, 1) entries rounded to the input
# type, drawn Q then K then V from numpy.random.default_rng(seed), each
# [B, H, n, d] (row-major, packed).
def attention_inputs(B, H, Nq, Nk, d, dtype, seed):
    rng = np.random.default_rng(seed)
    mk = lambda n: to_storage(rng.standard_normal((B, H, n, d), dtype=np.float32), dtype)
    return mk(Nq), mk(Nk), mk(Nk)


class AttnWorkload:
    def __init__(self, name, B, H, N, d, causal, scale, dtype=F16):
        self.name, self.B, self.H, self.N, self.d = name, B, H, N, d
        self.causal, self.scale, self.dtype = causal, scale, dtype

    def flops(self):
        """4 B H N^2 d for the two products (half of it with the causal mask,
        counted over the visible keys only: N (N + 1) / 2 per head)."""
        pairs = self.N * (self.N + 1) // 2 if self.causal else self.N * self.N
        return 4.0 * self.B * self.H * pairs * self.d


# The sequence of page "TileLang实战" §4.3 (1024 positions, model width 768,
# read as 12 heads of 64, no score scale as in its §4.2), and a long-sequence
# case (4096 positions, the length its §4.1 names) with 128-wide heads, plain
# and causal.
ATTN_WORKLOADS = [
    AttnWorkload("attn_b1_h12_n1024_d64", 1, 12, 1024, 64, False, 1.0),
    AttnWorkload("attn_b4_h16_n4096_d128", 4, 16, 4096, 128, False, 128 ** -0.5),
    AttnWorkload("attn_b4_h16_n4096_d128_causal", 4, 16, 4096, 128, True, 128 ** -0.5),
]
