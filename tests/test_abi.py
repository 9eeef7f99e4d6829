"""Host-side checks of libtgemm.so (no GPU needed): it loads, exports every
function include/*.h declares, rejects invalid arguments with the
documented codes before touching the GPU, picks the table's configuration,
and its workgroup -> tile map is a bijection."""
import ctypes
import os
import re

import pytest

import tiled_gemm_03_amd as T
from tiled_gemm_03_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
                 if f.endswith(".h"))


def declared_functions():
    text = "\n".join(open(h, encoding="utf-8").read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_library_exports_every_declared_function():
    lib = T.lib()
    names = declared_functions()
    assert set(names) == set(T.EXPORTED), names
    for n in names:
        assert hasattr(lib, n), f"libtgemm.so does not export {n}"
        assert ctypes.cast(getattr(lib, n), ctypes.c_void_p).value


def test_version_and_configs():
    assert "gfx950" in T.gemm_version()
    n = T.gemm_num_configs()
    assert n >= 4
    for i in range(n):
        c = T.gemm_config_info(i)
        assert c["id"] == i
        assert c["threads"] % 64 == 0
        assert c["threads"] == 64 * c["waves_m"] * c["waves_n"]
        assert c["lds_bytes"] <= 160 * 1024
        if c["stages"] == 0:  # the direct kernel: operands straight to registers
            assert c["lds_bytes"] == 0 and c["block_m"] == c["block_n"] == 32
            continue
        eb = 4 if c["in_dtype"] == T.F32 else 2
        # LDS holds `stages` copies of an A tile (block_m x block_k) and a B
        # tile (block_k x block_n), the budget formula of page
        # "企业官网建设流程全解析", §4.2, with A's own stage count and depth
        # where they differ (the ring kernel's row-major A)
        assert c["lds_bytes"] == (c["a_stages"] * c["a_block_k"] * c["block_m"] +
                                  c["stages"] * c["block_k"] * c["block_n"]) * eb
        if c["a_stages"] == c["stages"]:
            assert c["a_block_k"] == c["block_k"]
            assert c["lds_bytes"] == c["stages"] * (c["block_m"] + c["block_n"]) * c["block_k"] * eb
    with pytest.raises(T.TgemmError):
        T.gemm_config_info(n)


def test_lds_budget_formula_matches_page_example():
    """The page's own numbers: block_M = block_N = 128, block_K = 32, fp16
    gives 8 KB + 8 KB = 16 KB per stage, 48 KB at 3 stages, 64 KB at 4
    ("企业官网建设流程全解析", §4.2); the formula of the DeepSeek/Ascend
    toolkit page, §5.1, at 128/128/64/3 evaluates to 98304 bytes (the page
    prints twice that)."""
    def lds(bm, bn, bk, stages, eb):
        return stages * (bm * bk + bk * bn) * eb
    assert lds(128, 128, 32, 1, 2) == 16 * 1024
    assert lds(128, 128, 32, 3, 2) == 48 * 1024
    assert lds(128, 128, 32, 4, 2) == 64 * 1024
    assert lds(128, 128, 64, 3, 2) == 98304
    # the 256 x 256 configuration: A in 2 stages of 64, B in 4 stages of 32,
    # each ring 64 KiB
    big = T.gemm_config_info(0)
    assert big["lds_bytes"] == (lds(big["block_m"], 0, big["a_block_k"], big["a_stages"], 2) +
                                lds(0, big["block_n"], big["block_k"], big["stages"], 2)) == 128 * 1024


def _codes(M, N, K, A, lda, B, ldb, C, ldc, i, o):
    a = T.gemm(M, N, K, A, lda, B, ldb, C, ldc, i, o, None)
    s = T.gemm_select_config(M, N, K, A, lda, B, ldb, C, ldc, i, o)
    return a, s


FAKE = 1 << 40  # a well-aligned address that is never dereferenced


@pytest.mark.parametrize("args,code", [
    ((-1, 4, 4, FAKE, 4, FAKE, 4, FAKE, 4, 1, 1), T.ERR_DIM),
    ((4, -1, 4, FAKE, 4, FAKE, 4, FAKE, 4, 1, 1), T.ERR_DIM),
    ((4, 4, -1, FAKE, 4, FAKE, 4, FAKE, 4, 1, 1), T.ERR_DIM),
    (((1 << 30) + 1, 4, 4, FAKE, 4, FAKE, 4, FAKE, 4, 1, 1), T.ERR_DIM),
    ((4, 4, 4, FAKE, 4, FAKE, 4, FAKE, 4, 1, 2), T.ERR_DTYPE),
    ((4, 4, 4, FAKE, 4, FAKE, 4, FAKE, 4, 0, 1), T.ERR_DTYPE),
    ((4, 4, 4, FAKE, 4, FAKE, 4, FAKE, 4, 2, 1), T.ERR_DTYPE),
    ((4, 4, 4, FAKE, 4, FAKE, 4, FAKE, 4, 3, 0), T.ERR_DTYPE),
    ((4, 4, 4, FAKE, 3, FAKE, 4, FAKE, 4, 1, 1), T.ERR_LD),
    ((4, 4, 4, FAKE, 4, FAKE, 3, FAKE, 4, 1, 1), T.ERR_LD),
    ((4, 4, 4, FAKE, 4, FAKE, 4, FAKE, 3, 1, 1), T.ERR_LD),
    ((4, 4, 4, None, 4, FAKE, 4, FAKE, 4, 1, 1), T.ERR_NULL),
    ((4, 4, 4, FAKE, 4, None, 4, FAKE, 4, 1, 1), T.ERR_NULL),
    ((4, 4, 4, FAKE, 4, FAKE, 4, None, 4, 1, 1), T.ERR_NULL),
    ((4, 4, 4, FAKE, 4, FAKE + 4096, 4, FAKE + 16, 4, 1, 1), T.ERR_ALIAS),
    ((4, 4, 4, FAKE, 4, FAKE + 4096, 4, FAKE + 4096 + 30, 4, 1, 1), T.ERR_ALIAS),
    # pointers not aligned to their element's size
    ((4, 4, 4, FAKE + 1, 4, FAKE + 4096, 4, FAKE + 8192, 4, 1, 1), T.ERR_ALIGN),
    ((4, 4, 4, FAKE, 4, FAKE + 4097, 4, FAKE + 8192, 4, 2, 2), T.ERR_ALIGN),
    ((4, 4, 4, FAKE, 4, FAKE + 4096, 4, FAKE + 8193, 4, 1, 1), T.ERR_ALIGN),
    ((4, 4, 4, FAKE, 4, FAKE + 4096, 4, FAKE + 8194, 4, 1, 0), T.ERR_ALIGN),
    ((4, 4, 4, FAKE + 2, 4, FAKE + 4096, 4, FAKE + 8192, 4, 0, 0), T.ERR_ALIGN),
])
def test_invalid_arguments_rejected_without_launch(args, code):
    a, s = _codes(*args)
    assert a == code and s == code
    assert T.gemm_strerror(code) != "unknown error code"


def test_empty_problems_are_noops():
    # M == 0 or N == 0: nothing to do, success, even with NULL pointers
    assert T.gemm(0, 4, 4, None, 4, None, 4, None, 4, 1, 1, None) == T.OK
    assert T.gemm(4, 0, 4, None, 4, None, 0, None, 0, 1, 1, None) == T.OK
    # K == 0 needs only C
    assert T.gemm_select_config(4, 4, 0, None, 0, None, 4, FAKE, 4, 1, 1) >= 0


def test_gemm_ex_config_checks():
    n = T.gemm_num_configs()
    assert T.gemm_ex(4, 4, 4, FAKE, 4, FAKE + 4096, 4, FAKE + 8192, 4, 1, 1, None, n) == T.ERR_CONFIG
    assert T.gemm_ex(4, 4, 4, FAKE, 4, FAKE + 4096, 4, FAKE + 8192, 4, 1, 1, None, -2) == T.ERR_CONFIG
    for i in range(n):
        fam = T.gemm_config_info(i)["in_dtype"]
        other = T.F32 if fam != T.F32 else T.F16
        rc = T.gemm_ex(4, 4, 4, FAKE, 4, FAKE + 4096, 4, FAKE + 8192, 4, other, T.F32, None, i)
        assert rc == T.ERR_CONFIG


def test_table_choice_for_the_workloads():
    names = {i: T.gemm_config_info(i)["name"] for i in range(T.gemm_num_configs())}
    picks = {}
    for w in W.WORKLOADS:
        cid = T.gemm_select_config(w.M, w.N, w.K, FAKE, w.K, FAKE + (1 << 32), w.N, FAKE + (2 << 32), w.N,
                                   w.in_dtype, w.out_dtype)
        assert cid >= 0
        info = T.gemm_config_info(cid)
        assert info["in_dtype"] == (T.F32 if w.in_dtype == T.F32 else T.F16)
        picks[w.name] = names[cid]
    # the large square product takes the largest tile
    assert picks["f16_8192x8192x8192"] == names[0]


@pytest.mark.parametrize("tiles_m,tiles_n,group_m", [
    (1, 1, 1), (1, 7, 4), (7, 1, 4), (32, 32, 4), (32, 32, 1), (32, 32, 8), (5, 13, 3),
    (8, 16, 4), (33, 31, 4), (4, 8, 16), (16, 32, 6)])
def test_tile_map_is_a_bijection(tiles_m, tiles_n, group_m):
    seen = set()
    for bid in range(tiles_m * tiles_n):
        tm, tn = T.gemm_tile_map(bid, tiles_m, tiles_n, group_m)
        assert 0 <= tm < tiles_m and 0 <= tn < tiles_n
        seen.add((tm, tn))
    assert len(seen) == tiles_m * tiles_n


def test_tile_map_keeps_an_xcd_on_a_compact_block():
    """The 32 workgroups that one XCD runs first at 8192^3 with 256x256 tiles
    (ids x, x+8, ..., x+248) cover a 4 x 8 block of tiles: 4 A panels and 8
    B panels shared in that XCD's L2."""
    for xcd in range(8):
        tiles = [T.gemm_tile_map(xcd + 8 * j, 32, 32, 4) for j in range(32)]
        ms = {t[0] for t in tiles}
        ns = {t[1] for t in tiles}
        assert len(ms) == 4 and len(ns) == 8


def _kernel(M, N, K, lda=None, ldb=None, ldc=None, in_dt=T.F16, out_dt=T.F16, cid=-1, offs=(0, 0, 0)):
    lda = K if lda is None else lda
    ldb = N if ldb is None else ldb
    ldc = N if ldc is None else ldc
    eb = 4 if in_dt == T.F32 else 2
    return T.gemm_select_kernel(M, N, K, FAKE + offs[0] * eb, lda, FAKE + (1 << 36) + offs[1] * eb, ldb,
                                FAKE + (2 << 36) + offs[2] * 2, ldc, in_dt, out_dt, cid)


def test_kernel_choice_ring_path():
    """The direct-to-LDS ring kernel runs exactly for 16-bit inputs with K a
    multiple of 128 or above 128 (the K-tail variant) and operands whose
    every element its range-checked loads keep, whatever M, N and the
    alignment of C (edge tiles store masked;
    partial column groups and unaligned C rows through the fused epilogue's
    stores); anything else falls back to a register-staged kernel of the same
    tile."""
    R, TI, GE = T.KERNEL_RING, T.KERNEL_TILED, T.KERNEL_GENERAL
    assert _kernel(8192, 8192, 8192) == R
    assert _kernel(8192, 8192, 8192, in_dt=T.BF16, out_dt=T.F32) == R
    assert _kernel(1024, 2048, 512, out_dt=T.F32, cid=0) == R
    assert _kernel(1024, 2048, 512, out_dt=T.F32, cid=1) == R
    assert _kernel(256, 256, 128, cid=0) == R
    assert _kernel(8192, 8192, 8192 + 64) == R           # K not a multiple of 128: the K tail
    assert _kernel(8192, 8192, 8192 - 32) == R
    assert _kernel(256, 256, 129, lda=136, cid=0) == R   # K just above 128
    assert _kernel(256, 256, 120, cid=0) == R            # K below 128: the tail alone
    assert _kernel(4096, 4096, 16) == R and _kernel(4096, 4096, 100) == R
    assert _kernel(256, 256, 64, cid=1) == R
    assert _kernel(8192 - 256, 8192, 8192) == R          # still whole tiles
    assert _kernel(8191, 8192, 8192) == R                # ragged M: masked edge tiles
    assert _kernel(8191, 8000, 8192) == R                # ragged M and N
    assert _kernel(8192, 8190, 8192) == R                # B rows not whole 16-byte chunks
    assert _kernel(8192, 8192, 8192, ldc=8194) == R      # C rows not 4-element aligned
    assert _kernel(8192, 8192, 8192, offs=(0, 0, 1)) == R  # C base not 4-element aligned
    assert _kernel(8192, 8190, 8192, ldb=8192, ldc=8192) == R   # N % 4 != 0: partial column groups
    assert _kernel(8192, 8192, 8192, lda=8196) == R      # rows not whole 16-byte chunks
    assert _kernel(8192, 8192, 8192, lda=8192 + 8) == R  # padded, still aligned
    assert _kernel(8192, 8192, 8192, offs=(1, 0, 0)) == R
    assert _kernel(8192, 8192, 8192, cid=2) == TI        # configuration without a ring kernel
    assert _kernel(1024, 1024, 1024, in_dt=T.F32, out_dt=T.F32) != R
    # B offsets beyond 2^31 bytes: register-staged kernel
    assert _kernel(256, 256, 1 << 15, ldb=1 << 15, cid=0) == TI
    assert _kernel(-1, 4, 4) == T.ERR_DIM
    assert _kernel(4, 4, 4, in_dt=T.F16, out_dt=T.BF16) == T.ERR_DTYPE
    assert _kernel(4, 4, 4, cid=4) == T.ERR_CONFIG
    # the direct kernel takes any alignment and raggedness
    assert _kernel(127, 255, 512, ldb=255, ldc=255, cid=6) == T.KERNEL_DIRECT
    assert _kernel(128, 128, 128, in_dt=T.F32, out_dt=T.F32, cid=7) == T.KERNEL_DIRECT
    assert _kernel(5, 7, 3, offs=(1, 1, 1), cid=6) == T.KERNEL_DIRECT
    # offsets beyond 2^31 bytes: the checked register-staged kernel instead
    assert _kernel(64, 64, 1 << 20, ldb=1 << 12, cid=6) in (T.KERNEL_GENERAL, T.KERNEL_TILED)


def test_table_prefers_256_tiles_beyond_two_rounds_of_128_tiles():
    """256 x 256 tiles when they fill the 256 CUs or when 128 x 128 tiles
    would need three or more rounds; else 128 x 128 (or 64 x 128, also for
    small products that the direct kernel does not take)."""
    RING = T.KERNEL_RING
    assert _kernel_t(3072, 3072, 3072, R_, R_, R_) == (RING, 0)      # 144 big tiles, 576 mid ones
    assert _kernel_t(3000, 3000, 3000, R_, R_, R_) == (RING, 0)
    assert _kernel_t(2048, 2048, 2048, R_, R_, R_) == (RING, 1)      # 64 big, 256 mid
    assert _kernel_t(8192, 1024, 8192, R_, R_, R_) == (RING, 1)      # 128 big, 512 mid
    assert _kernel_t(1024, 8192, 1024, R_, R_, R_) == (RING, 1)
    assert _kernel_t(3072, 3072, 3072, C_, R_, R_) == (RING, 0)      # other layouts alike
    assert _kernel_t(4096, 4096, 1024, R_, R_, R_) == (RING, 0)
    # small products: the 64 x 128 ring from 4 of its tiles, or one tile
    # with K >= 1024, where the direct kernel does not take them
    for n in (512, 768):
        assert _kernel_t(n, n, n, R_, R_, R_) == (RING, 8), n
    assert _kernel_t(512, 512, 2048, R_, R_, R_) == (RING, 8)
    assert _kernel_t(64, 64, 1024, R_, R_, R_) == (RING, 8)


def test_table_sends_small_products_with_medium_k_to_the_direct_kernel():
    """128 <= K <= 512 (16-bit) or K >= 128 (fp32) with all of K's loads in
    flight at once and at most 576 (fp32: 256) workgroups: the direct kernel;
    K = 64, or more workgroups, or a longer K: the tiles or rings."""
    D, RING, TI = T.KERNEL_DIRECT, T.KERNEL_RING, T.KERNEL_TILED
    for n in (128, 256, 384):            # 384^3: K over the waves, 24 x 24 workgroups of 16 x 16
        assert _kernel_t(n, n, n, R_, R_, R_) == (D, 6), n
    assert _kernel_t(128, 128, 256, R_, R_, R_) == (D, 6)
    assert _kernel_t(128, 128, 64, R_, R_, R_) == (TI, 3)           # K = 64: 32 x 32 tiles
    assert _kernel_t(512, 512, 256, R_, R_, R_) == (RING, 8)       # 1024 workgroups of 16 x 16
    f32 = dict(in_dt=T.F32, out_dt=T.F32)
    assert _kernel_t(128, 128, 256, R_, R_, R_, **f32) == (D, 7)
    assert _kernel_t(256, 256, 256, R_, R_, R_, **f32) == (D, 7)     # 256 workgroups of 16 x 16
    assert _kernel_t(512, 512, 128, R_, R_, R_, **f32) == (TI, 5)    # 1024 of them
    assert _kernel_t(128, 128, 512, R_, R_, R_, **f32) == (TI, 5)    # a quarter of K exceeds the ring
    assert _kernel_t(128, 128, 64, R_, R_, R_, **f32) == (TI, 5)


def _splits(M, N, K, la=T.ROW_MAJOR, lb=T.ROW_MAJOR, lc=T.ROW_MAJOR, lda=None, ldb=None, ldc=None, in_dt=T.F16,
            out_dt=T.F16):
    row = T.ROW_MAJOR
    lda = (K if la == row else M) if lda is None else lda
    ldb = (N if lb == row else K) if ldb is None else ldb
    ldc = (N if lc == row else M) if ldc is None else ldc
    return T.gemm_split_count_t(M, N, K, FAKE, lda, la, FAKE + (1 << 36), ldb, lb, FAKE + (2 << 36), ldc, lc, in_dt,
                                out_dt)


def test_split_k_choice():
    """Products whose ring tiles leave most CUs idle (128 or fewer) and
    whose K is long (4096 or more) run in slices of K: about as many
    workgroups as the CUs hold at once (512 for these tiles), slices of at
    least 256 of K that are whole ring steps (the last one may carry the K
    tail), at most 32.  Never for a forced configuration, N % 4 != 0,
    unaligned operand rows, fp32 inputs or short K."""
    SPLIT, RING = T.KERNEL_RING_SPLITK, T.KERNEL_RING
    R_, C_ = T.ROW_MAJOR, T.COL_MAJOR
    assert _kernel_t(512, 512, 16384, R_, R_, R_) == (SPLIT, 8)        # 32 tiles of 64 x 128
    assert _splits(512, 512, 16384) == 16
    assert _splits(256, 256, 65536) == 32
    assert _splits(1024, 1024, 8192) == 4                              # 128 tiles: 512 workgroups
    assert _splits(32, 4096, 4096) == 16
    assert _splits(1024, 512, 2048) == 1                               # K below 4096
    assert _kernel_t(32, 4096, 4096, R_, R_, R_) == (SPLIT, 8)
    assert _splits(512, 512, 16384 + 100, lda=16384 + 128) > 1         # the last slice carries the tail
    assert _kernel_t(512, 512, 16384, R_, R_, R_, cid=8) == (RING, 8)  # forced: no slices
    assert _splits(512, 512, 1024) == 1                                # short K
    assert _splits(512, 510, 16384) == 1                               # N % 4 != 0
    assert _splits(512, 512, 16384, lda=16384 + 4) == 1                # rows not whole 16-byte chunks
    assert _splits(512, 512, 16384, in_dt=T.F32, out_dt=T.F32) == 1
    assert _splits(4096, 4096, 4096) == 1                              # enough tiles
    assert _kernel_t(512, 512, 16384, C_, R_, R_) == (SPLIT, 1)       # column-major A: 128 x 128 tiles
    for fmt in (T.F32, T.BF16):
        assert _kernel_t(512, 512, 16384, R_, R_, R_, in_dt=T.BF16, out_dt=fmt) == (SPLIT, 8)
    assert _kernel_t(512, 512, 16384, R_, R_, R_, out_dt=T.FP8_E4M3) == (SPLIT, 8)
    # the workspace stays within 256 MiB: fewer slices
    assert _splits(8192, 8192 // 128, 1 << 20, ldb=64) >= 1


def test_ring_configs_report_their_ring_kernel():
    for cid in (0, 1, 8):
        c = T.gemm_config_info(cid)
        assert (c["block_k"], c["stages"]) == (32, 4)
        assert (c["a_block_k"], c["a_stages"]) == (64, 2)
        assert (c["mfma_m"], c["mfma_n"], c["mfma_k"]) == (16, 16, 32)
    assert (T.gemm_config_info(8)["block_m"], T.gemm_config_info(8)["block_n"]) == (64, 128)


def test_fp8_outputs_are_checked_and_routed():
    """8-bit outputs: from 16-bit inputs only; written by the ring kernels
    where they apply, by the direct kernel elsewhere (never a register-staged
    kernel)."""
    RING, DIRECT = T.KERNEL_RING, T.KERNEL_DIRECT
    for fmt in (T.FP8_E4M3, T.FP8_E5M2):
        for in_dt in (T.F16, T.BF16):
            assert _kernel(8192, 8192, 8192, in_dt=in_dt, out_dt=fmt) == RING
            assert _kernel_t(1024, 2048, 512, R_, R_, R_, in_dt=in_dt, out_dt=fmt) == (RING, 8)
            assert _kernel_t(1000, 1000, 1000, C_, C_, C_, in_dt=in_dt, out_dt=fmt)[0] == RING
            assert _kernel(127, 255, 512, ldb=255, ldc=255, in_dt=in_dt, out_dt=fmt) == DIRECT
            # an operand at an odd address: rejected; an 8-bit C at any byte
            Bp, Cp = FAKE + (1 << 36), FAKE + (2 << 36)
            assert T.gemm_select_kernel(1024, 1024, 301, FAKE + 1, 301, Bp, 1027, Cp, 1024, in_dt, fmt) == \
                T.ERR_ALIGN
            assert T.gemm_select_kernel(1024, 1024, 301, FAKE, 301, Bp, 1027, Cp + 1, 1024, in_dt, fmt) == RING
            assert _kernel(256, 256, 64, cid=2, in_dt=in_dt, out_dt=fmt) == DIRECT
        assert _kernel(64, 64, 64, in_dt=T.F32, out_dt=fmt) == T.ERR_DTYPE
        assert _kernel(64, 64, 64, in_dt=fmt, out_dt=fmt) == T.ERR_DTYPE
        assert _kernel(64, 64, 64, in_dt=fmt, out_dt=T.F16) == T.ERR_DTYPE
        # C holds one byte per element: its span for the overlap check
        assert T.gemm(4, 4, 4, FAKE, 4, FAKE + 4096, 4, FAKE + 8, 4, T.F16, fmt, None) == T.ERR_ALIAS
    # offsets beyond 31 bits for the direct kernel: no kernel for an 8-bit output
    assert _kernel(64, 64, 1 << 20, ldb=1 << 12, out_dt=T.FP8_E4M3) == T.ERR_DIM
    assert _kernel(64, 64, 64, out_dt=5) == T.ERR_DTYPE


def test_ring_only_configuration_falls_back_to_128x128():
    """Configuration 8 (64 x 128 ring, row-major A) has no register-staged
    kernel: calls its ring does not take run configuration 1 instead, and the
    configuration reported is the one that runs."""
    RING = T.KERNEL_RING
    assert _kernel_t(1024, 2048, 512, R_, R_, R_, cid=8) == (RING, 8)
    assert _kernel_t(1024, 2048, 512, R_, C_, R_, cid=8) == (RING, 8)      # column-major B: k-contiguous
    assert _kernel_t(1024, 2048, 512, C_, R_, R_, cid=8) == (RING, 1)      # column-major A
    assert _kernel_t(1024, 2048, 512, R_, R_, R_, lda=516, cid=8) == (RING, 8)  # A rows not whole chunks
    # A's last element ending at a page boundary (odd K at 2 mod 4, no pad:
    # loaded on its own in the K tail)
    A = FAKE + (-(2 * 1024 * 513)) % 4096
    assert T.gemm_select_kernel_t(1024, 2048, 513, A, 513, R_, FAKE + (1 << 36), 2048, R_, FAKE + (2 << 36), 2048,
                                  R_, T.F16, T.F16, 8) == (RING, 8)
    assert _kernel_t(1024, 2048, 64, R_, R_, R_, cid=8) == (RING, 8)       # K below the ring's step: the tail
    # a product the ring does not take (buffer offsets beyond 31 bits):
    # the register-staged kernel of configuration 1
    assert T.gemm_select_kernel_t(1024, 2048, 64, FAKE, 1 << 24, R_, FAKE + (1 << 38), 2048, R_, FAKE + (2 << 38),
                                  2048, R_, T.F16, T.F16, 8) == (T.KERNEL_GENERAL, 1)
    assert _kernel_t(1000, 2000, 1000, R_, R_, R_, cid=8) == (RING, 8)     # ragged, K tail
    assert _kernel_t(4, 4, 4, R_, R_, R_, in_dt=T.F32, out_dt=T.F32, cid=8)[0] == T.ERR_CONFIG


R_, C_ = T.ROW_MAJOR, T.COL_MAJOR


def _kernel_t(M, N, K, la, lb, lc, lda=None, ldb=None, ldc=None, in_dt=T.F16, out_dt=T.F16, cid=-1):
    lda = (K if la == R_ else M) if lda is None else lda
    ldb = (N if lb == R_ else K) if ldb is None else ldb
    ldc = (N if lc == R_ else M) if ldc is None else ldc
    return T.gemm_select_kernel_t(M, N, K, FAKE, lda, la, FAKE + (1 << 36), ldb, lb, FAKE + (2 << 36), ldc, lc,
                                  in_dt, out_dt, cid)


def _last_fix(base, ld, kcontig, outer, K):
    """The range-check rule the ring's loads are held to, restated: the
    operand's last element is lost only if it starts a 4-byte part of its
    16-byte load (an odd number of elements from the row's first loaded one:
    K along a k-contiguous row, M or N along a k-strided one) at an address of
    2 mod 4; the range then takes the 2 bytes after it, unless they start a
    new 4 KiB page: then the kernel loads that element on its own in its K
    tail.  True for that last case."""
    rows, cols = (outer, K) if kcontig else (K, outer)
    last = base + 2 * ((rows - 1) * ld + cols - 1)
    return cols % 2 == 1 and last % 4 == 2 and (last + 2) % 4096 == 0


def test_ring_takes_unaligned_rows_where_every_element_is_kept():
    """Operands off 16-byte alignment or with rows not whole 16-byte chunks
    run the ring kernel whenever their elements are at even addresses (a
    2-byte range pad inside the last element's page, or that element loaded
    on its own in the K tail where the pad would reach the next page); odd
    byte addresses never do.  Every layout pair, odd and even sizes, element
    offsets 0..7 and leading dimensions with every residue mod 8, and
    placements that put the end of the last element at a page boundary."""
    RING = T.KERNEL_RING
    A0, B0, C0 = FAKE, FAKE + (1 << 36), FAKE + (2 << 36)
    n_ring = n_other = 0
    for la in (R_, C_):
        for lb in (R_, C_):
            for M, N, K in ((1024, 1024, 1024), (1023, 1021, 1025), (1024, 1023, 1023), (1021, 1024, 1026)):
                for oa, ob, pa, pb in ((0, 0, 0, 0), (1, 0, 0, 0), (0, 1, 0, 0), (3, 5, 1, 2), (2, 7, 3, 5),
                                       (1, 1, 1, 1), (0, 0, 7, 6), (6, 2, 4, 0)):
                    lda = (K if la == R_ else M) + pa
                    ldb = (N if lb == R_ else K) + pb
                    A, B = A0 + 2 * oa, B0 + 2 * ob
                    got = T.gemm_select_kernel_t(M, N, K, A, lda, la, B, ldb, lb, C0, N, R_, T.F16, T.F16, 1)
                    assert got[0] == RING, (la, lb, M, N, K, oa, ob, pa, pb, got)
                    n_ring += 1
                    n_other += _last_fix(A, lda, la == R_, M, K) or _last_fix(B, ldb, lb == C_, N, K)
                    # an odd byte address: rejected
                    got = T.gemm_select_kernel_t(M, N, K, A + 1, lda, la, B, ldb, lb, C0, N, R_, T.F16, T.F16, 1)
                    assert got[0] == T.ERR_ALIGN
    assert n_ring > 0
    # the last element of A ending at a page boundary (no pad possible: the
    # element loaded on its own), a pad, no pad
    M, N, K = 1024, 1024, 301
    end = 2 * M * K  # bytes from A to the end of its last element (lda = K)
    A = A0 + (-end) % 4096
    assert (A + end) % 4096 == 0 and A % 2 == 0 and _last_fix(A, K, True, M, K)
    for a in (A, A + 2, A + 4):
        assert T.gemm_select_kernel(M, N, K, a, K, B0, N, C0, N, T.F16, T.F16, -1) == RING
    # an M that is a multiple of 2048 with an odd K and contiguous rows always
    # ends A at a page boundary (from a page-aligned base)
    assert _last_fix(A0, 8191, True, 8192, 8191)
    assert _kernel(8192, 8192, 8191) == RING
    # the square odd sizes: every element kept with contiguous rows, with or
    # without a base offset
    for n in (8191, 4095, 2047):
        assert _kernel(n, n, n) == RING
        assert _kernel(n, n, n, offs=(1, 0, 0)) == RING


def test_layout_arguments_are_checked():
    # layouts other than 0 / 1
    assert T.gemm_t(4, 4, 4, FAKE, 4, 2, FAKE + 4096, 4, 0, FAKE + 8192, 4, 0, 1, 1, None, -1) == T.ERR_LAYOUT
    assert T.gemm_t(4, 4, 4, FAKE, 4, 0, FAKE + 4096, 4, -1, FAKE + 8192, 4, 0, 1, 1, None, -1) == T.ERR_LAYOUT
    assert T.gemm_t(4, 4, 4, FAKE, 4, 0, FAKE + 4096, 4, 0, FAKE + 8192, 4, 7, 1, 1, None, -1) == T.ERR_LAYOUT
    # leading dimensions follow the stored shape: a column-major A (K x M
    # stored) needs lda >= M, a column-major B ldb >= K, a column-major C
    # ldc >= M
    assert T.gemm_t(8, 4, 2, FAKE, 7, C_, FAKE + 4096, 4, R_, FAKE + 8192, 4, R_, 1, 1, None, -1) == T.ERR_LD
    assert T.gemm_t(8, 4, 2, FAKE, 8, C_, FAKE + 4096, 4, R_, FAKE + 8192, 4, R_, 1, 1, None, -1) != T.ERR_LD
    assert T.gemm_t(8, 4, 6, FAKE, 6, R_, FAKE + 4096, 5, C_, FAKE + 8192, 4, R_, 1, 1, None, -1) == T.ERR_LD
    assert T.gemm_t(8, 4, 6, FAKE, 6, R_, FAKE + 4096, 4, R_, FAKE + 8192, 7, C_, 1, 1, None, -1) == T.ERR_LD
    # gemm is gemm_t with every operand row-major
    assert T.gemm(-1, 4, 4, FAKE, 4, FAKE, 4, FAKE, 4, 1, 1, None) == T.ERR_DIM


def test_kernel_choice_for_layouts():
    RING, DIRECT = T.KERNEL_RING, T.KERNEL_DIRECT
    for la in (R_, C_):
        for lb in (R_, C_):
            for lc in (R_, C_):
                k, cfg = _kernel_t(8192, 8192, 8192, la, lb, lc)
                assert (k, cfg) == (RING, 0), (la, lb, lc)
                k, cfg = _kernel_t(1024, 2048, 512, la, lb, lc, out_dt=T.F32)
                # 128 tiles of 128 x 128: the 64 x 128 ring when both operands
                # of the row-major product it runs are row-major (a column-major
                # C swaps A and B and flips their layouts), else 128 x 128
                row_row = (la, lb) == (R_, R_) if lc == R_ else (la, lb) == (C_, C_)
                assert (k, cfg) == (RING, 8 if row_row else 1), (la, lb, lc)
                k, cfg = _kernel_t(127, 255, 512, la, lb, lc, out_dt=T.F32)
                if (la, lb, lc) == (R_, R_, R_):
                    assert k == DIRECT or k >= 0
                else:
                    assert (k, cfg) == (DIRECT, 6), (la, lb, lc)
                k, cfg = _kernel_t(100, 60, 30, la, lb, lc, in_dt=T.F32, out_dt=T.F32)
                if (la, lb, lc) != (R_, R_, R_):
                    assert (k, cfg) == (DIRECT, 7)
    # a column-major operand and a configuration that has only a
    # register-staged kernel
    assert _kernel_t(256, 256, 256, C_, R_, R_, cid=2)[0] == T.ERR_CONFIG
    assert _kernel_t(256, 256, 256, R_, R_, R_, cid=2)[0] == T.KERNEL_TILED
    # forced ring configuration on a ragged shape: the ring (column-major A
    # rows of 250 elements, or of 249 with its range padded or its last
    # element loaded on its own), the direct kernel for an odd address
    assert _kernel_t(250, 256, 256, C_, C_, R_, cid=0) == (RING, 0)
    assert _kernel_t(249, 256, 256, C_, C_, R_, cid=0) == (RING, 0)  # padded range
    A = FAKE + (-(2 * 256 * 249)) % 4096  # A's last element ending at a page boundary
    assert T.gemm_select_kernel_t(249, 256, 256, A, 249, C_, FAKE + (1 << 36), 256, C_, FAKE + (2 << 36), 256, R_,
                                  T.F16, T.F16, 0) == (RING, 0)
    # an odd address: rejected
    assert T.gemm_select_kernel_t(249, 256, 256, FAKE + 1, 249, C_, FAKE + (1 << 36), 256, C_, FAKE + (2 << 36), 256,
                                  R_, T.F16, T.F16, 0)[0] == T.ERR_ALIGN
    # a column-major C swaps the roles of A and B: its 128 rows become the
    # N of the row-major product (128 x 128 tiles)
    # (64 of them, K = 8192: in slices of K)
    assert _kernel_t(128, 8192, 8192, R_, R_, C_) == (T.KERNEL_RING_SPLITK, 1)
    assert _kernel_t(128, 8192, 1024, R_, R_, C_) == (RING, 1)


def test_fused_epilogue_arguments_are_checked():
    """gemm_fused rejects bad epilogue arguments before touching the GPU."""
    FAKE = 1 << 40
    def call(ep, M=64, N=64, K=64, C=None):
        C = FAKE + (2 << 36) if C is None else C
        return T.gemm_fused(M, N, K, FAKE, K, T.ROW_MAJOR, FAKE + (1 << 36), N, T.ROW_MAJOR, C, N, T.ROW_MAJOR,
                            T.F16, T.F16, ep, None, -1)
    assert call(T.Epilogue(1.0, 0.0, None, T.BIAS_NONE, T.F32, 9)) == T.ERR_EPILOGUE
    assert call(T.Epilogue(1.0, 0.0, None, T.BIAS_NONE, T.F32, -1)) == T.ERR_EPILOGUE
    assert call(T.Epilogue(1.0, 0.0, FAKE + (3 << 36), 3, T.F32, T.ACT_NONE)) == T.ERR_EPILOGUE
    assert call(T.Epilogue(1.0, 0.0, None, T.BIAS_COL, T.F32, T.ACT_NONE)) == T.ERR_EPILOGUE
    assert call(T.Epilogue(1.0, 0.0, FAKE + (3 << 36), T.BIAS_COL, 7, T.ACT_NONE)) == T.ERR_EPILOGUE
    # checked before the sizes: wrong whatever the sizes
    assert call(T.Epilogue(1.0, 0.0, None, T.BIAS_NONE, T.F32, 9), M=0) == T.ERR_EPILOGUE
    # a bias overlapping C
    C = FAKE + (2 << 36)
    assert call(T.Epilogue(1.0, 0.0, C + 16, T.BIAS_COL, T.F16, T.ACT_NONE), C=C) == T.ERR_ALIAS
    assert call(T.Epilogue(1.0, 0.0, C - 64, T.BIAS_ROW, T.F32, T.ACT_NONE), C=C) == T.ERR_ALIAS
    # the usual checks still apply
    assert call(T.Epilogue(1.0, 0.0, None, T.BIAS_NONE, T.F32, T.ACT_RELU), M=-1) == T.ERR_DIM
    assert T.gemm_strerror(T.ERR_EPILOGUE).startswith("epilogue")


def test_fused_epilogue_struct_layout():
    """The ctypes mirror of tgemm_epilogue: two floats, a pointer, three ints."""
    assert ctypes.sizeof(T.Epilogue) == 32
    assert T.Epilogue.bias.offset == 8 and T.Epilogue.activation.offset == 24


def _read_tuned_table(path):
    rows = []
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("//"):
            continue
        m = re.fullmatch(r"\{([-0-9, ]+)\},", line)
        assert m, f"unexpected line in the tuned table: {line!r}"
        rows.append(tuple(int(x) for x in m.group(1).split(",")))
    return rows


def test_tuned_table_entries_are_valid():
    """Every entry of the committed table names a configuration of its input
    type's family and a supported type pair."""
    from tiled_gemm_03_amd import tune
    for M, N, K, lda, ldb, ldc, i, o, cfg in _read_tuned_table(tune.TABLE):
        assert min(M, N, K) >= 0 and lda >= K and ldb >= N and ldc >= N
        assert (i, o) in ((T.F32, T.F32), (T.F16, T.F16), (T.F16, T.F32), (T.BF16, T.BF16), (T.BF16, T.F32))
        fam = T.F32 if i == T.F32 else T.F16
        assert T.gemm_config_info(cfg)["in_dtype"] == fam
        # the library picks that configuration for exactly that call
        FAKE = 1 << 40
        assert T.gemm_select_config(M, N, K, FAKE, lda, FAKE + (1 << 36), ldb, FAKE + (2 << 36), ldc, i, o) == cfg


def test_tuner_emits_a_table_the_parser_reads(tmp_path):
    from tiled_gemm_03_amd import tune
    entries = [(8192, 8192, 8192, T.F16, T.F16, 8192, 8192, 8192, 0), (127, 255, 512, T.F16, T.F32, 512, 255, 255, 6)]
    path = str(tmp_path / "t.inc")
    tune.emit(entries, path=path, note="test")
    assert _read_tuned_table(path) == [(8192, 8192, 8192, 8192, 8192, 8192, 1, 1, 0), (127, 255, 512, 512, 255, 255, 1, 0, 6)]
    assert tune.parse_spec("1,2,3,1,0") == (1, 2, 3, 1, 0, 3, 2, 2)
    assert tune.parse_spec("1,2,3,1,0,8,9,10") == (1, 2, 3, 1, 0, 8, 9, 10)
