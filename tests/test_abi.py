"""The C-ABI library without a GPU: it loads, exports every declared symbol,
and rejects bad arguments on the host before any HIP call."""

import ctypes
import os
import re

import pytest

import fp32_gemm_row_amd as fgr
from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "fp32_gemm_row.h")


def declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?(?:\w+[\s*]+)+(\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def declared_macros():
    text = open(HEADER, encoding="utf-8").read()
    return {m.group(1): int(m.group(2)) for m in re.finditer(r"#define\s+FGR_(\w+)\s+\(?(-?\d+)\)?", text)}


@pytest.fixture(scope="module")
def lib():
    return fgr.load_library()


def test_library_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(fgr.EXPORTS), names
    for name in names:
        assert hasattr(lib, name), f"{name} not exported"


def test_python_constants_match_header():
    macros = declared_macros()
    for key, value in macros.items():
        if key.startswith("ERR_") or key == "OK":
            assert getattr(fgr, key) == value, key
        elif key.startswith("PATH_") or key.startswith("TILE_"):
            assert getattr(fgr, key) == value, key


def test_controlled_comparison_variants(lib):
    # host-only: the variant list along buffering x tile x chunk, names
    # unique, out-of-range indices rejected before any HIP call
    names = fgr.variant_names()
    assert len(names) == 15 and len(set(names)) == 15
    for buf in ("single", "double"):
        for tile in ("256x256", "256x128", "128x128"):
            for bk in ("bk16", "bk32"):
                assert f"regs {buf} {tile} {bk}" in names
    for ring in (3, 4, 5):
        assert f"direct ring{ring} 256x256 bk16" in names
    assert lib.fgr_variant_name(-1) is None and lib.fgr_variant_name(len(names)) is None
    assert lib.fgr_solve_variant(A0, B0, C0, 64, 64, 64, None, len(names)) == fgr.ERR_BAD_PATH
    assert lib.fgr_solve_variant(A0, B0, C0, 64, 64, 64, None, -1) == fgr.ERR_BAD_PATH
    assert lib.fgr_solve_variant(A0, B0, C0, 64, 63, 64, None, 0) == fgr.ERR_BAD_PATH  # N % 4
    assert lib.fgr_solve_variant(A0 + 4, B0, C0, 64, 64, 64, None, 0) == fgr.ERR_BAD_PATH  # 4-byte aligned A
    assert lib.fgr_solve_variant(A0, B0, C0, 64, 60, 64, None, 12) == fgr.ERR_BAD_PATH  # direct copies, N < 64
    assert lib.fgr_solve_variant(A0, B0, C0, 0, 64, 64, None, 0) == fgr.ERR_BAD_DIMS


def test_version_and_status_strings(lib):
    assert fgr.version() == 200
    assert fgr.status_string(fgr.OK) == "ok"
    for code in range(-8, 0):
        s = fgr.status_string(code)
        assert s and s != "unknown status"
    assert fgr.status_string(12345) == "unknown status"


# Fake, well-separated, 256-byte aligned "device" addresses: validation runs on
# the host before any HIP call, so they are never dereferenced.
A0, B0, C0 = 0x10000000, 0x20000000, 0x30000000


def call(lib, a, b, c, M, N, K, path=0, tile=0):
    return lib.fgr_solve_path(a, b, c, M, N, K, None, path, tile)


def test_null_pointers_rejected(lib):
    assert call(lib, 0, B0, C0, 2, 2, 2) == fgr.ERR_NULL_POINTER
    assert call(lib, A0, 0, C0, 2, 2, 2) == fgr.ERR_NULL_POINTER
    assert call(lib, A0, B0, 0, 2, 2, 2) == fgr.ERR_NULL_POINTER
    assert lib.solve(A0, B0, 0, 2, 2, 2, None) == fgr.ERR_NULL_POINTER
    assert lib.fgr_solve_default(0, B0, C0, 2, 2, 2) == fgr.ERR_NULL_POINTER


@pytest.mark.parametrize("dims", [(0, 1, 1), (1, 0, 1), (1, 1, 0), (-1, 4, 4), (4, 4, -8)])
def test_bad_dims_rejected(lib, dims):
    assert call(lib, A0, B0, C0, *dims) == fgr.ERR_BAD_DIMS
    assert lib.solve(A0, B0, C0, *dims, None) == fgr.ERR_BAD_DIMS


def test_misaligned_pointers_rejected(lib):
    assert call(lib, A0 + 2, B0, C0, 4, 4, 4) == fgr.ERR_MISALIGNED
    assert call(lib, A0, B0 + 1, C0, 4, 4, 4) == fgr.ERR_MISALIGNED
    assert call(lib, A0, B0, C0 + 3, 4, 4, 4) == fgr.ERR_MISALIGNED


def test_overlap_of_output_rejected(lib):
    M, N, K = 16, 16, 16
    # C starts inside A
    assert call(lib, A0, B0, A0 + 4 * (M * N - 1), M, N, K) == fgr.ERR_ALIAS
    # C ends inside B
    assert call(lib, A0, B0, B0 - 4 * (M * K - 1), M, N, K) == fgr.ERR_ALIAS
    # A and B may alias each other
    assert fgr.select_path(A0, A0, C0, M, N, K) == fgr.PATH_MFMA_SPLIT
    # adjacent, not overlapping
    assert fgr.select_path(A0, B0, A0 + 4 * M * N, M, N, K) == fgr.PATH_MFMA_SPLIT


def test_forced_path_rejections(lib):
    # vec path needs N % 4 == 0, K % 4 == 0 and 16-byte aligned pointers
    assert call(lib, A0, B0, C0, 8, 6, 8, fgr.PATH_MFMA_VEC) == fgr.ERR_BAD_PATH
    assert call(lib, A0, B0, C0, 8, 8, 6, fgr.PATH_MFMA_VEC) == fgr.ERR_BAD_PATH
    assert call(lib, A0 + 4, B0, C0, 8, 8, 8, fgr.PATH_MFMA_VEC) == fgr.ERR_BAD_PATH
    # matrix-vector paths need M <= 8
    assert call(lib, A0, B0, C0, 9, 8, 8, fgr.PATH_GEMV_VEC) == fgr.ERR_BAD_PATH
    assert call(lib, A0, B0, C0, 9, 8, 8, fgr.PATH_GEMV_SCALAR) == fgr.ERR_BAD_PATH
    assert call(lib, A0, B0, C0, 1, 8, 6, fgr.PATH_GEMV_VEC) == fgr.ERR_BAD_PATH
    # the direct-copy paths need N >= 64 and tile 256; rows that are not
    # 16-byte aligned take 4-byte copies (accepted: without a GPU the call then
    # stops at the device check)
    assert call(lib, A0, B0, C0, 512, 60, 512, fgr.PATH_MFMA_DMA) == fgr.ERR_BAD_PATH
    assert call(lib, A0, B0, C0, 512, 128, 512, fgr.PATH_MFMA_DMA, 128) == fgr.ERR_BAD_PATH
    assert call(lib, A0, B0, C0, 512, 60, 512, fgr.PATH_MFMA_DMA_TAIL) == fgr.ERR_BAD_PATH
    # the copies address 256 rows of A and 16 rows of B with 32-bit byte
    # offsets: N <= 4194303 (= (2^32 - 1) / 1024), K <= 67108863
    # (operands far apart, so that these sizes do not overlap)
    a, b, c = 1 << 44, 2 << 44, 3 << 44
    for path in (fgr.PATH_MFMA_KSPLIT, fgr.PATH_MFMA_SPLITK):
        assert call(lib, a, b, c, 16, 33554432, 128, path, fgr.TILE_32X128) == fgr.ERR_BAD_PATH
        assert call(lib, a, b, c, 16, 128, 134217728, path, fgr.TILE_32X128) == fgr.ERR_BAD_PATH
        assert call(lib, a, b, c, 16, 33554431, 128, path, fgr.TILE_32X128) == fgr.ERR_DEVICE
    for path in (fgr.PATH_MFMA_DMA, fgr.PATH_MFMA_DMA_TAIL):
        assert call(lib, a, b, c, 512, 4194304, 512, path) == fgr.ERR_BAD_PATH
        assert call(lib, a, b, c, 512, 4194303, 512, path) == fgr.ERR_DEVICE
        assert call(lib, a, b, c, 256, 128, 67108864, path) == fgr.ERR_BAD_PATH
        assert call(lib, a, b, c, 256, 128, 67108863, path) == fgr.ERR_DEVICE
    for path in (fgr.PATH_MFMA_DMA, fgr.PATH_MFMA_DMA_TAIL):
        assert call(lib, A0, B0, C0, 512, 130, 512, path) == fgr.ERR_DEVICE
        assert call(lib, A0, B0, C0, 512, 128, 502, path) == fgr.ERR_DEVICE
        assert call(lib, A0 + 4, B0, C0, 512, 128, 512, path) == fgr.ERR_DEVICE
    # the k-split paths need N >= 64; tile 128 takes rows at any alignment
    # but needs K >= 4 (four columns of B per lane); the tail form has no
    # 32x32 tiles
    assert call(lib, A0, B0, C0, 512, 60, 512, fgr.PATH_MFMA_KSPLIT) == fgr.ERR_BAD_PATH
    assert call(lib, A0, B0, C0, 512, 130, 502, fgr.PATH_MFMA_KSPLIT, 128) == fgr.ERR_DEVICE  # neither aligned
    assert call(lib, A0 + 4, B0 + 4, C0, 512, 128, 512, fgr.PATH_MFMA_KSPLIT_TAIL, 128) == fgr.ERR_DEVICE
    assert call(lib, A0 + 4, B0, C0 + 4, 512, 128, 512, fgr.PATH_MFMA_KSPLIT, 128) == fgr.ERR_DEVICE  # B, not C
    assert call(lib, A0, B0, C0, 512, 128, 3, fgr.PATH_MFMA_KSPLIT, 128) == fgr.ERR_BAD_PATH  # K < 4
    assert call(lib, A0, B0, C0, 512, 128, 4, fgr.PATH_MFMA_KSPLIT, 128) == fgr.ERR_DEVICE
    assert call(lib, A0, B0, C0, 512, 128, 502, fgr.PATH_MFMA_KSPLIT, 128) == fgr.ERR_DEVICE  # A rows only
    assert call(lib, A0, B0 + 4, C0, 512, 128, 512, fgr.PATH_MFMA_KSPLIT_TAIL, 128) == fgr.ERR_DEVICE
    assert call(lib, A0 + 4, B0, C0, 512, 128, 512, fgr.PATH_MFMA_KSPLIT, 128) == fgr.ERR_DEVICE  # B and C rows
    assert call(lib, A0, B0, C0, 512, 128, 512, fgr.PATH_MFMA_KSPLIT, 256) == fgr.ERR_BAD_PATH
    assert call(lib, A0, B0, C0, 512, 128, 512, fgr.PATH_MFMA_KSPLIT_TAIL, 32) == fgr.ERR_BAD_PATH
    for tile in (0, 64, 32):
        assert call(lib, A0, B0, C0, 512, 128, 502, fgr.PATH_MFMA_KSPLIT, tile) == fgr.ERR_DEVICE
        assert call(lib, A0 + 4, B0, C0, 512, 128, 512, fgr.PATH_MFMA_KSPLIT, tile) == fgr.ERR_DEVICE
    # the cross-workgroup split needs N >= 128 (two parts of 8 chunks); tile
    # 128 needs K >= 4; no 256 tiles
    assert call(lib, A0, B0, C0, 512, 120, 512, fgr.PATH_MFMA_SPLITK) == fgr.ERR_BAD_PATH
    assert call(lib, A0 + 4, B0, C0 + 4, 512, 128, 512, fgr.PATH_MFMA_SPLITK, 128) == fgr.ERR_DEVICE
    assert call(lib, A0, B0, C0, 512, 128, 2, fgr.PATH_MFMA_SPLITK, 128) == fgr.ERR_BAD_PATH
    assert call(lib, A0, B0, C0, 512, 128, 512, fgr.PATH_MFMA_SPLITK, 256) == fgr.ERR_BAD_PATH
    for tile in (0, 128, 64, 32):
        assert call(lib, A0, B0, C0, 512, 128, 512, fgr.PATH_MFMA_SPLITK, tile) == fgr.ERR_DEVICE
    # 32x128 tiles exist on the k-split paths (not their tail form) only
    assert call(lib, A0, B0, C0, 64, 128, 512, fgr.PATH_MFMA_KSPLIT, fgr.TILE_32X128) == fgr.ERR_DEVICE
    assert call(lib, A0, B0, C0, 64, 128, 512, fgr.PATH_MFMA_SPLITK, fgr.TILE_32X128) == fgr.ERR_DEVICE
    assert call(lib, A0, B0, C0, 64, 128, 512, fgr.PATH_MFMA_KSPLIT_TAIL, fgr.TILE_32X128) == fgr.ERR_BAD_PATH
    assert call(lib, A0, B0, C0, 64, 128, 512, fgr.PATH_MFMA_VEC, fgr.TILE_32X128) == fgr.ERR_BAD_PATH
    assert call(lib, A0, B0, C0, 64, 60, 512, fgr.PATH_MFMA_KSPLIT, fgr.TILE_32X128) == fgr.ERR_BAD_PATH
    assert call(lib, A0, B0, C0, 64, 60, 512, 0, fgr.TILE_32X128) == fgr.ERR_BAD_PATH
    # the vector-ALU path takes any shape, tile 128 only
    assert call(lib, A0 + 4, B0, C0, 7, 5, 3, fgr.PATH_VALU) == fgr.ERR_DEVICE
    assert call(lib, A0, B0, C0, 64, 64, 64, fgr.PATH_VALU, 128) == fgr.ERR_DEVICE
    assert call(lib, A0, B0, C0, 64, 64, 64, fgr.PATH_VALU, 64) == fgr.ERR_BAD_PATH
    # 32x32 tiles exist on the split and k-split paths only
    assert call(lib, A0, B0, C0, 64, 64, 64, fgr.PATH_MFMA_VEC, 32) == fgr.ERR_BAD_PATH
    assert call(lib, A0, B0, C0, 64, 64, 64, fgr.PATH_MFMA_SPLIT, 128) == fgr.ERR_BAD_PATH
    # unknown path or tile values
    assert call(lib, A0, B0, C0, 8, 8, 8, 99) == fgr.ERR_BAD_PATH
    assert call(lib, A0, B0, C0, 8, 8, 8, fgr.PATH_MFMA_VEC, 100) == fgr.ERR_BAD_PATH


def test_path_selection_rules():
    sp, st = fgr.select_path, fgr.select_tile
    assert sp(A0, B0, C0, 8192, 6144, 4096) == fgr.PATH_MFMA_DMA
    assert sp(A0, B0, C0, 4096, 4096, 4096) == fgr.PATH_MFMA_DMA
    assert sp(A0, B0, C0, 4096, 4060, 4096) == fgr.PATH_MFMA_DMA  # ragged reduction
    assert sp(A0, B0, C0, 4000, 4096, 4004) == fgr.PATH_MFMA_DMA  # partial tiles
    assert sp(A0, B0, C0, 4096, 60, 4096) == fgr.PATH_MFMA_VEC  # N < 64
    # past the direct-copy kernel's 32-bit copy offsets: 128x128 k-split tiles
    a, b, c = 1 << 44, 2 << 44, 3 << 44
    assert sp(a, b, c, 4096, 4194303, 4096) == fgr.PATH_MFMA_DMA
    assert sp(a, b, c, 4096, 4194304, 4096) == fgr.PATH_MFMA_KSPLIT
    assert st(a, b, c, 4096, 4194304, 4096) == fgr.TILE_128
    # the skinny 32x128 tiles address 32 rows of A with 32-bit offsets: past
    # N = 33554431 the skinny shape takes the split plan's 32x32 tiles
    assert st(a, b, c, 16, 33554431, 128) == fgr.TILE_32X128
    assert st(a, b, c, 16, 33554432, 128) != fgr.TILE_32X128
    # a last partial wave of at most 176 tiles of 256x256 goes to the split kernel
    assert sp(A0, B0, C0, 4096, 4096, 4160) == fgr.PATH_MFMA_DMA_TAIL  # 272 tiles
    assert sp(A0, B0, C0, 65792, 128, 256) == fgr.PATH_MFMA_DMA_TAIL  # 257 tiles
    assert sp(A0, B0, C0, 4096, 4096, 6144) == fgr.PATH_MFMA_DMA_TAIL  # 384 tiles
    assert sp(A0, B0, C0, 4096, 4096, 6656) == fgr.PATH_MFMA_DMA_TAIL  # 416 tiles: 160 left over
    assert sp(A0, B0, C0, 4096, 4096, 7168) == fgr.PATH_MFMA_DMA  # 448 tiles: 192 left over
    assert sp(A0, B0, C0, 8192, 6208, 4160) == fgr.PATH_MFMA_DMA_TAIL  # 544 tiles
    assert sp(A0 + 4, B0, C0, 4096, 4096, 4160) == fgr.PATH_MFMA_DMA_TAIL  # 4-byte copies
    assert sp(A0, B0, C0, 2048, 2048, 2048) == fgr.PATH_MFMA_KSPLIT  # 64 tiles of 256, 256 of 128
    assert sp(A0, B0, C0, 1024, 6144, 4096) == fgr.PATH_MFMA_KSPLIT  # a row shard of the timed shape
    # 128x128 tiles in whole waves, three waves or more, or a last wave more
    # than three quarters full; else 64x64 tiles
    assert sp(A0, B0, C0, 3072, 3072, 3072) == fgr.PATH_MFMA_KSPLIT  # 576 of 128 (2.25 waves), aligned
    assert st(A0, B0, C0, 3072, 3072, 3072) == 64  # 2304 of 64: 9 whole waves
    assert sp(A0, B0, C0, 2048, 4096, 4096) == fgr.PATH_MFMA_KSPLIT  # 512 of 128: two whole waves
    assert st(A0, B0, C0, 2048, 4096, 4096) == 128
    assert sp(A0, B0, C0, 3001, 3001, 3001) == fgr.PATH_MFMA_KSPLIT  # 576 of 128, unaligned: 2209 of 64
    assert st(A0, B0, C0, 3001, 3001, 3001) == 64
    assert sp(A0, B0, C0, 2000, 3000, 2100) == fgr.PATH_MFMA_KSPLIT_TAIL  # 272 of 128: 1056 of 64
    assert st(A0, B0, C0, 2000, 3000, 2100) == 64
    assert sp(A0, B0, C0, 2304, 2304, 2304) == fgr.PATH_MFMA_KSPLIT_TAIL  # 324 of 128: 1296 of 64
    assert st(A0, B0, C0, 2304, 2304, 2304) == 64
    assert sp(A0, B0, C0, 2816, 2816, 2816) == fgr.PATH_MFMA_KSPLIT  # 484 of 128: 228 in the last wave
    assert st(A0, B0, C0, 2816, 2816, 2816) == 128
    assert sp(A0, B0, C0, 3584, 3584, 3584) == fgr.PATH_MFMA_KSPLIT_TAIL  # 784 of 128: three waves and 16
    assert st(A0, B0, C0, 3584, 3584, 3584) == 128
    assert sp(A0, B0, C0, 2047, 2047, 2047) == fgr.PATH_MFMA_KSPLIT  # 256 of 128, unaligned rows
    assert st(A0, B0, C0, 2047, 2047, 2047) == 128
    assert sp(A0, B0, C0, 2048, 60, 2048) == fgr.PATH_MFMA_VEC  # N < 64: no direct copies
    assert sp(A0, B0, C0, 2560, 2560, 2560) == fgr.PATH_MFMA_KSPLIT_TAIL  # 400 of 128: 1600 of 64, 64 left
    assert sp(A0, B0, C0, 8, 8, 6) == fgr.PATH_GEMV_SCALAR  # skinny, K % 4 != 0
    assert sp(A0, B0, C0, 40, 8, 6) == fgr.PATH_MFMA_SPLIT
    assert sp(A0 + 4, B0, C0, 8192, 8192, 8192) == fgr.PATH_MFMA_DMA  # misaligned A: 4-byte copies
    assert sp(A0, B0, C0 + 8, 8192, 8192, 8192) == fgr.PATH_MFMA_DMA
    # neither operand's rows aligned: direct copies (4 bytes wide) in whole
    # waves of 256x256 tiles or below N = 768 (the register-staged tiles below
    # N = 384); 128x128 k-split tiles where the 256x256 tiles leave a partial
    # last wave
    assert sp(A0, B0, C0, 8191, 6143, 4095) == fgr.PATH_MFMA_DMA  # 512 of 256: two whole waves
    assert sp(A0, B0, C0, 8191, 1023, 8191) == fgr.PATH_MFMA_DMA  # 1024 of 256
    assert sp(A0, B0, C0, 4095, 4097, 4099) == fgr.PATH_MFMA_KSPLIT_TAIL  # 272 of 256; 1056 of 128: 32 left
    assert st(A0, B0, C0, 4095, 4097, 4099) == 128
    assert sp(A0, B0, C0, 6143, 4095, 6143) == fgr.PATH_MFMA_KSPLIT  # 576 of 256; 2304 of 128
    assert st(A0, B0, C0, 6143, 4095, 6143) == 128
    assert sp(A0, B0, C0, 7167, 769, 7167) == fgr.PATH_MFMA_KSPLIT_TAIL  # 784 of 256; 3136 of 128: 64 left
    assert sp(A0, B0, C0, 7167, 767, 7167) == fgr.PATH_MFMA_DMA_TAIL
    assert sp(A0, B0, C0, 8191, 511, 8191) == fgr.PATH_MFMA_DMA
    assert sp(A0 + 4, B0, C0, 4096, 6144, 4096) == fgr.PATH_MFMA_DMA  # one operand aligned
    assert sp(A0, B0, C0, 8192, 60, 8190) == fgr.PATH_MFMA_SCALAR  # N < 64
    assert sp(A0, B0, C0, 1, 8192, 8192) == fgr.PATH_GEMV_VEC
    assert sp(A0, B0, C0, 1, 3, 1) == fgr.PATH_GEMV_SCALAR
    assert sp(A0, B0 + 4, C0, 1, 8, 8) == fgr.PATH_GEMV_SCALAR
    assert sp(A0, B0, C0, 2, 8192, 8192) == fgr.PATH_GEMV_VEC  # skinny: B streamed once
    assert sp(A0, B0, C0, 4, 8192, 8192) == fgr.PATH_GEMV_VEC
    assert sp(A0, B0, C0, 4, 8192, 8190) == fgr.PATH_GEMV_SCALAR
    assert sp(A0, B0, C0, 8, 8192, 64) == fgr.PATH_GEMV_VEC  # K < 128: no 32x128 tiles
    assert sp(A0, B0, C0, 8, 2048, 2048) == fgr.PATH_MFMA_SPLITK  # 5 <= M <= 8, small B: the split plan
    assert sp(A0, B0, C0, 4, 2048, 2048) == fgr.PATH_GEMV_VEC  # M <= 4: the matrix-vector kernel
    assert sp(A0, B0, C0, 8, 8192, 8192) == fgr.PATH_MFMA_SPLITK  # skinny: 32x128 tiles
    assert sp(A0, B0, C0, 9, 8192, 8192) == fgr.PATH_MFMA_SPLITK
    assert sp(0, B0, C0, 1, 8, 8) == fgr.ERR_NULL_POINTER


def test_tile_selection():
    st = fgr.select_tile
    assert st(A0, B0, C0, 8192, 6144, 4096) == 256  # 512 tiles of 256x256
    assert st(A0, B0, C0, 4096, 4096, 4096) == 256  # 256 tiles
    assert st(A0, B0, C0, 4096, 4096, 4160) == 256  # whole waves of 256x256, then the tail
    assert st(A0, B0, C0, 2048, 512, 2048) == 128  # k-split, 128x128
    assert st(A0, B0, C0, 1024, 1024, 1024) == 64  # k-split, 64x64 (256 of them)
    assert st(A0, B0, C0, 1023, 1025, 1027) == 64  # k-split 64x64 and a column strip
    assert st(A0, B0, C0, 256, 256, 256) == 32  # k-split, 32x32
    assert st(A0, B0, C0, 2048, 512, 1024) == 64  # 128 tiles of 128, 512 of 64
    assert st(A0, B0, C0, 2048, 60, 2048) == 64  # no direct copies (N < 64): register-staged 64x64
    assert st(A0, B0, C0, 4095, 4097, 4099) == 128  # unaligned rows, long reduction: k-split 128x128
    assert st(A0, B0, C0, 4095, 60, 4099) == 128  # N < 64: 32-bit loads, many tiles
    assert st(A0, B0, C0, 1, 8192, 8192) == 0  # matrix-vector
    assert st(0, B0, C0, 4, 4, 4) == fgr.ERR_NULL_POINTER


def test_split_path_choices():
    sp = fgr.select_path
    # fewer 256x256 tiles than CUs, N >= 64: k-split tiles, the largest that
    # still give every CU one (then the tail rule), else 32x32
    assert sp(A0, B0, C0, 1024, 1024, 1024) == fgr.PATH_MFMA_KSPLIT  # 256 tiles of 64
    assert sp(A0, B0, C0, 1024, 8192, 1024) == fgr.PATH_MFMA_KSPLIT
    assert sp(A0, B0, C0, 1536, 4096, 1536) == fgr.PATH_MFMA_KSPLIT_TAIL  # 576 of 64: 64 left over
    assert sp(A0, B0, C0, 1023, 1025, 1027) == fgr.PATH_MFMA_STRIP  # 256 of 64 and a 3-column strip
    assert sp(A0, B0, C0, 1023, 1025, 1036) == fgr.PATH_MFMA_KSPLIT_TAIL  # 272 of 64: a 12-column strip
    assert sp(A0, B0, C0, 2047, 2049, 2051) == fgr.PATH_MFMA_KSPLIT_TAIL  # 1056 of 64
    assert sp(A0, B0, C0, 256, 256, 256) == fgr.PATH_MFMA_KSPLIT  # 32x32
    assert sp(A0, B0, C0, 300, 500, 261) == fgr.PATH_MFMA_KSPLIT  # unaligned, few tiles: 32x32, operands into registers
    assert sp(A0 + 4, B0 + 4, C0, 512, 4096, 512) == fgr.PATH_MFMA_KSPLIT  # misaligned A and B
    # N < 64: the register-staged and split kernels
    assert sp(A0, B0, C0, 2048, 60, 2048) == fgr.PATH_MFMA_VEC
    assert sp(A0, B0, C0, 1024, 60, 1024) == fgr.PATH_MFMA_VEC  # 256 tiles of 64
    assert sp(A0, B0, C0, 512, 60, 512) == fgr.PATH_MFMA_SPLIT  # 64 tiles of 64
    assert sp(A0, B0, C0, 2047, 61, 2051) == fgr.PATH_MFMA_SCALAR


def test_short_reduction_choices():
    sp, st = fgr.select_path, fgr.select_tile
    # N < 104 with a 64x64 tile per CU: register-staged 64x64 tiles (the
    # work is writing C), even where 256x256 tiles would fill the device; but
    # from N = 72 on the direct-copy kernel where those make whole waves
    for shape in [(8192, 16, 8192), (8192, 64, 8192), (8192, 68, 8192), (6144, 100, 6144), (65792, 96, 256),
                  (1024, 8, 1024)]:
        assert sp(A0, B0, C0, *shape) == fgr.PATH_MFMA_VEC, shape
        assert st(A0, B0, C0, *shape) == 64, shape
    for shape in [(8192, 72, 8192), (4096, 100, 4096), (8192, 104, 8192)]:
        assert sp(A0, B0, C0, *shape) == fgr.PATH_MFMA_DMA, shape
    # unaligned rows: 32-bit loads, 128x128 tiles when there are many
    assert sp(A0, B0, C0, 8191, 17, 8191) == fgr.PATH_MFMA_SCALAR
    assert st(A0, B0, C0, 8191, 17, 8191) == 128
    assert st(A0, B0, C0, 1023, 33, 1025) == 64
    # unaligned rows up to N = 104, and up to 384 where the direct-copy kernel
    # would copy B 4 bytes at a time: 32-bit loads; B's rows aligned: direct copies
    assert sp(A0, B0, C0, 8191, 65, 8191) == fgr.PATH_MFMA_SCALAR
    assert st(A0, B0, C0, 8191, 65, 8191) == 128
    assert sp(A0, B0, C0, 8191, 383, 8191) == fgr.PATH_MFMA_SCALAR
    assert sp(A0, B0, C0, 8191, 385, 8191) == fgr.PATH_MFMA_DMA
    assert sp(A0, B0, C0, 8191, 128, 8191) == fgr.PATH_MFMA_SCALAR  # A's rows aligned, B's not
    assert sp(A0, B0, C0, 8191, 384, 8191) == fgr.PATH_MFMA_DMA
    assert sp(A0, B0, C0, 8192, 129, 8192) == fgr.PATH_MFMA_DMA  # B's rows aligned
    assert sp(A0, B0, C0, 8192, 101, 8192) == fgr.PATH_MFMA_SCALAR
    assert sp(A0, B0, C0, 2047, 97, 2049) == fgr.PATH_MFMA_SCALAR  # 1056 tiles of 64
    assert st(A0, B0, C0, 2047, 97, 2049) == 64
    assert sp(A0, B0, C0, 2047, 255, 2049) == fgr.PATH_MFMA_KSPLIT_TAIL  # few 256x256 tiles: k-split


def test_skinny_choices():
    sp, st = fgr.select_path, fgr.select_tile
    A0, B0, C0 = 1 << 40, 2 << 40, 3 << 40
    # 5 <= M <= 32 with K >= 128 and B of at least 32 MiB: 32x128 tiles, the
    # reduction split into the largest number of parts that keeps
    # tiles x parts <= CUs and parts >= 512 long (none: the k-split path)
    for shape, path in [((16, 4096, 4096), fgr.PATH_MFMA_SPLITK), ((32, 11008, 4096), fgr.PATH_MFMA_SPLITK),
                        ((5, 65536, 256), fgr.PATH_MFMA_SPLITK), ((8, 8192, 28672), fgr.PATH_MFMA_KSPLIT),
                        ((32, 4097, 4099), fgr.PATH_MFMA_SPLITK), ((16, 512, 65536), fgr.PATH_MFMA_KSPLIT)]:
        assert sp(A0, B0, C0, *shape) == path, shape
        assert st(A0, B0, C0, *shape) == fgr.TILE_32X128, shape
    parts = fgr.select_parts
    assert parts(A0, B0, C0, 33, 8200, 2052) == 7  # 34 tiles: 238 workgroups
    assert parts(A0, B0, C0, 16, 100000, 640) == 51  # 5 tiles
    assert parts(A0, B0, C0, 32, 11008, 4096) == 8  # 32 tiles
    assert parts(A0, B0, C0, 5, 65536, 256) == 128  # 2 tiles
    assert sp(A0, B0, C0, 4, 8192, 8192) == fgr.PATH_GEMV_VEC  # M < 5: the matrix-vector kernel
    assert st(A0, B0, C0, 64, 8192, 8192) == fgr.TILE_32X128  # two rows of tiles
    assert st(A0, B0, C0, 65, 8192, 8192) == 64  # M > 64: the tile-count rules
    assert st(A0, B0, C0, 16, 1048576, 64) == 32  # K < 128


def test_split_reduction_choices():
    sp, st = fgr.select_path, fgr.select_tile
    A0, B0, C0 = 1 << 40, 2 << 40, 3 << 40  # room for the long operands
    # few output tiles and a long reduction: the reduction is also split
    # across workgroups; 64x64 tiles for tall outputs, 32x32 for skinny ones
    # (less padding), by the time estimate
    for shape, tile in [((256, 65536, 256), 64), ((128, 262144, 128), 64), ((64, 65536, 1024), fgr.TILE_32X128),
                        ((512, 65536, 512), 128), ((16, 1048576, 64), 32), ((130, 20000, 66), 32),
                        ((24, 65536, 1024), fgr.TILE_32X128), ((16, 16384, 4096), fgr.TILE_32X128),
                        ((512, 8192, 512), 64), ((1024, 32768, 512), 128), ((96, 8192, 4096), 32)]:
        assert sp(A0, B0, C0, *shape) == fgr.PATH_MFMA_SPLITK, shape
        assert st(A0, B0, C0, *shape) == tile, shape
        assert sp(A0 + 4, B0, C0, *shape) == fgr.PATH_MFMA_SPLITK, shape  # 4-byte copies too
    # 128x128 split tiles (any row alignment): parts of at least 2048 and no
    # more padding than 64x64 tiles; shorter parts: 64x64
    for shape, tile in [((128, 524288, 128), 128), ((640, 65536, 640), 128), ((192, 262144, 192), 64),
                        ((320, 200000, 320), 64), ((256, 100000, 256), 64), ((128, 262144, 128), 64)]:
        assert sp(A0, B0, C0, *shape) == fgr.PATH_MFMA_SPLITK, shape
        assert st(A0, B0, C0, *shape) == tile, shape
    assert st(A0 + 4, B0, C0, 128, 524288, 128) == 128
    assert st(A0 + 4, B0 + 4, C0, 128, 524288, 128) == 128
    # parts per tile: powers of two, or the counts filling whole rounds of
    # the 256 CUs (nine 128x128 tiles: 28 parts, 252 workgroups; ten 64x64
    # tiles: 25); 1 off the split path, error codes for bad arguments
    parts = fgr.select_parts
    assert parts(A0, B0, C0, 384, 131072, 384) == 28
    assert parts(A0, B0, C0, 100, 30000, 300) == 25
    assert parts(A0, B0, C0, 512, 8192, 512) == 8
    assert parts(A0, B0, C0, 128, 262144, 128) == 128
    assert parts(A0, B0, C0, 8192, 6144, 4096) == 1
    assert parts(A0, B0, C0, 512, 4096, 512) == 1
    assert parts(A0, B0, C0, 0, 4096, 512) < 0
    # enough 32x32 tiles for every CU, or too short a reduction: no split
    assert sp(A0, B0, C0, 512, 4096, 512) == fgr.PATH_MFMA_KSPLIT
    assert sp(A0, B0, C0, 64, 8192, 4096) == fgr.PATH_MFMA_SPLITK  # skinny: 32x128 tiles
    assert sp(A0, B0, C0, 96, 2048, 4096) == fgr.PATH_MFMA_KSPLIT
    assert sp(A0, B0, C0, 640, 2048, 640) == fgr.PATH_MFMA_KSPLIT
    assert sp(A0, B0, C0, 65, 8192, 8192) == fgr.PATH_MFMA_KSPLIT
    assert sp(A0, B0, C0, 64, 100, 64) == fgr.PATH_MFMA_KSPLIT
    # tiles enough for every CU: the whole-device kernels, never a split
    assert sp(A0, B0, C0, 1024, 32768, 1024) == fgr.PATH_MFMA_KSPLIT
    assert sp(A0, B0, C0, 8192, 65536, 8192) == fgr.PATH_MFMA_DMA


def test_python_wrapper_rejects_cpu_tensors():
    torch = pytest.importorskip("torch")
    a = torch.zeros(4, dtype=torch.float32)
    with pytest.raises(ValueError):
        fgr.solve(a, a, a, 2, 2, 2)
    with pytest.raises(TypeError):
        fgr.solve(a.double(), a, a, 2, 2, 2)


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    monkeypatch.setattr(fgr, "_lib", None)
    with pytest.raises(ImportError):
        fgr.load_library(str(tmp_path / "nope.so"))


def test_matrix_vector_rows_as_documented():
    # the header's rule: M <= 4 always takes the matrix-vector path; 5 <= M <= 8
    # too, unless N >= 64 and K >= 128 (then the k-split or split plans)
    sp = fgr.select_path
    a, b, c = 1 << 40, 2 << 40, 3 << 40
    gemv = (fgr.PATH_GEMV_VEC, fgr.PATH_GEMV_SCALAR)
    for M in range(1, 9):
        for N in (1, 17, 63, 64, 1000, 8192, 65536):
            for K in (1, 7, 64, 127, 128, 1000, 8192):
                p = sp(a, b, c, M, N, K)
                if M <= 4 or N < 64 or K < 128:
                    assert p in gemv, (M, N, K, p)
                else:
                    assert p not in gemv, (M, N, K, p)
    assert sp(a, b, c, 9, 8192, 64) not in gemv


def test_workspace_limit_round_trip(lib):
    # host only: the previous limit comes back; negative values mean no limit
    assert fgr.set_workspace_limit(0) == -1
    assert fgr.set_workspace_limit(1 << 20) == 0
    assert fgr.set_workspace_limit(-5) == 1 << 20
    assert fgr.set_workspace_limit(-1) == -1


def test_strip_choices():
    sp, st = fgr.select_path, fgr.select_tile
    a, b, c = 1 << 40, 2 << 40, 3 << 40
    # K = 64 q + w, 1 <= w <= 8: when the q column blocks of 64x64 tiles fit
    # one per CU and the w columns would add a partial second wave
    for shape in [(1023, 1025, 1027), (1024, 1024, 1028), (1023, 1024, 1027), (16384, 512, 67),
                  (1000, 2049, 1030), (1023, 1025, 1032), (4096, 1025, 257)]:
        assert sp(a, b, c, *shape) == fgr.PATH_MFMA_STRIP, shape
        assert st(a, b, c, *shape) == 64, shape
    assert sp(a, b, c, 1023, 1025, 1033) != fgr.PATH_MFMA_STRIP  # w = 9
    assert sp(a, b, c, 960, 1025, 1027) == fgr.PATH_MFMA_KSPLIT  # 255 tiles: one wave already
    assert sp(a, b, c, 1088, 1025, 1027) != fgr.PATH_MFMA_STRIP  # 17 x 16 whole tiles > 256
    # forced: any shape with such a K, N >= 64; tile AUTO or 64
    assert call(lib_handle(), A0, B0, C0, 100, 63, 70, fgr.PATH_MFMA_STRIP) == fgr.ERR_BAD_PATH  # N < 64
    assert call(lib_handle(), A0, B0, C0, 100, 64, 73, fgr.PATH_MFMA_STRIP) == fgr.ERR_BAD_PATH  # w = 9
    assert call(lib_handle(), A0, B0, C0, 100, 64, 64, fgr.PATH_MFMA_STRIP) == fgr.ERR_BAD_PATH  # w = 0
    assert call(lib_handle(), A0, B0, C0, 100, 64, 65, fgr.PATH_MFMA_STRIP, 128) == fgr.ERR_BAD_PATH


def lib_handle():
    return fgr.load_library()


def test_stream_read_rejects_bad_arguments(lib):
    # host-only checks of the measurement hook, before any HIP call
    sr = lib.fgr_stream_read
    assert sr(0, 1024, C0, 4, None) == fgr.ERR_NULL_POINTER
    assert sr(A0, 1024, 0, 4, None) == fgr.ERR_NULL_POINTER
    assert sr(A0, 1022, C0, 4, None) == fgr.ERR_BAD_DIMS  # n % 4
    assert sr(A0, 0, C0, 4, None) == fgr.ERR_BAD_DIMS
    assert sr(A0, 1024, C0, 0, None) == fgr.ERR_BAD_DIMS
    assert sr(A0 + 4, 1024, C0, 4, None) == fgr.ERR_MISALIGNED
    assert sr(A0, 1024, A0 + 16, 4, None) == fgr.ERR_ALIAS


def test_header_path_rules_in_order():
    # one shape per numbered rule of the header's "Alignment and paths" list
    sp, st = fgr.select_path, fgr.select_tile
    assert sp(A0, B0, C0, 4, 8192, 8192) == fgr.PATH_GEMV_VEC  # 1: M <= 4
    assert sp(A0, B0, C0, 8, 32, 8192) == fgr.PATH_GEMV_VEC  # 1: M <= 8, N < 64
    assert st(A0, B0, C0, 16, 8192, 8192) == fgr.TILE_32X128  # 2: B of 64 Mi floats
    assert sp(A0, B0, C0, 8, 2048, 2048) != fgr.PATH_GEMV_VEC  # 2: the shape, small B: on to 3-6
    assert (sp(A0, B0, C0, 6144, 100, 6144), st(A0, B0, C0, 6144, 100, 6144)) == (fgr.PATH_MFMA_VEC, 64)  # 3
    assert sp(A0, B0, C0, 8192, 100, 8192) == fgr.PATH_MFMA_DMA  # 3: N >= 72 with whole waves
    assert sp(A0, B0, C0, 8192, 6144, 4096) == fgr.PATH_MFMA_DMA  # 4
    assert (sp(A0, B0, C0, 2048, 2048, 2048), st(A0, B0, C0, 2048, 2048, 2048)) == (fgr.PATH_MFMA_KSPLIT, 128)  # 5
    assert sp(A0, B0, C0, 1023, 1025, 1027) == fgr.PATH_MFMA_STRIP  # 5: the strip plan
    assert sp(A0, B0, C0, 128, 262144, 128) == fgr.PATH_MFMA_SPLITK  # 5: few tiles, long N
    assert (sp(A0, B0, C0, 256, 32, 256), st(A0, B0, C0, 256, 32, 256)) == (fgr.PATH_MFMA_SPLIT, 32)  # 6
