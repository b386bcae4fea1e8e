"""GPU parity: the HIP library through its C ABI against the CPU oracle.

Bars (per element):
  * exactly-summing inputs (the tutorial's eighths, small integers, the
    worked examples): bit-exact, C_gpu == C_oracle;
  * other inputs: finite and |C_gpu - C| <= 1e-5 * S + 1e-6 with
    S = sum_n |A[m,n]||B[n,k]|, both from the fp64 oracle.
C is prefilled with NaN before every call, so an element the kernels never
write fails the finiteness check.
"""

import collections
import sys

import numpy as np
import pytest

import oracle
import synth
from conftest import GOLDEN_FILES, load_golden

torch = pytest.importorskip("torch")
import fp32_gemm_row_amd as fgr  # noqa: E402

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
ALL_TILES = [fgr.TILE_256, fgr.TILE_128, fgr.TILE_64]


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def gpu_gemm(A, B, path=fgr.PATH_AUTO, tile=fgr.TILE_AUTO, offsets=(0, 0, 0), stream=None):
    """Run the library on A, B (numpy float32); return C as numpy float32.

    offsets shift each operand by that many floats inside a larger buffer, to
    hand the library pointers that are 4-byte but not 16-byte aligned."""
    M, N = A.shape
    K = B.shape[1]
    oa, ob, oc = offsets
    ba = torch.empty(M * N + oa, dtype=torch.float32, device=DEV)
    bb = torch.empty(N * K + ob, dtype=torch.float32, device=DEV)
    bc = torch.full((M * K + oc,), float("nan"), dtype=torch.float32, device=DEV)
    da, db, dc = ba[oa:], bb[ob:], bc[oc:]
    da.copy_(torch.from_numpy(np.ascontiguousarray(A, dtype=np.float32).ravel()))
    db.copy_(torch.from_numpy(np.ascontiguousarray(B, dtype=np.float32).ravel()))
    torch.cuda.synchronize()
    if path == fgr.PATH_AUTO and tile == fgr.TILE_AUTO:
        fgr.solve(da, db, dc, M, N, K, stream=stream)
    else:
        fgr.solve_path(da, db, dc, M, N, K, path, tile, stream=stream)
    torch.cuda.synchronize()
    return dc.cpu().numpy().reshape(M, K)


def assert_exact(C, Cref, label):
    C64 = C.astype(np.float64)
    bad = ~(C64 == Cref)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        detail = ", ".join(f"[{i},{j}] gpu={C[i, j]!r} ref={Cref[i, j]!r}" for i, j in idx)
        pytest.fail(f"{label}: {int(bad.sum())} of {bad.size} elements differ: {detail}")


def assert_within_tolerance(C, Cref, S, label):
    C64 = C.astype(np.float64)
    finite = np.isfinite(C64)
    if not finite.all():
        idx = np.argwhere(~finite)[:5]
        pytest.fail(f"{label}: {int((~finite).sum())} non-finite outputs, first at {idx.tolist()}")
    err = np.abs(C64 - Cref)
    tol = oracle.tolerance(S)
    bad = err > tol
    if bad.any():
        i = np.unravel_index(np.argmax(err / tol), err.shape)
        pytest.fail(
            f"{label}: {int(bad.sum())} elements beyond 1e-5*S+1e-6; worst at {tuple(int(x) for x in i)} "
            f"err={err[i]:.3e} tol={tol[i]:.3e}"
        )


def paths_for(M, N, K):
    """(path, tile) pairs able to run an (M, N, K) product from aligned buffers."""
    out = []
    for tile in ALL_TILES:
        out.append((fgr.PATH_MFMA_SCALAR, tile))
        if N % 4 == 0 and K % 4 == 0:
            out.append((fgr.PATH_MFMA_VEC, tile))
    if N >= 64:
        # direct copies: 16 bytes wide for 16-byte rows, 4 bytes otherwise
        out.append((fgr.PATH_MFMA_DMA, fgr.TILE_256))
        # below one wave of 256x256 tiles every tile is in the tail: the split
        # kernel's big-tile mode alone, partial big tiles included
        out.append((fgr.PATH_MFMA_DMA_TAIL, fgr.TILE_256))
    if N >= 64:
        # tiles whose reduction is split over the waves (operands into
        # registers for unaligned rows; 128x128 tiles need 16-byte rows); and
        # the tail form
        for tile in (fgr.TILE_64, fgr.TILE_32):
            out.append((fgr.PATH_MFMA_KSPLIT, tile))
        out.append((fgr.PATH_MFMA_KSPLIT_TAIL, fgr.TILE_64))
    if N >= 64 and K >= 4:
        # 128x128 tiles, operands into registers at any alignment
        out.append((fgr.PATH_MFMA_KSPLIT, fgr.TILE_128))
        out.append((fgr.PATH_MFMA_KSPLIT_TAIL, fgr.TILE_128))
    if N >= 64:
        out.append((fgr.PATH_MFMA_KSPLIT, fgr.TILE_32X128))
    if N >= 128:
        # the reduction also split across workgroups (two parts at least)
        for tile in (fgr.TILE_64, fgr.TILE_32, fgr.TILE_32X128):
            out.append((fgr.PATH_MFMA_SPLITK, tile))
        if K >= 4:
            out.append((fgr.PATH_MFMA_SPLITK, fgr.TILE_128))
    out.append((fgr.PATH_MFMA_SPLIT, fgr.TILE_32))
    out.append((fgr.PATH_MFMA_SPLIT, fgr.TILE_64))
    if N >= 64 and K > 64 and 1 <= K % 64 <= 8:
        out.append((fgr.PATH_MFMA_STRIP, fgr.TILE_64))  # the last K % 64 columns on the vector ALUs
    out.append((fgr.PATH_VALU, fgr.TILE_AUTO))  # vector ALUs, any shape
    if M <= 8:
        out.append((fgr.PATH_GEMV_SCALAR, 0))
        if K % 4 == 0:
            out.append((fgr.PATH_GEMV_VEC, 0))
    return out


# ------------------------------------------------------------ worked examples


@pytest.mark.parametrize("name", GOLDEN_FILES)
def test_worked_examples_every_path(name):
    M, N, K, A, B, C_expected = load_golden(name)
    say(f"worked example {name} M={M} N={N} K={K}")
    assert_exact(gpu_gemm(A, B), C_expected, f"{name} auto")
    for path, tile in paths_for(M, N, K):
        assert_exact(gpu_gemm(A, B, path, tile), C_expected, f"{name} path={path} tile={tile}")


# ------------------------------------------------- exact shapes, every path

EXACT_SHAPES = [
    (1, 1, 1), (2, 2, 2), (1, 3, 1), (2, 3, 2), (3, 5, 4), (17, 19, 23), (17, 19, 31),
    (129, 96, 132), (256, 96, 256), (255, 257, 129), (257, 129, 193), (512, 512, 512),
    (2, 64, 64), (5, 64, 60), (8, 64, 64),
    (70, 1, 70), (70, 15, 70), (70, 16, 70), (70, 17, 70),
    (70, 70, 1), (70, 70, 3), (70, 70, 4), (70, 70, 5),
    (1, 8, 4), (1, 1000, 999), (1, 4097, 1028), (1, 17, 33),
    (513, 600, 515), (300, 2050, 260),
    # skinny products (M <= 8, B streamed once): several staged chunks of A
    # (2048 reduction indices per chunk at M = 8, 8192 at M = 2), ragged K
    (8, 4100, 96), (5, 4500, 100), (3, 4500, 36), (2, 9000, 40), (8, 2050, 33), (7, 3000, 1),
    # direct global->LDS copy path: whole tiles, every count of 16-deep
    # chunks mod 3, 4 and 5 (4 to 9 chunks), ragged reduction (first chunk
    # partly below n = 0), partial tiles
    (256, 64, 256), (256, 128, 512), (512, 96, 256), (768, 320, 512),
    (300, 68, 260), (257, 100, 516), (520, 132, 300), (255, 1028, 257),
    (264, 84, 260), (256, 116, 264), (300, 1004, 300), (260, 144, 516),
]


@pytest.mark.parametrize("shape", EXACT_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_eighths_bit_exact_every_path(shape):
    M, N, K = shape
    A, B = synth.make_inputs(M, N, K, "eighths")
    Cref, _ = oracle.gemm(A, B)
    say(f"eighths {shape} auto")
    assert_exact(gpu_gemm(A, B), Cref, f"eighths {shape} auto")
    for path, tile in paths_for(M, N, K):
        say(f"eighths {shape} path={fgr.PATH_NAMES[path]} tile={tile}")
        assert_exact(gpu_gemm(A, B, path, tile), Cref, f"eighths {shape} path={path} tile={tile}")


@pytest.mark.parametrize("shape", [(64, 64, 64), (129, 96, 132), (33, 20, 45), (1, 64, 64), (1, 13, 7)],
                         ids=lambda s: "x".join(map(str, s)))
def test_misaligned_pointers_take_scalar_path(shape):
    M, N, K = shape
    A, B = synth.make_inputs(M, N, K, "eighths")
    Cref, _ = oracle.gemm(A, B)
    for offs in [(1, 0, 0), (0, 1, 0), (0, 0, 1), (3, 2, 1)]:
        say(f"misaligned {shape} offsets={offs}")
        assert_exact(gpu_gemm(A, B, offsets=offs), Cref, f"misaligned {shape} {offs}")
        if N >= 64:  # the direct-copy kernel with 4-byte copies
            assert_exact(gpu_gemm(A, B, fgr.PATH_MFMA_DMA, fgr.TILE_256, offsets=offs), Cref,
                         f"misaligned {shape} {offs} direct copies")


def test_vec_path_refuses_misaligned_pointer():
    A, B = synth.make_inputs(8, 8, 8, "eighths")
    ba = torch.zeros(65, device=DEV)
    b = torch.from_numpy(B.ravel()).to(DEV)
    c = torch.zeros(64, device=DEV)
    with pytest.raises(fgr.GemmError) as e:
        fgr.solve_path(ba[1:], b, c, 8, 8, 8, fgr.PATH_MFMA_VEC)
    assert e.value.code == fgr.ERR_BAD_PATH


# ----------------------------------------------------- the five workloads


def test_cube256_integer_bit_exact():
    w = synth.WORKLOADS["cube256_int"]
    A, B = synth.workload_inputs(w)
    Cref, _ = oracle.gemm(A, B)
    assert_exact(gpu_gemm(A, B), Cref, "cube256 integer auto")
    for tile in ALL_TILES:
        assert_exact(gpu_gemm(A, B, fgr.PATH_MFMA_VEC, tile), Cref, f"cube256 integer tile={tile}")
    assert_exact(gpu_gemm(A, B, fgr.PATH_MFMA_DMA, fgr.TILE_256), Cref, "cube256 integer direct-copy path")


@pytest.mark.parametrize("name", ["cube256", "ragged1023"])
def test_small_workloads_full_compare(name):
    w = synth.WORKLOADS[name]
    A, B = synth.workload_inputs(w)
    Cref, S = oracle.gemm(A, B)
    say(f"{name} auto path={fgr.PATH_NAMES[fgr.select_path(1 << 40, 2 << 40, 3 << 40, w.M, w.N, w.K)]}")
    assert_within_tolerance(gpu_gemm(A, B), Cref, S, f"{name} auto")
    for path, tile in paths_for(w.M, w.N, w.K):
        say(f"{name} path={fgr.PATH_NAMES[path]} tile={tile}")
        assert_within_tolerance(gpu_gemm(A, B, path, tile), Cref, S, f"{name} path={path} tile={tile}")


def sample_positions(M, K, tile, rng, extra=2048):
    """Corners of every tile (the ragged tail included) plus random positions."""
    rows, cols = [], []
    for m0 in range(0, M, tile):
        for k0 in range(0, K, tile):
            m1 = min(m0 + tile, M) - 1
            k1 = min(k0 + tile, K) - 1
            for (r, c) in ((m0, k0), (m0, k1), (m1, k0), (m1, k1)):
                rows.append(r)
                cols.append(c)
    rows.extend(rng.integers(0, M, size=extra).tolist())
    cols.extend(rng.integers(0, K, size=extra).tolist())
    return np.array(rows, dtype=np.int64), np.array(cols, dtype=np.int64)


@pytest.mark.parametrize("name", ["cube4096", "leetgpu8192", "longn128"])
def test_large_workloads_full_compare(name):
    # every output of the timed shape (8192 x 6144 x 4096), the 4096^3 cube and
    # the long-reduction shape against the full fp64 oracle product, as the
    # pages check their results (every element of C, not a sample)
    w = synth.WORKLOADS[name]
    say(f"{name}: generating inputs")
    A, B = synth.workload_inputs(w)
    path = fgr.select_path(1 << 40, 2 << 40, 3 << 40, w.M, w.N, w.K)
    tile = fgr.select_tile(1 << 40, 2 << 40, 3 << 40, w.M, w.N, w.K)
    say(f"{name}: GPU run (auto path {fgr.PATH_NAMES[path]}, tile {tile})")
    C = gpu_gemm(A, B)
    say(f"{name}: full oracle product ({w.M}x{w.N}x{w.K})")
    Cref, S = oracle.gemm(A, B)
    ratio = float(np.max(np.abs(C.astype(np.float64) - Cref) / oracle.tolerance(S)))
    say(f"{name}: {C.size} outputs, max |err| / tol = {ratio:.4f}")
    assert_within_tolerance(C, Cref, S, f"{name} full")


@pytest.mark.parametrize("shape", [(8000, 6000, 4000), (3072, 3072, 3072), (1024, 8192, 1024), (2047, 2049, 2051),
                                   (4096, 1028, 4160), (8192, 2052, 4100), (4300, 1000, 4096),
                                   (1024, 6144, 4096), (2000, 3000, 2100), (8191, 6143, 4095), (4099, 1001, 4351)],
                         ids=lambda s: "x".join(map(str, s)))
def test_large_ragged_sampled(shape):
    # partial 256x256 tiles with a ragged reduction (direct-copy path), the
    # split path at 64x64 with eight and four waves, and the 32-bit path
    M, N, K = shape
    A, B = synth.make_inputs(M, N, K, "uniform", seed=11)
    say(f"large ragged {shape}: path {fgr.PATH_NAMES[fgr.select_path(1 << 40, 2 << 40, 3 << 40, M, N, K)]}")
    C = gpu_gemm(A, B)
    rng = np.random.default_rng(5)
    rows, cols = sample_positions(M, K, 64, rng, extra=1024)
    Cref, S = oracle.gemm_at(A, B, rows, cols)
    assert_within_tolerance(C[rows, cols][None, :], Cref[None, :], S[None, :], f"{shape} sampled")


@pytest.mark.parametrize("shape,path,tile", [
    ((2048, 128, 2048), fgr.PATH_MFMA_KSPLIT, 128), ((2040, 1000, 2044), fgr.PATH_MFMA_KSPLIT, 128),
    ((2176, 136, 2048), fgr.PATH_MFMA_KSPLIT_TAIL, 128), ((3072, 132, 3076), fgr.PATH_MFMA_KSPLIT_TAIL, 128),
    ((1024, 200, 1024), fgr.PATH_MFMA_KSPLIT, 64), ((1023, 1025, 1039), fgr.PATH_MFMA_KSPLIT_TAIL, 64),
    ((1536, 104, 1540), fgr.PATH_MFMA_KSPLIT_TAIL, 64), ((509, 300, 515), fgr.PATH_MFMA_KSPLIT, 32),
    ((512, 128, 512), fgr.PATH_MFMA_KSPLIT, 32),
    # long reductions: the tail tiles' reduction split across workgroups
    ((1023, 4097, 1039), fgr.PATH_MFMA_KSPLIT_TAIL, 64), ((2176, 4096, 2048), fgr.PATH_MFMA_KSPLIT_TAIL, 128),
    ((1088, 4100, 1024), fgr.PATH_MFMA_KSPLIT_TAIL, 64),
    # 128x128 tiles with one operand's rows unaligned: B's, then A's; ragged
    # M and K, a partial last wave
    ((2048, 2048, 2047), fgr.PATH_MFMA_KSPLIT, 128), ((2000, 1028, 2045), fgr.PATH_MFMA_KSPLIT, 128),
    ((2176, 1028, 2047), fgr.PATH_MFMA_KSPLIT_TAIL, 128), ((2047, 2051, 2048), fgr.PATH_MFMA_KSPLIT, 128),
    ((2040, 1025, 2044), fgr.PATH_MFMA_KSPLIT, 128), ((2176, 1025, 2048), fgr.PATH_MFMA_KSPLIT_TAIL, 128),
    # neither operand's rows aligned (N mod 4 = 3, 2, 1)
    ((2040, 2047, 2043), fgr.PATH_MFMA_KSPLIT, 128), ((2000, 2046, 2045), fgr.PATH_MFMA_KSPLIT, 128),
    ((2047, 2049, 2051), fgr.PATH_MFMA_KSPLIT_TAIL, 128),
    # tails of 64x64 tiles with N >= 1024: whole and split tiles in one grid
    # (16-byte copies of both operands, of B only, of A only)
    ((1040, 2048, 1040), fgr.PATH_MFMA_KSPLIT_TAIL, 64), ((1024, 1025, 1088), fgr.PATH_MFMA_KSPLIT_TAIL, 64),
    ((1088, 1028, 1027), fgr.PATH_MFMA_KSPLIT_TAIL, 64), ((1536, 1536, 1536), fgr.PATH_MFMA_KSPLIT_TAIL, 64),
], ids=lambda v: "x".join(map(str, v)) if isinstance(v, tuple) else str(v))
def test_ksplit_exact(shape, path, tile):
    # tiles whose reduction is split over a workgroup's waves (128, 64 or 32
    # square; operands through LDS or straight into registers by tile and
    # alignment), the listed form forced; with a partial last wave of them, the
    # rest cut into split-kernel tiles or split across workgroups: exact on
    # integer data whichever kernel computed an output. The automatic plan of
    # each shape (whose rules the CPU tests pin) too.
    M, N, K = shape
    A, B = synth.make_inputs(M, N, K, "integer", seed=6)
    say(f"k-split {shape}: oracle")
    Cref, _ = oracle.gemm(A, B)
    say(f"k-split {shape}: GPU, path {path} tile {tile}")
    assert_exact(gpu_gemm(A, B, path, tile), Cref, f"{shape} path {path} tile {tile}")
    assert_exact(gpu_gemm(A, B, fgr.PATH_MFMA_KSPLIT, tile), Cref, f"{shape} k-split only")
    assert_exact(gpu_gemm(A, B), Cref, f"{shape} auto")


@pytest.mark.parametrize("shape,tile", [
    ((128, 262144, 128), 64), ((256, 16384, 256), 64), ((100, 30000, 300), 64), ((16, 65536, 64), 32),
    ((130, 20000, 66), 32),
    ((96, 50001, 97), 64), ((64, 16384, 64), 32), ((512, 8192, 512), 64), ((384, 131072, 384), 128)], ids=lambda v: "x".join(map(str, v)) if isinstance(v, tuple) else str(v))
def test_split_reduction_exact(shape, tile):
    # few output tiles, long reduction: each tile's reduction split into parts
    # over workgroups, partial tiles added in part order by a second kernel;
    # on integer data every sum is exact (|sum| <= 16 N < 2^24), so the result
    # must be the oracle's bits whatever the split (and for forced tiles too)
    M, N, K = shape
    A, B = synth.make_inputs(M, N, K, "integer", seed=12)
    say(f"split reduction {shape}: oracle")
    Cref, _ = oracle.gemm(A, B)
    assert fgr.select_path(1 << 40, 2 << 40, 3 << 40, M, N, K) == fgr.PATH_MFMA_SPLITK
    assert fgr.select_tile(1 << 40, 2 << 40, 3 << 40, M, N, K) == tile
    assert fgr.select_parts(1 << 40, 2 << 40, 3 << 40, M, N, K) >= 2
    say(f"split reduction {shape}: GPU ({fgr.select_parts(1 << 40, 2 << 40, 3 << 40, M, N, K)} parts)")
    assert_exact(gpu_gemm(A, B), Cref, f"{shape} auto")
    tiles = [fgr.TILE_64, fgr.TILE_32] + ([fgr.TILE_128] if N % 4 == 0 and K % 4 == 0 else [])
    for t in tiles:
        assert_exact(gpu_gemm(A, B, fgr.PATH_MFMA_SPLITK, t), Cref, f"{shape} split tile {t}")
    assert_exact(gpu_gemm(A, B, offsets=(1, 1, 1)), Cref, f"{shape} 4-byte aligned")


@pytest.mark.parametrize("shape", [(1, 262144, 64), (4, 131072, 256), (5, 100003, 33), (3, 65536, 1000)],
                         ids=lambda s: "x".join(map(str, s)))
def test_split_matrix_vector_exact(shape):
    # matrix-vector and skinny products with few 32-column blocks: rows of B
    # split into parts over workgroups; exact on integer data
    M, N, K = shape
    A, B = synth.make_inputs(M, N, K, "integer", seed=13)
    say(f"split matrix-vector {shape}: oracle")
    Cref, _ = oracle.gemm(A, B)
    say(f"split matrix-vector {shape}: GPU")
    assert_exact(gpu_gemm(A, B), Cref, f"{shape} auto")
    assert_exact(gpu_gemm(A, B, fgr.PATH_GEMV_SCALAR), Cref, f"{shape} scalar")
    assert_exact(gpu_gemm(A, B, offsets=(1, 1, 1)), Cref, f"{shape} 4-byte aligned")


@pytest.mark.parametrize("shape,offsets", [
    ((1023, 1025, 1027), (0, 0, 0)),   # neither operand aligned, w = 3
    ((1023, 1025, 1027), (1, 2, 3)),
    ((1023, 1024, 1027), (0, 0, 0)),   # A aligned, B not
    ((1024, 1024, 1028), (0, 0, 0)),   # all aligned, w = 4
    ((1024, 1024, 1028), (0, 0, 1)),   # C misaligned
    ((1000, 2049, 1030), (0, 0, 0)),   # w = 6, ragged rows
    ((1023, 1025, 1032), (3, 0, 0)),   # w = 8, A misaligned, B aligned
    ((16384, 512, 67), (0, 0, 0)),     # one column block, many rows
    ((4096, 1025, 257), (0, 0, 0)),    # four column blocks, w = 1
], ids=lambda v: "x".join(map(str, v)) if isinstance(v, tuple) else str(v))
def test_strip_plan_exact(shape, offsets):
    # the last K % 64 columns on the vector ALUs, 64x64 k-split tiles on the
    # rest (operands through LDS with every row aligned, else into registers):
    # exact on integer data, auto and forced
    M, N, K = shape
    A, B = synth.make_inputs(M, N, K, "integer", seed=16)
    say(f"strip plan {shape} offsets {offsets}: oracle")
    Cref, _ = oracle.gemm(A, B)
    assert fgr.select_path(1 << 40, 2 << 40, 3 << 40, M, N, K) == fgr.PATH_MFMA_STRIP
    say(f"strip plan {shape} offsets {offsets}: GPU")
    assert_exact(gpu_gemm(A, B, offsets=offsets), Cref, f"{shape} auto {offsets}")
    assert_exact(gpu_gemm(A, B, fgr.PATH_MFMA_STRIP, 64, offsets=offsets), Cref, f"{shape} forced {offsets}")


@pytest.mark.parametrize("shape", [(100, 300, 70), (37, 64, 65), (5, 128, 72), (300, 4097, 129), (64, 64, 136)],
                         ids=lambda s: "x".join(map(str, s)))
def test_strip_plan_forced_small_exact(shape):
    M, N, K = shape
    A, B = synth.make_inputs(M, N, K, "integer", seed=17)
    Cref, _ = oracle.gemm(A, B)
    for offsets in [(0, 0, 0), (1, 1, 1)]:
        say(f"strip plan forced {shape} offsets {offsets}")
        assert_exact(gpu_gemm(A, B, fgr.PATH_MFMA_STRIP, 64, offsets=offsets), Cref, f"{shape} {offsets}")


# The register-fed k-split tiles: 128x128 and 32x32 tiles, and 64x64 tiles
# whenever a row of A, B or C is not 16-byte aligned, load their operands
# straight into registers (16-, 8- and 4-byte loads at 4-byte alignment). Cases: one, two and
# three columns (64x64 tiles take B two columns at a time; one column runs on
# 32x32 tiles; with three the last lane's pair is shifted back by one), N not
# a multiple of 8 (chunk 0 reaches below n = 0 and is zero-filled), partial
# row and column tiles, split parts written to copies of C and to compact
# slots (the tail tiles beside whole ones), the strip, and each operand's
# pointer 4 bytes past a 16-byte boundary.
KREG_CASES = [
    ((64, 64, 2), fgr.PATH_MFMA_KSPLIT, 64, (0, 0, 0)),
    ((65, 67, 3), fgr.PATH_MFMA_KSPLIT, 64, (0, 0, 0)),
    ((100, 71, 1), fgr.PATH_MFMA_KSPLIT, 64, (0, 0, 0)),
    ((100, 71, 1), fgr.PATH_MFMA_KSPLIT_TAIL, 64, (0, 0, 0)),
    ((130, 1025, 129), fgr.PATH_MFMA_KSPLIT, 64, (0, 0, 0)),
    ((130, 1025, 129), fgr.PATH_MFMA_SPLITK, 64, (0, 0, 0)),
    ((130, 1025, 129), fgr.PATH_MFMA_SPLITK, 32, (0, 0, 0)),
    ((1023, 1025, 1027), fgr.PATH_MFMA_KSPLIT_TAIL, 64, (0, 0, 0)),
    ((1023, 1025, 1027), fgr.PATH_MFMA_KSPLIT, 64, (0, 0, 0)),
    ((1023, 1025, 1027), fgr.PATH_MFMA_STRIP, 64, (0, 0, 0)),
    ((256, 256, 256), fgr.PATH_MFMA_KSPLIT, 64, (1, 1, 1)),
    ((256, 256, 256), fgr.PATH_MFMA_KSPLIT, 64, (1, 0, 0)),
    ((256, 256, 256), fgr.PATH_MFMA_KSPLIT, 64, (0, 3, 0)),
    ((256, 256, 256), fgr.PATH_MFMA_KSPLIT, 64, (0, 0, 2)),
    ((256, 256, 256), fgr.PATH_MFMA_KSPLIT, 32, (0, 0, 0)),
    ((96, 333, 97), fgr.PATH_MFMA_KSPLIT, 32, (0, 0, 0)),
    ((96, 8192, 96), fgr.PATH_MFMA_SPLITK, 32, (1, 2, 3)),
    # 128x128: four columns of B per lane, so the right edge shifts a lane
    # back by one to three columns; all alignments; split parts and tails
    ((130, 67, 4), fgr.PATH_MFMA_KSPLIT, 128, (0, 0, 0)),
    ((130, 67, 5), fgr.PATH_MFMA_KSPLIT, 128, (0, 0, 0)),
    ((130, 67, 6), fgr.PATH_MFMA_KSPLIT, 128, (1, 1, 1)),
    ((130, 67, 7), fgr.PATH_MFMA_KSPLIT, 128, (0, 0, 0)),
    ((257, 1025, 263), fgr.PATH_MFMA_KSPLIT, 128, (0, 0, 0)),
    ((257, 1025, 265), fgr.PATH_MFMA_KSPLIT, 128, (0, 1, 0)),
    ((256, 256, 256), fgr.PATH_MFMA_KSPLIT, 128, (0, 0, 0)),
    ((256, 256, 256), fgr.PATH_MFMA_KSPLIT, 128, (1, 0, 2)),
    ((130, 4097, 131), fgr.PATH_MFMA_SPLITK, 128, (0, 0, 0)),
    ((1023, 1025, 1027), fgr.PATH_MFMA_KSPLIT_TAIL, 128, (0, 0, 0)),
    ((2047, 2049, 2051), fgr.PATH_MFMA_KSPLIT, 128, (0, 0, 0)),
]


@pytest.mark.parametrize("shape,path,tile,offsets", KREG_CASES,
                         ids=lambda v: "x".join(map(str, v)) if isinstance(v, tuple) else str(v))
def test_register_fed_ksplit_exact(shape, path, tile, offsets):
    M, N, K = shape
    A, B = synth.make_inputs(M, N, K, "integer", seed=23)
    say(f"register-fed k-split {shape} path {path} tile {tile} offsets {offsets}: oracle")
    Cref, _ = oracle.gemm(A, B)
    say(f"register-fed k-split {shape} path {path} tile {tile} offsets {offsets}: GPU")
    assert_exact(gpu_gemm(A, B, path, tile, offsets=offsets), Cref, f"{shape} path={path} tile={tile} {offsets}")


@pytest.mark.parametrize("n,blocks", [(4, 1), (1 << 20, 256), ((1 << 20) + 36, 1000), (64, 512)])
def test_stream_read_sums(n, blocks):
    # the read-ceiling hook reads every float once: with small integers every
    # workgroup's sum is exact and the sums add up to the whole buffer's
    x = torch.from_numpy((np.arange(n) % 7).astype(np.float32)).to(DEV)
    out = torch.full((blocks,), float("nan"), device=DEV)
    fgr.stream_read(x, n, out, blocks)
    torch.cuda.synchronize()
    sums = out.cpu().numpy().astype(np.float64)
    assert np.isfinite(sums).all()
    assert sums.sum() == float((np.arange(n) % 7).sum())


def test_unaligned_128_with_split_tail_exact():
    # neither operand's rows 16-byte aligned (N, K odd), 128x128 register-fed
    # tiles forced with the tail form: 9 tiles, none in a whole wave, so all
    # of them are the tail, whose reduction (N >= 4096) is split over 28
    # parts through a workspace; the last column tile has 3 columns
    M, N, K = 300, 4097, 259
    A, B = synth.make_inputs(M, N, K, "integer", seed=14)
    Cref, _ = oracle.gemm(A, B)
    say(f"unaligned 128x128, split tail {M}x{N}x{K}")
    assert_exact(gpu_gemm(A, B, fgr.PATH_MFMA_KSPLIT_TAIL, fgr.TILE_128), Cref, "128x128 + split tail")
    assert_exact(gpu_gemm(A, B, fgr.PATH_MFMA_KSPLIT_TAIL, fgr.TILE_128, offsets=(1, 2, 3)), Cref,
                 "128x128 + split tail, 4-byte aligned pointers")


@pytest.mark.parametrize("shape,path,tile", [
    ((300, 4097, 259), fgr.PATH_MFMA_KSPLIT_TAIL, 128),     # 128x128 split tail -> split kernel
    ((2047, 2049, 2051), fgr.PATH_AUTO, 0),                 # 64x64 tail split in the tiles' grid
    ((1023, 1025, 1027), fgr.PATH_AUTO, 0),                 # strip plan: no workspace anyway
    ((1023, 1025, 1036), fgr.PATH_AUTO, 0),                 # tail split in the whole tiles' grid
    ((1023, 4097, 1027), fgr.PATH_MFMA_KSPLIT_TAIL, 64),    # tail split after the whole tiles
    ((128, 262144, 128), fgr.PATH_AUTO, 0),                 # split reduction -> unsplit tiles
    ((301, 8191, 127), fgr.PATH_MFMA_SPLITK, 128),          # forced 128x128 split -> unsplit
    ((1, 262144, 64), fgr.PATH_AUTO, 0),                    # split matrix-vector -> unsplit
], ids=lambda v: "x".join(map(str, v)) if isinstance(v, tuple) else str(v))
def test_no_workspace_fallbacks_exact(shape, path, tile):
    # with the workspace limit at 0 every plan that needs device memory beyond
    # A, B and C runs its form without it (no error); exact on integer data
    M, N, K = shape
    A, B = synth.make_inputs(M, N, K, "integer", seed=15)
    Cref, _ = oracle.gemm(A, B)
    say(f"no-workspace fallback {shape} path {path} tile {tile}")
    prev = fgr.set_workspace_limit(0)
    try:
        assert_exact(gpu_gemm(A, B, path, tile), Cref, f"{shape} without workspace")
        assert_exact(gpu_gemm(A, B, path, tile, offsets=(1, 1, 1)), Cref, f"{shape} without workspace, offsets")
    finally:
        fgr.set_workspace_limit(prev)
    assert_exact(gpu_gemm(A, B, path, tile), Cref, f"{shape} with workspace")


@pytest.mark.parametrize("shape", [(128, 262144, 128), (16, 1048576, 64), (1, 4194304, 16), (512, 65536, 512)],
                         ids=lambda s: "x".join(map(str, s)))
def test_split_reduction_long_sampled(shape):
    # long reductions at full size on uniform data: sampled outputs within
    # the tolerance (every tile and part boundary crossed by the samples)
    M, N, K = shape
    A, B = synth.make_inputs(M, N, K, "uniform", seed=14)
    say(f"long reduction {shape}: path {fgr.PATH_NAMES[fgr.select_path(1 << 40, 2 << 40, 3 << 40, M, N, K)]}")
    C = gpu_gemm(A, B)
    rng = np.random.default_rng(7)
    rows, cols = sample_positions(M, K, 32, rng, extra=256)
    Cref, S = oracle.gemm_at(A, B, rows, cols)
    assert_within_tolerance(C[rows, cols][None, :], Cref[None, :], S[None, :], f"{shape} sampled")


@pytest.mark.parametrize("shape,offsets", [
    ((520, 1023, 516), (0, 0, 0)),   # A rows unaligned: 4-byte copies of A, 16-byte of B, 128-bit stores
    ((520, 1024, 515), (0, 0, 0)),   # B and C rows unaligned
    ((520, 1024, 516), (0, 0, 1)),   # only C misaligned: 32-bit stores
    ((520, 1024, 516), (1, 0, 0)),   # only A misaligned
    ((520, 1024, 516), (0, 3, 0)),   # only B misaligned
    ((520, 1023, 515), (0, 0, 0)),   # nothing aligned: 4-byte copies of both, 3 stages
], ids=lambda v: "x".join(map(str, v)) if isinstance(v, tuple) else str(v))
def test_direct_copy_operand_alignments_exact(shape, offsets):
    # the direct-copy kernel picks 16- or 4-byte copies per operand and 128-
    # or 32-bit stores for C; every combination exact on integer data
    M, N, K = shape
    A, B = synth.make_inputs(M, N, K, "integer", seed=23)
    Cref, _ = oracle.gemm(A, B)
    say(f"direct copies {shape} offsets {offsets}")
    assert_exact(gpu_gemm(A, B, fgr.PATH_MFMA_DMA, fgr.TILE_256, offsets=offsets), Cref, f"{shape} {offsets}")
    assert_exact(gpu_gemm(A, B, fgr.PATH_MFMA_DMA_TAIL, fgr.TILE_256, offsets=offsets), Cref,
                 f"{shape} {offsets} tail form")


@pytest.mark.parametrize("shape,offsets", [
    ((300, 1023, 260), (0, 0, 0)), ((300, 1024, 259), (0, 0, 0)), ((300, 1024, 260), (0, 0, 1)),
    ((300, 1024, 260), (1, 0, 0)), ((300, 1024, 260), (0, 2, 0)), ((300, 1023, 259), (0, 0, 0)),
], ids=lambda v: "x".join(map(str, v)) if isinstance(v, tuple) else str(v))
def test_ksplit_operand_alignments_exact(shape, offsets):
    # the k-split kernel likewise picks 16- or 4-byte copies per operand, at
    # every tile size, split across workgroups or not; exact on integer data
    M, N, K = shape
    A, B = synth.make_inputs(M, N, K, "integer", seed=24)
    Cref, _ = oracle.gemm(A, B)
    say(f"k-split copies {shape} offsets {offsets}")
    for path, tile in [(fgr.PATH_MFMA_KSPLIT, 64), (fgr.PATH_MFMA_KSPLIT, 32), (fgr.PATH_MFMA_KSPLIT, fgr.TILE_32X128),
                       (fgr.PATH_MFMA_SPLITK, 64), (fgr.PATH_MFMA_SPLITK, fgr.TILE_32X128),
                       (fgr.PATH_MFMA_KSPLIT_TAIL, 64)]:
        assert_exact(gpu_gemm(A, B, path, tile, offsets=offsets), Cref, f"{shape} {offsets} path={path} tile={tile}")
    # 128x128 tiles, operands straight into registers at any alignment
    for path in (fgr.PATH_MFMA_KSPLIT, fgr.PATH_MFMA_SPLITK, fgr.PATH_MFMA_KSPLIT_TAIL):
        assert_exact(gpu_gemm(A, B, path, 128, offsets=offsets), Cref, f"{shape} {offsets} path={path} tile=128")


@pytest.mark.parametrize("shape", [(1023, 1025, 1027), (1024, 1024, 1024), (300, 2000, 260), (1, 3, 1), (129, 17, 5)],
                         ids=lambda s: "x".join(map(str, s)))
def test_vector_alu_path_exact(shape):
    # the register-tiled vector-ALU kernel: ragged tiles, ragged reduction,
    # 32-bit loads for unaligned rows; exact on integer data
    M, N, K = shape
    A, B = synth.make_inputs(M, N, K, "integer", seed=15)
    say(f"vector ALU {shape}: oracle")
    Cref, _ = oracle.gemm(A, B)
    say(f"vector ALU {shape}: GPU")
    assert_exact(gpu_gemm(A, B, fgr.PATH_VALU), Cref, f"{shape} vector ALU")
    assert_exact(gpu_gemm(A, B, fgr.PATH_VALU, offsets=(1, 2, 3)), Cref, f"{shape} vector ALU, 4-byte aligned")


def test_vector_alu_path_timed_shape_sampled():
    w = synth.WORKLOADS["leetgpu8192"]
    A, B = synth.workload_inputs(w)
    say("vector ALU at the timed shape: GPU")
    C = gpu_gemm(A, B, fgr.PATH_VALU)
    rng = np.random.default_rng(8)
    rows, cols = sample_positions(w.M, w.K, 128, rng)
    Cref, S = oracle.gemm_at(A, B, rows, cols)
    assert_within_tolerance(C[rows, cols][None, :], Cref[None, :], S[None, :], "vector ALU sampled")


@pytest.mark.parametrize("shape", [(4352, 112, 4096), (4100, 104, 4100), (2304, 108, 8192), (65792, 128, 256)],
                         ids=lambda s: "x".join(map(str, s)))
def test_partial_last_wave_exact(shape):
    # one or more whole waves of 256x256 tiles on the direct-copy kernel, the
    # last partial wave cut into small tiles for the split kernel: on integer
    # data every output is exact, whichever kernel computed it
    M, N, K = shape
    A, B = synth.make_inputs(M, N, K, "integer", seed=4)
    say(f"partial last wave {shape}: oracle")
    Cref, _ = oracle.gemm(A, B)
    assert fgr.select_path(1 << 40, 2 << 40, 3 << 40, M, N, K) == fgr.PATH_MFMA_DMA_TAIL
    say(f"partial last wave {shape}: GPU")
    assert_exact(gpu_gemm(A, B), Cref, f"{shape} auto (tail split)")
    assert_exact(gpu_gemm(A, B, fgr.PATH_MFMA_DMA, fgr.TILE_256), Cref, f"{shape} direct-copy only")


@pytest.mark.parametrize("shape,path,tile", [
    ((4352, 64, 4096), fgr.PATH_MFMA_VEC, 64), ((4100, 68, 4100), fgr.PATH_MFMA_VEC, 64),
    ((2304, 100, 8192), fgr.PATH_MFMA_VEC, 64), ((8191, 17, 8191), fgr.PATH_MFMA_SCALAR, 128),
    ((1023, 33, 1025), fgr.PATH_MFMA_SCALAR, 64), ((4096, 4, 4096), fgr.PATH_MFMA_VEC, 64),
    ((4096, 1, 4096), fgr.PATH_MFMA_SCALAR, 128)],
    ids=lambda v: "x".join(map(str, v)) if isinstance(v, tuple) else str(v))
def test_short_reduction_exact(shape, path, tile):
    # short reductions over many tiles take register-staged 64x64 (or, for
    # unaligned rows, 128x128) tiles; exact on integer data, and the same bits
    # as the direct-copy kernel where that can run
    M, N, K = shape
    A, B = synth.make_inputs(M, N, K, "integer", seed=18)
    say(f"short reduction {shape}: oracle")
    Cref, _ = oracle.gemm(A, B)
    assert fgr.select_path(1 << 40, 2 << 40, 3 << 40, M, N, K) == path
    assert fgr.select_tile(1 << 40, 2 << 40, 3 << 40, M, N, K) == tile
    say(f"short reduction {shape}: GPU")
    assert_exact(gpu_gemm(A, B), Cref, f"{shape} auto")
    if N >= 64:
        assert_exact(gpu_gemm(A, B, fgr.PATH_MFMA_DMA, fgr.TILE_256), Cref, f"{shape} direct copies")


@pytest.mark.parametrize("M", [2, 3, 5, 8, 16, 32])
def test_skinny_products_full_compare(M):
    # M rows of A against a 8192 x 8192 B: one pass over B for all rows (the
    # matrix-vector kernel for M <= 4, 32x128 k-split tiles from M = 5)
    N = K = 8192
    A, B = synth.make_inputs(M, N, K, "uniform", seed=20 + M)
    say(f"skinny M={M}: oracle")
    Cref, S = oracle.gemm(A, B)
    expect = fgr.PATH_GEMV_VEC if M < 5 else fgr.PATH_MFMA_SPLITK
    assert fgr.select_path(1 << 40, 2 << 40, 3 << 40, M, N, K) == expect
    say(f"skinny M={M}: GPU")
    assert_within_tolerance(gpu_gemm(A, B), Cref, S, f"skinny M={M} auto")
    if M <= 8:
        assert_within_tolerance(gpu_gemm(A, B, fgr.PATH_GEMV_SCALAR), Cref, S, f"skinny M={M} scalar")
    assert_within_tolerance(gpu_gemm(A, B, fgr.PATH_MFMA_KSPLIT, fgr.TILE_32X128), Cref, S,
                            f"skinny M={M} 32x128 unsplit")


@pytest.mark.parametrize("shape,path", [
    ((16, 8192, 4096), fgr.PATH_MFMA_SPLITK), ((24, 65536, 1024), fgr.PATH_MFMA_SPLITK),
    ((5, 65536, 256), fgr.PATH_MFMA_SPLITK), ((8, 8192, 28672), fgr.PATH_MFMA_KSPLIT),
    ((32, 4097, 4099), fgr.PATH_MFMA_SPLITK), ((31, 32768, 1000), fgr.PATH_MFMA_SPLITK),
    # two rows of 32x128 tiles
    ((48, 8192, 4096), fgr.PATH_MFMA_SPLITK), ((64, 4096, 11008), fgr.PATH_MFMA_KSPLIT),
    ((33, 8200, 2052), fgr.PATH_MFMA_SPLITK)],
    ids=lambda v: "x".join(map(str, v)) if isinstance(v, tuple) else str(v))
def test_skinny_tiles_exact(shape, path):
    # 32x128 tiles for skinny outputs: rows past M and columns past K padded,
    # 4-byte copies for unaligned rows, the reduction split across workgroups
    # or not; exact on integer data, forced unsplit and split alike
    M, N, K = shape
    A, B = synth.make_inputs(M, N, K, "integer", seed=19)
    say(f"skinny tiles {shape}: oracle")
    Cref, _ = oracle.gemm(A, B)
    assert fgr.select_path(1 << 40, 2 << 40, 3 << 40, M, N, K) == path
    assert fgr.select_tile(1 << 40, 2 << 40, 3 << 40, M, N, K) == fgr.TILE_32X128
    say(f"skinny tiles {shape}: GPU")
    assert_exact(gpu_gemm(A, B), Cref, f"{shape} auto")
    assert_exact(gpu_gemm(A, B, fgr.PATH_MFMA_KSPLIT, fgr.TILE_32X128), Cref, f"{shape} 32x128 unsplit")
    assert_exact(gpu_gemm(A, B, fgr.PATH_MFMA_SPLITK, fgr.TILE_32X128), Cref, f"{shape} 32x128 split")
    assert_exact(gpu_gemm(A, B, offsets=(1, 1, 1)), Cref, f"{shape} 4-byte aligned")


def test_gemv_workload_full_compare():
    w = synth.WORKLOADS["gemv8192"]
    A, B = synth.workload_inputs(w)
    Cref, S = oracle.gemm(A, B)
    assert fgr.select_path(1 << 40, 2 << 40, 3 << 40, w.M, w.N, w.K) == fgr.PATH_GEMV_VEC
    assert_within_tolerance(gpu_gemm(A, B), Cref, S, "gemv8192 auto")
    assert_within_tolerance(gpu_gemm(A, B, fgr.PATH_GEMV_SCALAR), Cref, S, "gemv8192 scalar")


# ------------------------------------------------------------- properties


@pytest.mark.parametrize("shape,path,tile", [
    ((1023, 1025, 1027), fgr.PATH_AUTO, 0),
    ((512, 256, 768), fgr.PATH_MFMA_DMA, 256),
    ((300, 500, 260), fgr.PATH_MFMA_SPLIT, 64),
    ((300, 500, 260), fgr.PATH_MFMA_KSPLIT, 128),
    ((300, 500, 261), fgr.PATH_MFMA_DMA, 256),
    ((1, 3000, 900), fgr.PATH_GEMV_VEC, 0),
    ((5, 3000, 900), fgr.PATH_GEMV_VEC, 0),
    ((256, 16384, 256), fgr.PATH_MFMA_SPLITK, 64),
    ((1, 262144, 64), fgr.PATH_GEMV_VEC, 0),
], ids=["ragged-auto", "dma", "split64", "ksplit", "dma-4byte", "gemv", "skinny", "splitk", "gemv-parts"])
def test_repeat_runs_are_bitwise_identical(shape, path, tile):
    # fixed reduction order and no atomics: identical bits on every run
    M, N, K = shape
    A, B = synth.make_inputs(M, N, K, "uniform", seed=3)
    first = gpu_gemm(A, B, path, tile)
    for _ in range(4):
        assert np.array_equal(gpu_gemm(A, B, path, tile), first, equal_nan=True)


def test_kernels_agree_bitwise_on_integer_data():
    # every MFMA kernel walks the reduction in the same order (the split kernel
    # only adds its per-wave partials at the end): on integer data all sums are
    # exact, so every path must give the oracle's bits
    A, B = synth.make_inputs(300, 256, 260, "integer", seed=9)
    Cref, _ = oracle.gemm(A, B)
    for path, tile in paths_for(300, 256, 260):
        assert_exact(gpu_gemm(A, B, path, tile), Cref, f"integer path={path} tile={tile}")


def test_identity_and_one_hot():
    rng = np.random.default_rng(0)
    B = rng.uniform(-1, 1, size=(300, 260)).astype(np.float32)
    assert_exact(gpu_gemm(np.eye(300, dtype=np.float32), B), B.astype(np.float64), "I x B")
    A = np.zeros((70, 300), dtype=np.float32)
    A[13, 299] = 1.0
    A[69, 0] = 1.0
    exp = np.zeros((70, 260))
    exp[13] = B[299]
    exp[69] = B[0]
    assert_exact(gpu_gemm(A, B), exp, "one-hot rows")


@pytest.mark.parametrize("shape", [(300, 500, 260), (1023, 1025, 1027), (64, 20000, 96), (4, 3000, 50)],
                         ids=lambda s: "x".join(map(str, s)))
def test_algebraic_invariants(shape):
    # properties of the product that hold exactly on integer data whichever
    # kernel runs each call: A = 0 gives C = 0; scaling A by a power of two
    # scales C exactly (on any finite data); (A B)^T = B^T A^T; column and row
    # blocks of C are the products of the matching blocks of A and B
    M, N, K = shape
    A, B = synth.make_inputs(M, N, K, "integer", seed=16)
    C = gpu_gemm(A, B)
    Cref, _ = oracle.gemm(A, B)
    assert_exact(C, Cref, f"{shape} product")
    assert_exact(gpu_gemm(np.zeros_like(A), B), np.zeros((M, K)), f"{shape} zero A")
    Au, Bu = synth.make_inputs(M, N, K, "uniform", seed=17)
    Cu = gpu_gemm(Au, Bu).astype(np.float64)
    assert_exact(gpu_gemm(Au * np.float32(2.0), Bu), 2.0 * Cu, f"{shape} 2A")
    assert_exact(gpu_gemm(Au, Bu * np.float32(0.25)), 0.25 * Cu, f"{shape} B/4")
    At = np.ascontiguousarray(A.T)
    Bt = np.ascontiguousarray(B.T)
    assert_exact(gpu_gemm(Bt, At), Cref.T, f"{shape} transpose")
    k1 = K // 3 + 1
    assert_exact(gpu_gemm(A, np.ascontiguousarray(B[:, :k1])), Cref[:, :k1], f"{shape} columns [0, {k1})")
    if k1 < K:
        assert_exact(gpu_gemm(A, np.ascontiguousarray(B[:, k1:])), Cref[:, k1:], f"{shape} columns [{k1}, K)")
    m1 = M // 2 + 1
    assert_exact(gpu_gemm(np.ascontiguousarray(A[:m1]), B), Cref[:m1], f"{shape} rows [0, {m1})")


def test_output_offsets_past_32_bits():
    # 256 rows of a 17,000,004-column C: row * K passes 2^32 inside a tile, so
    # the store offsets must be 64-bit (C alone is 17.4 GB, B 8.7 GB); integer
    # inputs, exact at sampled outputs (the last rows and columns included)
    M, N, K = 256, 128, 17_000_004
    gen = torch.Generator(device=DEV)
    gen.manual_seed(21)
    say("offsets past 2^32: inputs")
    dA = torch.randint(-4, 5, (M * N,), device=DEV, generator=gen).float()
    dB = torch.randint(-4, 5, (N * K,), device=DEV, generator=gen).float()
    dC = torch.full((M * K,), float("nan"), device=DEV)
    torch.cuda.synchronize()
    say(f"offsets past 2^32: GPU ({fgr.PATH_NAMES[fgr.select_path(dA, dB, dC, M, N, K)]})")
    fgr.solve(dA, dB, dC, M, N, K)
    torch.cuda.synchronize()
    rng = np.random.default_rng(22)
    rows = np.concatenate([np.array([255, 255, 254, 0, 128, 255]), rng.integers(0, M, 2000)])
    cols = np.concatenate([np.array([K - 1, K - 4, K - 1, K - 1, 16_777_217, 0]), rng.integers(0, K, 2000)])
    got = dC.view(M, K)[torch.from_numpy(rows).to(DEV), torch.from_numpy(cols).to(DEV)].cpu().numpy()
    del dC
    say("offsets past 2^32: oracle at sampled outputs")
    A = dA.cpu().numpy().reshape(M, N)
    B = dB.cpu().numpy().reshape(N, K)
    Cref, _ = oracle.gemm_at(A, B, rows, cols)
    assert_exact(got[None, :], Cref[None, :], "K = 17,000,004 sampled")


def test_single_product_reduction_is_exact():
    # N = 1: C[m,k] = a * b, one product (the padding adds exact zeros)
    rng = np.random.default_rng(1)
    a = rng.uniform(-1, 1, size=(130, 1)).astype(np.float32)
    b = rng.uniform(-1, 1, size=(1, 140)).astype(np.float32)
    exp = (a * b).astype(np.float64)  # float32 product, correctly rounded
    for path, tile in paths_for(130, 1, 140):
        assert_exact(gpu_gemm(a, b, path, tile), exp, f"N=1 path={path} tile={tile}")


def test_nan_in_a_row_poisons_only_that_row():
    A, B = synth.make_inputs(64, 64, 64, "eighths")
    A = A.copy()
    A[5, 7] = np.nan
    C = gpu_gemm(A, B)
    assert np.isnan(C[5]).all()
    mask = np.ones(64, dtype=bool)
    mask[5] = False
    Cref, _ = oracle.gemm(A[mask], B)
    assert_exact(C[mask], Cref, "rows without NaN")


@pytest.mark.parametrize("shape", [(1023, 1025, 1027), (1023, 1025, 1039), (128, 16384, 128), (4, 100000, 96),
                                   (16, 65536, 64), (300, 500, 261), (4100, 104, 4100)],
                         ids=lambda s: "x".join(map(str, s)))
def test_special_values_stay_in_their_row_and_column(shape):
    # a NaN in A poisons exactly its row of C and an infinity in B exactly its
    # column (with a sign mix, NaN or +-inf there), on the paths that pad,
    # clamp or split: the k-split tail in one grid, the split reduction
    # through the workspace, the split matrix-vector kernel, 32x32 tiles with
    # 4-byte copies, short reductions. Padding only ever multiplies zeros by
    # zeros, and clamped copies feed only outputs that are not stored.
    M, N, K = shape
    A, B = synth.make_inputs(M, N, K, "integer", seed=60)
    A, B = A.copy(), B.copy()
    rm, cn = M // 2, K - 1
    A[rm, N // 3] = np.nan
    B[N - 1, cn] = np.inf
    say(f"special values {shape}: {fgr.PATH_NAMES[fgr.select_path(1 << 40, 2 << 40, 3 << 40, M, N, K)]}")
    C = gpu_gemm(A, B)
    assert np.isnan(C[rm]).all()
    col = np.delete(C[:, cn], rm)
    assert (~np.isfinite(col)).all()
    rows = np.delete(np.arange(M), rm)
    Cref, _ = oracle.gemm(np.delete(A, rm, axis=0), np.delete(B, cn, axis=1))
    assert_exact(np.delete(C[rows], cn, axis=1), Cref, f"{shape} outside the poisoned row and column")


def test_runs_on_a_side_stream():
    A, B = synth.make_inputs(257, 129, 193, "eighths")
    Cref, _ = oracle.gemm(A, B)
    s = torch.cuda.Stream()
    assert_exact(gpu_gemm(A, B, stream=s), Cref, "side stream")


def test_concurrent_calls_on_separate_streams():
    # four host threads, each on its own stream, calling the library at once
    # (ctypes releases the GIL): the per-device probe and workspace pool are
    # shared, each split call's workspace is its own; exact on integer data
    import threading

    shapes = [(128, 65536, 64), (4, 100000, 96), (300, 500, 260), (16, 65536, 64)]
    cases = []
    for i, (M, N, K) in enumerate(shapes):
        A, B = synth.make_inputs(M, N, K, "integer", seed=30 + i)
        Cref, _ = oracle.gemm(A, B)
        cases.append((M, N, K, torch.from_numpy(A.ravel()).to(DEV), torch.from_numpy(B.ravel()).to(DEV), Cref))
    torch.cuda.synchronize()
    results, errors = [None] * len(cases), []

    def work(i):
        try:
            M, N, K, dA, dB, _ = cases[i]
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                outs = [torch.full((M * K,), float("nan"), device=DEV) for _ in range(8)]
                for dC in outs:
                    fgr.solve(dA, dB, dC, M, N, K, stream=s)
            s.synchronize()
            results[i] = [o.cpu().numpy().reshape(M, K) for o in outs]
        except Exception as e:  # reported below, in the main thread
            errors.append(f"thread {i}: {e!r}")

    threads = [threading.Thread(target=work, args=(i,)) for i in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for i, (M, N, K, _, _, Cref) in enumerate(cases):
        say(f"concurrent {M}x{N}x{K}: {fgr.PATH_NAMES[fgr.select_path(1 << 40, 2 << 40, 3 << 40, M, N, K)]}")
        for j, C in enumerate(results[i]):
            assert_exact(C, Cref, f"{M}x{N}x{K} call {j}")


@pytest.mark.parametrize("shape", [(264, 200, 520), (512, 96, 256), (300, 1028, 260)],
                         ids=lambda s: "x".join(map(str, s)))
def test_controlled_comparison_variants_exact(shape):
    # every controlled-comparison variant (LDS buffering x output tile x
    # reduction chunk) alone over the whole product: ragged M and K tails and
    # a reduction tail, exact on integer data
    M, N, K = shape
    A, B = synth.make_inputs(M, N, K, "integer", seed=50)
    Cref, _ = oracle.gemm(A, B)
    dA = torch.from_numpy(A.ravel()).to(DEV)
    dB = torch.from_numpy(B.ravel()).to(DEV)
    for v, name in enumerate(fgr.variant_names()):
        say(f"variant {name} {shape}")
        dC = torch.full((M * K,), float("nan"), device=DEV)
        fgr.solve_variant(dA, dB, dC, M, N, K, v)
        torch.cuda.synchronize()
        assert_exact(dC.cpu().numpy().reshape(M, K), Cref, f"{shape} {name}")


def random_shapes(count, seed):
    """Seeded random (M, N, K, offsets): dimensions log-uniform over 1..700
    (some reductions up to 20000), pointer offsets of 0-3 floats."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        M, N, K = (int(np.exp(rng.uniform(0, np.log(700)))) for _ in range(3))
        if i % 6 == 5:
            N = int(rng.integers(2000, 20000))
        offsets = tuple(int(x) for x in rng.integers(0, 4, size=3)) if i % 3 == 2 else (0, 0, 0)
        out.append((M, N, K, offsets))
    return out


def test_random_shapes_exact():
    # 60 seeded random shapes and alignments through solve()'s own choice
    # (every path the rules reach at these sizes), exact on integer data
    seen = collections.Counter()
    for (M, N, K, offsets) in random_shapes(60, seed=70):
        A, B = synth.make_inputs(M, N, K, "integer", seed=M * 7 + N * 3 + K)
        Cref, _ = oracle.gemm(A, B)
        path = fgr.PATH_NAMES[fgr.select_path(1 << 40, 2 << 40, 3 << 40, M, N, K)]
        seen[path] += 1
        say(f"random {M}x{N}x{K} offsets {offsets}: {path}")
        assert_exact(gpu_gemm(A, B, offsets=offsets), Cref, f"{M}x{N}x{K} offsets {offsets}")
    say(f"paths taken: {dict(seen)}")
    assert len(seen) >= 4


def test_random_large_shapes_sampled():
    # 16 seeded random shapes from 700 to 5000 per dimension, with random
    # alignments: the direct-copy, k-split (128x128 with buffer copies
    # included), tail and split-reduction paths as solve() picks them; on
    # integer data the sampled outputs (tile corners of 64x64 tiles and random
    # positions) must equal the oracle's exactly
    rng = np.random.default_rng(80)
    seen = collections.Counter()
    for i in range(16):
        M, N, K = (int(np.exp(rng.uniform(np.log(700), np.log(5000)))) for _ in range(3))
        offsets = tuple(int(x) for x in rng.integers(0, 4, size=3)) if i % 2 else (0, 0, 0)
        path = fgr.PATH_NAMES[fgr.select_path(1 << 40, 2 << 40, 3 << 40, M, N, K)]
        say(f"random large {M}x{N}x{K} offsets {offsets}: {path}")
        A, B = synth.make_inputs(M, N, K, "integer", seed=i + 90)
        C = gpu_gemm(A, B, offsets=offsets)
        rows, cols = sample_positions(M, K, 64, np.random.default_rng(i), extra=512)
        Cref, _ = oracle.gemm_at(A, B, rows, cols)
        assert_exact(C[rows, cols][None, :], Cref[None, :], f"{M}x{N}x{K} offsets {offsets} sampled")
        seen[path] += 1
    say(f"paths taken: {dict(seen)}")


def test_long_reduction_128_split_exact():
    # few output tiles over a long reduction, where solve() splits the
    # reduction over 128x128 tiles (parts of 2048 or more): aligned, and with
    # A's rows unaligned; exact on integer data at sampled outputs
    # (every |partial sum| stays below 4 * 4 * 524288 < 2^24)
    for (M, N, K), offsets in [((128, 524288, 128), (0, 0, 0)), ((128, 524288, 128), (1, 0, 0)),
                               ((512, 65536, 512), (0, 0, 0))]:
        assert fgr.select_tile((1 << 40) + 4 * offsets[0], 2 << 40, 3 << 40, M, N, K) == 128
        say(f"128x128 split {M}x{N}x{K} offsets {offsets}")
        A, B = synth.make_inputs(M, N, K, "integer", seed=M + 7)
        C = gpu_gemm(A, B, offsets=offsets)
        rows, cols = sample_positions(M, K, 128, np.random.default_rng(M), extra=256)
        Cref, _ = oracle.gemm_at(A, B, rows, cols)
        assert_exact(C[rows, cols][None, :], Cref[None, :], f"{M}x{N}x{K} offsets {offsets} sampled")


@pytest.mark.parametrize("N,tile", [(8388612, fgr.TILE_128), (16777220, fgr.TILE_64), (33554436, fgr.TILE_32)],
                         ids=["128-N8388612", "64-N16777220", "32-N33554436"])
def test_k_split_tiles_past_32bit_offsets(N, tile):
    # The k-split kernels address a tile's rows of A with 32-bit byte offsets
    # where tile * N * 4 < 2^32; past that (these N) they fall back to 64-bit
    # addresses (the LDS form of 64x64 and 32x32 tiles to the register-fed
    # one). Two rows, four columns, split over workgroups; within tolerance
    # against the fp64 oracle.
    M, K = 2, 4
    assert tile * N * 4 > 0xFFFFFFFF
    say(f"k-split tile {tile} past 32-bit offsets: {M}x{N}x{K}")
    A, B = synth.make_inputs(M, N, K, "uniform", seed=N % 1000)
    C = gpu_gemm(A, B, fgr.PATH_MFMA_SPLITK, tile)
    Cref, S = oracle.gemm(A, B)
    assert_within_tolerance(C, Cref, S, f"{M}x{N}x{K} tile {tile}")


def test_default_stream_is_torchs_current_stream():
    # solve() without a stream argument enqueues on torch's current stream
    # (the binding reads its raw handle); inside `with torch.cuda.stream(s)`
    # that is s
    assert fgr._current_stream_handle() == torch.cuda.current_stream().cuda_stream
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        assert fgr._current_stream_handle() == side.cuda_stream == torch.cuda.current_stream().cuda_stream
    assert fgr._current_stream_handle() == torch.cuda.current_stream().cuda_stream


def test_split_workspace_reuse_between_calls():
    # split calls back to back without synchronising: each stream's cached
    # workspace is reused by every call on it, and replaced by a larger one
    # mid-sequence (the old one freed in stream order); two streams
    # interleave their calls, each with its own workspace; then the
    # per-thread default stream (handle 2), which takes a workspace per call.
    # Exact on integer data.
    shapes = [(128, 16384, 128), (256, 65536, 256), (4, 100000, 96), (128, 16384, 128), (16, 65536, 64),
              (512, 8192, 512)]
    cases = []
    for i, (M, N, K) in enumerate(shapes):
        A, B = synth.make_inputs(M, N, K, "integer", seed=40 + i)
        Cref, _ = oracle.gemm(A, B)
        assert fgr.select_path(1 << 40, 2 << 40, 3 << 40, M, N, K) in (fgr.PATH_MFMA_SPLITK, fgr.PATH_GEMV_VEC)
        cases.append((M, N, K, torch.from_numpy(A.ravel()).to(DEV), torch.from_numpy(B.ravel()).to(DEV), Cref))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    for rep in range(2):
        for i, (M, N, K, dA, dB, _) in enumerate(cases):
            for j, st in enumerate(streams):
                dC = torch.full((M * K,), float("nan"), device=DEV)
                st.wait_stream(torch.cuda.current_stream())  # dC's fill
                fgr.solve(dA, dB, dC, M, N, K, stream=st)
                dC.record_stream(st)
                outs.append((i, f"stream {j} round {rep}", dC))
    per_thread = 2  # hipStreamPerThread
    for i, (M, N, K, dA, dB, _) in enumerate(cases):
        dC = torch.full((M * K,), float("nan"), device=DEV)
        torch.cuda.synchronize()
        fgr.solve(dA, dB, dC, M, N, K, stream=per_thread)
        outs.append((i, "per-thread stream", dC))
    torch.cuda.synchronize()
    for i, label, dC in outs:
        M, N, K, _, _, Cref = cases[i]
        say(f"workspace reuse {M}x{N}x{K} {label}")
        assert_exact(dC.cpu().numpy().reshape(M, K), Cref, f"{M}x{N}x{K} {label}")


@pytest.mark.parametrize("shape", [(512, 512, 512), (1023, 1025, 1027), (100, 30000, 300), (1, 262144, 64),
                                   (16, 8192, 4096)], ids=lambda s: "x".join(map(str, s)))
def test_graph_capture_replays(shape):
    # solve() captured into a HIP graph (torch.cuda.graph) and replayed three
    # times with eager work in between: one-kernel paths, the two-launch tail,
    # and the split paths whose stream-ordered workspace becomes a graph
    # allocation; every replay exact on integer data
    M, N, K = shape
    A, B = synth.make_inputs(M, N, K, "integer", seed=40)
    Cref, _ = oracle.gemm(A, B)
    dA = torch.from_numpy(A.ravel()).to(DEV)
    dB = torch.from_numpy(B.ravel()).to(DEV)
    dC = torch.full((M * K,), float("nan"), device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fgr.solve(dA, dB, dC, M, N, K)  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    say(f"graph capture {shape}: {fgr.PATH_NAMES[fgr.select_path(1 << 40, 2 << 40, 3 << 40, M, N, K)]}")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fgr.solve(dA, dB, dC, M, N, K)
    for r in range(3):
        dC.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_exact(dC.cpu().numpy().reshape(M, K), Cref, f"{shape} replay {r}")
        torch.randn(1000, device=DEV).sum().item()  # eager work between replays


def test_six_argument_form_uses_null_stream():
    A, B = synth.make_inputs(33, 40, 36, "eighths")
    Cref, _ = oracle.gemm(A, B)
    da = torch.from_numpy(A.ravel()).to(DEV)
    db = torch.from_numpy(B.ravel()).to(DEV)
    dc = torch.full((33 * 36,), float("nan"), device=DEV)
    torch.cuda.synchronize()
    lib = fgr.load_library()
    assert lib.fgr_solve_default(da.data_ptr(), db.data_ptr(), dc.data_ptr(), 33, 40, 36) == 0
    torch.cuda.synchronize()
    assert_exact(dc.cpu().numpy().reshape(33, 36), Cref, "six-argument form")
