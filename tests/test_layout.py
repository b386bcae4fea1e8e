"""The kernels' index and LDS layout helpers, checked on the CPU through a
test-only shim (tests/shim) that calls the library's own __host__ __device__
functions: the XCD renumbering and the grouped tile order are bijections whose
XCD shares are contiguous; the swizzled A layouts of the direct-copy and
k-split kernels put every element where the operand reads look for it, and
their 128-bit operand reads hit distinct 16-byte bank groups within every 8
lanes (32 banks) and every 16 lanes (64 banks). One GPU test runs a single
FP32 MFMA with the operand and result lane layouts the kernels assume and
compares it with the oracle."""

import ctypes
import importlib.util
import os

import numpy as np
import pytest

from conftest import ROOT

SHIM_DIR = os.path.join(ROOT, "tests", "shim")


def _load_shim():
    spec = importlib.util.spec_from_file_location("shim_build", os.path.join(SHIM_DIR, "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    lib = ctypes.CDLL(mod.build())
    ci, pi = ctypes.c_int, ctypes.POINTER(ctypes.c_int)
    lib.shim_xcd_remap.argtypes = [ci, ci]
    lib.shim_grouped_tile.argtypes = [ci, ci, ci, ci, pi, pi]
    lib.shim_grouped_tile.restype = None
    for name in ("shim_a_swizzle", "shim_a_swizzle2", "shim_dma_a_col", "shim_ksplit_a_col"):
        getattr(lib, name).argtypes = [ci]
    lib.shim_dma_a_read.argtypes = [ci, ci, ci]
    lib.shim_ksplit_a_read.argtypes = [ci, ci]
    lib.shim_kreg_cols.argtypes = [ci, ci, ci, ci, pi, pi]
    lib.shim_kreg_cols.restype = None
    vp = ctypes.c_void_p
    lib.shim_mfma_probe.argtypes = [vp, vp, vp, vp]
    return lib


@pytest.fixture(scope="module")
def shim():
    return _load_shim()


def tile_of(shim, logical, tiles_m, tiles_n, group):
    tm, tn = ctypes.c_int(), ctypes.c_int()
    shim.shim_grouped_tile(logical, tiles_m, tiles_n, group, ctypes.byref(tm), ctypes.byref(tn))
    return tm.value, tn.value


def test_xcd_remap_is_a_permutation_with_contiguous_xcd_shares(shim):
    # workgroup b runs on XCD b % 8; its logical id must be unique, and the ids
    # of one XCD a contiguous range (so neighbouring tiles share that XCD's L2)
    for nwg in list(range(1, 600)) + [1023, 1024, 2048, 4097, 8192]:
        ids = [shim.shim_xcd_remap(b, nwg) for b in range(nwg)]
        assert sorted(ids) == list(range(nwg)), nwg
        for x in range(8):
            mine = sorted(ids[b] for b in range(x, nwg, 8))
            if mine:
                assert mine == list(range(mine[0], mine[0] + len(mine))), (nwg, x)


@pytest.mark.parametrize("group", [1, 2, 3, 4, 8])
def test_grouped_tile_order_is_a_bijection(shim, group):
    shapes = [(tm, tn) for tm in range(1, 19) for tn in range(1, 19)] + [(32, 16), (16, 16), (4, 5), (8, 9),
                                                                         (16, 17), (33, 65), (1, 257)]
    for tm, tn in shapes:
        seen = [tile_of(shim, i, tm, tn, group) for i in range(tm * tn)]
        assert sorted(seen) == [(a, b) for a in range(tm) for b in range(tn)], (tm, tn, group)
        # `group` tile-rows at a time, row index fastest
        for i, (a, b) in enumerate(seen):
            assert a // group == i // (group * tn), (tm, tn, group, i)


def test_kernel_grid_order_covers_every_tile_once(shim):
    # the direct-copy and k-split kernels: block b -> grouped_tile(xcd_remap(b))
    for tm, tn in [(32, 16), (16, 16), (16, 17), (4, 5), (17, 15), (1, 1)]:
        grid = tm * tn
        seen = {tile_of(shim, shim.shim_xcd_remap(b, grid), tm, tn, 4) for b in range(grid)}
        assert len(seen) == grid, (tm, tn)


def bank_groups_distinct(offsets, lanes, groups):
    """Float offsets of one 128-bit read per lane: every `lanes` consecutive
    lanes hit `lanes` distinct 16-byte bank groups out of `groups`."""
    for a in range(0, len(offsets), lanes):
        g = [(o // 4) % groups for o in offsets[a:a + lanes]]
        if len(set(g)) != len(g):
            return False
    return True


def test_direct_copy_a_layout(shim):
    # A stage: 256 rows x 16 floats. Copy side: float position pos holds row
    # pos // 16, column dma_a_col(pos): a bijection onto the 256 x 16 chunk.
    where = {}
    for pos in range(256 * 16):
        r, c = pos // 16, shim.shim_dma_a_col(pos)
        assert 0 <= c < 16
        where[pos] = (r, c)
    assert sorted(where.values()) == [(r, c) for r in range(256) for c in range(16)]
    # Read side: lane (li, lg) of wave row wm reads quad q = 2h + lg of rows
    # a_row0 + 32 i, a_row0 = 128 wm + li; those four floats must be that
    # row's columns 4q .. 4q + 3, and each read conflict-free
    for wm in range(2):
        for i in range(4):
            for h in range(2):
                offs = []
                for lane in range(64):
                    li, lg = lane & 31, lane >> 5
                    row0, q = 128 * wm + li, 2 * h + lg
                    off = shim.shim_dma_a_read(row0, i, q)
                    assert off % 4 == 0
                    assert [where[off + e] for e in range(4)] == [(row0 + 32 * i, 4 * q + e) for e in range(4)]
                    offs.append(off)
                assert bank_groups_distinct(offs, 8, 8), (wm, i, h)
                assert bank_groups_distinct(offs, 16, 16), (wm, i, h)


@pytest.mark.parametrize("bm", [32, 64, 128])
def test_ksplit_a_layout(shim, bm):
    # a wave's A piece: bm rows x 8 floats
    where = {}
    for pos in range(bm * 8):
        r, c = pos // 8, shim.shim_ksplit_a_col(pos)
        assert 0 <= c < 8
        where[pos] = (r, c)
    assert sorted(where.values()) == [(r, c) for r in range(bm) for c in range(8)]
    for i in range(bm // 32):
        offs = []
        for lane in range(64):
            li, lg = lane & 31, lane >> 5
            off = shim.shim_ksplit_a_read(li, lg) + 32 * 8 * i
            assert [where[off + e] for e in range(4)] == [(li + 32 * i, 4 * lg + e) for e in range(4)]
            offs.append(off)
        assert bank_groups_distinct(offs, 8, 8), (bm, i)
        assert bank_groups_distinct(offs, 16, 16), (bm, i)


@pytest.mark.parametrize("kcb", [1, 2, 4])
def test_register_fed_columns(shim, kcb):
    # the register-fed k-split tiles (32 kcb columns, kcb adjacent columns per
    # lane): every lane's B load stays inside [0, K); the columns the tile's
    # lanes store cover [k0, min(k0 + 32 kcb, K)) exactly once; no store lies
    # left of the tile's first column (the store address is formed from
    # first - k0, which is negative at the right edge)
    first, skip = ctypes.c_int(), ctypes.c_int()
    bn = 32 * kcb
    for K in list(range(kcb, 4 * bn + 9)) + [1023, 1025, 1027, 4097, 6143]:
        for k0 in range(0, K, bn):
            stored = []
            for li in range(32):
                shim.shim_kreg_cols(k0, li, K, kcb, ctypes.byref(first), ctypes.byref(skip))
                f, sk = first.value, skip.value
                assert 0 <= f and f + kcb <= K, (K, k0, li, f)
                assert sk >= 0, (K, k0, li, sk)
                if sk == 0:
                    assert f == k0 + kcb * li
                cols = [f + j for j in range(sk, kcb)]
                assert all(c >= k0 for c in cols), (K, k0, li, cols)
                stored += cols
            assert sorted(stored) == list(range(k0, min(k0 + bn, K))), (K, k0)


def test_swizzles_stay_in_range(shim):
    assert {shim.shim_a_swizzle(r) for r in range(4096)} == {0, 1, 2, 3}
    assert {shim.shim_a_swizzle2(r) for r in range(4096)} == {0, 1}


@pytest.mark.gpu
def test_mfma_lane_layout_against_oracle(shim):
    # one v_mfma_f32_32x32x2_f32 fed and read back with the lane layouts the
    # kernels are written against: D must be the oracle's A x B exactly
    # (small integers: every sum exact); a wrong layout misplaces values
    torch = pytest.importorskip("torch")
    import oracle
    import synth

    for seed in range(4):
        A, B = synth.make_inputs(32, 2, 32, "integer", seed=70 + seed)
        dA = torch.from_numpy(A.ravel()).cuda()
        dB = torch.from_numpy(B.ravel()).cuda()
        dD = torch.full((32 * 32,), float("nan"), device="cuda")
        torch.cuda.synchronize()
        assert shim.shim_mfma_probe(dA.data_ptr(), dB.data_ptr(), dD.data_ptr(), None) == 0
        torch.cuda.synchronize()
        Cref, _ = oracle.gemm(A, B)
        D = dD.cpu().numpy().reshape(32, 32).astype(np.float64)
        assert np.array_equal(D, Cref), f"seed {seed}: MFMA layout differs from the oracle"
    # one-hot A: row i of D is row kk of B, every other row zero
    for i, kk in [(0, 0), (5, 1), (31, 0), (17, 1)]:
        A = np.zeros((32, 2), dtype=np.float32)
        A[i, kk] = 1.0
        B = (np.arange(64, dtype=np.float32) + 1).reshape(2, 32)
        dA = torch.from_numpy(A.ravel()).cuda()
        dB = torch.from_numpy(B.ravel()).cuda()
        dD = torch.full((32 * 32,), float("nan"), device="cuda")
        torch.cuda.synchronize()
        assert shim.shim_mfma_probe(dA.data_ptr(), dB.data_ptr(), dD.data_ptr(), None) == 0
        torch.cuda.synchronize()
        D = dD.cpu().numpy().reshape(32, 32)
        expect = np.zeros((32, 32), dtype=np.float32)
        expect[i] = B[kk]
        assert np.array_equal(D, expect), (i, kk)
