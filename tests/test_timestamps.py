"""The measurement build (libfp32_gemm_row_ts.so, per-workgroup timestamps).

CPU: it exports everything the plain library does plus the one entry point
its header declares, the plain library does not export that one, its host
checks reject bad arguments, and bench.py's summary turns records into the
figures it reports (checked on synthetic records). GPU: a launch through the
measurement build records one plausible record per workgroup and computes
the same product as the oracle."""

import ctypes
import os
import re

import numpy as np
import pytest

import fp32_gemm_row_amd as fgr
from conftest import ROOT
from fp32_gemm_row_amd import build as fgr_build

TS_HEADER = os.path.join(ROOT, "include", "fp32_gemm_row_timestamps.h")


def ts_lib():
    if not os.path.exists(fgr_build.TS_LIB_PATH):
        pytest.fail(f"{fgr_build.TS_LIB_PATH} is not built (python -m fp32_gemm_row_amd.build --timestamps)")
    lib = ctypes.CDLL(fgr_build.TS_LIB_PATH)
    lib.fgr_timestamps_read.argtypes = [ctypes.c_void_p, ctypes.c_int]
    lib.fgr_timestamps_read.restype = ctypes.c_int
    return lib


def test_measurement_build_exports():
    text = re.sub(r"/\*.*?\*/", "", open(TS_HEADER, encoding="utf-8").read(), flags=re.S)
    declared = set(re.findall(r"^\s*(?:const\s+)?(?:\w+[\s*]+)+(\w+)\s*\(", text, flags=re.M))
    assert declared == {"fgr_timestamps_read"}
    lib = ts_lib()
    for name in declared | set(fgr.EXPORTS):
        assert hasattr(lib, name), name
    plain = fgr.load_library()
    with pytest.raises(AttributeError):
        plain.fgr_timestamps_read  # noqa: B018


def test_timestamps_read_argument_checks():
    lib = ts_lib()
    buf = np.zeros((1, 8), dtype=np.uint64)
    assert lib.fgr_timestamps_read(None, 1) == fgr.ERR_NULL_POINTER
    assert lib.fgr_timestamps_read(buf.ctypes.data, 0) == fgr.ERR_BAD_DIMS
    assert lib.fgr_timestamps_read(buf.ctypes.data, 4097) == fgr.ERR_BAD_DIMS


def test_summary_of_synthetic_records(tmp_path):
    # two launches of 16 workgroups, 2 per XCD; XCD x starts x * 0.5 us late,
    # loops last 1000 us at 2.4 GHz (2.4 M shader clocks), ends 6 us
    import bench
    import synth

    w = synth.Workload("t", 512, 4096, 512, "uniform", 0)
    launches = []
    for launch in range(2):
        rec = np.zeros((4096, 8), dtype=np.int64)
        base = 10_000_000 + launch * 1_000_000
        for b in range(16):
            x = b % 8
            t0 = base + x * 50  # 100 MHz ticks
            rec[b] = [t0, t0 + 100_000, t0 + 100_600, 7_000_000, 7_000_000 + 2_400_000, (x << 32) | 5, 0, 0]
        launches.append(rec)
    out = tmp_path / "ts.md"
    bench.timestamps_summary(w, "mfma_dma", 256, 1, launches, str(out), "cmd")
    text = out.read_text()
    assert "workgroups recorded per launch (tiles) | 16 (16)" in text
    assert "last XCD's first start after the first XCD's | 3.50 us" in text
    assert "| a tile workgroup's loop | 1000.00 us, 2400000 shader clocks |" in text
    assert "| a tile workgroup's end phase | 6.00 us |" in text
    assert "2.400 - 2.400 GHz" in text
    # a 256x256 tile over N = 4096: 2 * 256 * 256 * 4096 / 256 clocks per wave
    assert "| 2097152 (loop at 87.4% of them) |" in text
    assert "launch-span-us: 1009.50" in text


@pytest.mark.gpu
def test_measurement_build_records_and_result():
    import torch

    import oracle
    import synth

    lib = ts_lib()
    vp, ci = ctypes.c_void_p, ctypes.c_int
    lib.solve.argtypes = [vp, vp, vp, ci, ci, ci, vp]
    lib.solve.restype = ci
    M = N = K = 256
    A, B = synth.make_inputs(M, N, K, "integer", seed=3)
    dev = torch.device("cuda:0")
    dA = torch.from_numpy(A.ravel()).to(dev)
    dB = torch.from_numpy(B.ravel()).to(dev)
    dC = torch.full((M * K,), float("nan"), device=dev)
    torch.cuda.synchronize()
    print("measurement build: 256^3 through libfp32_gemm_row_ts.so", flush=True)
    assert lib.solve(dA.data_ptr(), dB.data_ptr(), dC.data_ptr(), M, N, K, None) == 0
    torch.cuda.synchronize()
    Cref, _ = oracle.gemm(A, B)
    assert np.array_equal(dC.cpu().numpy().reshape(M, K).astype(np.float64), Cref)
    buf = np.zeros((4096, 8), dtype=np.uint64)
    assert lib.fgr_timestamps_read(buf.ctypes.data, 4096) == 0
    rec = buf.astype(np.int64)
    live = rec[rec[:, 0] != 0]
    # 256^3 takes 32x32 k-split tiles: 64 workgroups, each a tile
    assert len(live) == 64 and (live[:, 6] == 0).all()
    assert (live[:, 0] <= live[:, 1]).all() and (live[:, 1] <= live[:, 2]).all()
    assert (live[:, 2] - live[:, 0] < 100_000).all()  # under 1 ms each
    assert (live[:, 4] > live[:, 3]).all()
    assert set(((live[:, 5] >> 32) & 0xFFFF).tolist()) <= set(range(8))
