"""fgr_solve_noalloc through the C ABI: its workspace comes from the library's
static 64 MiB device scratch instead of an allocation. Checked against
solve() (the same plan and kernels, so the same bits) and against the fp64
oracle (bit-exact on integer data, within 1e-5 * S + 1e-6 on uniform data),
on calls in a row whose later inputs are smaller, so that each call runs over
what the previous one left in the scratch."""

import sys

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
import fp32_gemm_row_amd as fgr  # noqa: E402

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_both(A, B):
    """(C from fgr_solve_noalloc, C from solve()) for numpy A, B; C prefilled with NaN."""
    M, N = A.shape
    K = B.shape[1]
    dA = torch.from_numpy(np.ascontiguousarray(A).ravel()).to(DEV)
    dB = torch.from_numpy(np.ascontiguousarray(B).ravel()).to(DEV)
    c_noalloc = torch.full((M * K,), float("nan"), device=DEV)
    c_solve = torch.full((M * K,), float("nan"), device=DEV)
    torch.cuda.synchronize()
    fgr.solve_noalloc(dA, dB, c_noalloc, M, N, K)
    torch.cuda.synchronize()
    fgr.solve(dA, dB, c_solve, M, N, K)
    torch.cuda.synchronize()
    return c_noalloc.cpu().numpy().reshape(M, K), c_solve.cpu().numpy().reshape(M, K)


def check(A, B, dist, label):
    C, C_solve = run_both(A, B)
    Cref, S = oracle.gemm(A, B)
    assert np.array_equal(C.view(np.uint32), C_solve.view(np.uint32)), f"{label}: differs from solve()"
    C64 = C.astype(np.float64)
    assert np.isfinite(C64).all(), f"{label}: non-finite outputs"
    if dist == "integer":
        assert np.array_equal(C64, Cref), f"{label}: not the oracle's exact result"
    else:
        err = np.abs(C64 - Cref) / oracle.tolerance(S)
        assert err.max() <= 1.0, f"{label}: max |err| / tol = {err.max():.3f}"


# Sequences of calls, each later input smaller than the one before. Plans:
# 128x128 split reduction (the largest split workspace), 64x64 split
# reduction, the tail split in the whole tiles' grid, the split
# matrix-vector product, and plans with no workspace.
SEQUENCES = [
    [(512, 65536, 512), (128, 262144, 128), (100, 30000, 300)],
    [(2047, 2049, 2051), (1023, 1025, 1027), (1, 262144, 64)],
    [(1536, 4096, 1536), (300, 4097, 259), (64, 64, 64)],
]


@pytest.mark.parametrize("seq", range(len(SEQUENCES)))
def test_noalloc_matches_solve_on_calls_in_a_row(seq):
    for i, (M, N, K) in enumerate(SEQUENCES[seq]):
        dist = "integer" if (i + seq) % 2 == 0 else "uniform"
        path = fgr.PATH_NAMES[fgr.select_path(1 << 40, 2 << 40, 3 << 40, M, N, K)]
        say(f"noalloc call {i}: {M}x{N}x{K} ({dist}, {path})")
        A, B = synth.make_inputs(M, N, K, dist, seed=50 + i)
        check(A, B, dist, f"{M}x{N}x{K} {dist}")


def test_noalloc_refuses_plans_beyond_the_limit():
    # a 128x128 split reduction whose partial tiles take 16 MiB, with the
    # workspace limit at 4 MiB: the call fails with FGR_ERR_SCRATCH and leaves
    # C as it was; with the limit lifted the same call runs
    M, N, K = 512, 65536, 512
    assert fgr.select_path(1 << 40, 2 << 40, 3 << 40, M, N, K) == fgr.PATH_MFMA_SPLITK
    say(f"noalloc refusal {M}x{N}x{K}")
    dA = torch.zeros(M * N, device=DEV)
    dB = torch.zeros(N * K, device=DEV)
    dC = torch.full((M * K,), float("nan"), device=DEV)
    torch.cuda.synchronize()
    old = fgr.set_workspace_limit(4 << 20)
    try:
        with pytest.raises(fgr.GemmError) as err:
            fgr.solve_noalloc(dA, dB, dC, M, N, K)
        assert err.value.code == fgr.ERR_SCRATCH
        torch.cuda.synchronize()
        assert torch.isnan(dC).all().item(), "a refused call wrote to C"
    finally:
        fgr.set_workspace_limit(old)
    fgr.solve_noalloc(dA, dB, dC, M, N, K)
    torch.cuda.synchronize()
    assert (dC == 0).all().item()
    # a small call right after still works
    A, B = synth.make_inputs(200, 3000, 100, "integer", seed=60)
    check(A, B, "integer", "200x3000x100 after a refusal")
