"""Seeded synthetic inputs for the row-major FP32 GEMM C[M,K] = A[M,N] x B[N,K].

This module only makes input matrices. It holds none of the product's
arithmetic, so both the HIP path and the CPU oracle can be fed from it
without sharing any code with each other.

Random stream
    One Mersenne Twister MT19937 stream per workload, seeded with a 32-bit
    integer by the classic initialisation of Matsumoto and Nishimura (1998),
    i.e. the same sequence as C++ ``std::mt19937(seed)``. numpy's legacy
    ``RandomState(seed)`` uses that generator and that seeding; its
    ``randint(0, 2**32, dtype=uint32)`` hands back the raw 32-bit draws
    (pinned in tests against the C++ standard's 10000th-draw value and
    against ``std::mt19937`` itself). A is filled row-major first, then B
    continues the same stream.

Value recipes (the pages fix none of them for the timed shape, beyond
"deterministic, non-zero"; these are the workloads' stated distributions):
    uniform  (u >> 8) * 2**-23 - 1       exact FP32 values in [-1, 1 - 2**-23]
    integer  (u mod 9) - 4               integers in {-4, ..., 4}
    normal   Box-Muller on two 53-bit uniforms, each uniform built from
             two draws as ((a >> 5) * 2**26 + (b >> 6)) * 2**-53;
             z = sqrt(-2 ln(1 - u1)) * cos(2 pi u2), times ``scale``,
             rounded to FP32.
    eighths  the exactly-summing deterministic pattern of the tutorial
             "分块计算与矩阵乘法" (section 3, the complete program):
             a[i] = ((17 i) mod 13 - 6) / 8 and b[i] = ((29 i) mod 11 - 5) / 8.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

__all__ = [
    "mt19937_draws",
    "uniform_values",
    "integer_values",
    "normal_values",
    "eighths_a",
    "eighths_b",
    "Workload",
    "WORKLOADS",
    "make_inputs",
]


def mt19937_draws(seed: int, count: int) -> np.ndarray:
    """The first ``count`` raw 32-bit outputs of MT19937 seeded with ``seed``."""
    if count == 0:
        return np.zeros(0, dtype=np.uint32)
    rs = np.random.RandomState(seed & 0xFFFFFFFF)
    return rs.randint(0, 2**32, size=count, dtype=np.uint32)


def uniform_values(draws: np.ndarray) -> np.ndarray:
    """One FP32 value in [-1, 1) per draw: (u >> 8) * 2**-23 - 1 (exact)."""
    hi = (draws >> np.uint32(8)).astype(np.float64)
    return (hi * 2.0**-23 - 1.0).astype(np.float32)


def integer_values(draws: np.ndarray) -> np.ndarray:
    """One integer-valued FP32 in {-4..4} per draw: (u mod 9) - 4."""
    return ((draws % np.uint32(9)).astype(np.int64) - 4).astype(np.float32)


def normal_values(draws: np.ndarray, scale: float) -> np.ndarray:
    """One N(0, scale^2) FP32 value per four draws (Box-Muller, cosine branch)."""
    if draws.size % 4:
        raise ValueError("normal_values needs four draws per value")
    d = draws.reshape(-1, 4).astype(np.uint64)
    u1 = ((d[:, 0] >> np.uint64(5)) * np.uint64(1 << 26) + (d[:, 1] >> np.uint64(6))).astype(np.float64)
    u2 = ((d[:, 2] >> np.uint64(5)) * np.uint64(1 << 26) + (d[:, 3] >> np.uint64(6))).astype(np.float64)
    u1 *= 2.0**-53
    u2 *= 2.0**-53
    z = np.sqrt(-2.0 * np.log1p(-u1)) * np.cos(2.0 * math.pi * u2)
    return (z * scale).astype(np.float32)


def eighths_a(count: int) -> np.ndarray:
    i = np.arange(count, dtype=np.int64)
    return (((i * 17) % 13 - 6) / 8.0).astype(np.float32)


def eighths_b(count: int) -> np.ndarray:
    i = np.arange(count, dtype=np.int64)
    return (((i * 29) % 11 - 5) / 8.0).astype(np.float32)


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    dist: str  # "uniform" | "integer" | "normal" | "eighths"
    seed: int

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K

    @property
    def algorithmic_bytes(self) -> int:
        return 4 * (self.M * self.N + self.N * self.K + self.M * self.K)


# The workloads: small cube (plus its integer twin for bit-exact checks),
# ragged odd sizes, large cube, the timed shape of the LeetGPU problem, the
# single-row (matrix-vector shaped) case, and a few-tile output over a long
# reduction (the shape class whose reduction is split across workgroups).
WORKLOADS = {
    "cube256": Workload("cube256", 256, 256, 256, "uniform", 0),
    "cube256_int": Workload("cube256_int", 256, 256, 256, "integer", 0),
    "ragged1023": Workload("ragged1023", 1023, 1025, 1027, "uniform", 1),
    "cube4096": Workload("cube4096", 4096, 4096, 4096, "uniform", 2),
    "leetgpu8192": Workload("leetgpu8192", 8192, 6144, 4096, "normal", 3),
    "gemv8192": Workload("gemv8192", 1, 8192, 8192, "uniform", 4),
    "longn128": Workload("longn128", 128, 262144, 128, "uniform", 5),
}


def make_inputs(M: int, N: int, K: int, dist: str, seed: int = 0):
    """Row-major A (M x N) and B (N x K) as contiguous float32 numpy arrays."""
    na, nb = M * N, N * K
    if dist == "eighths":
        return eighths_a(na).reshape(M, N), eighths_b(nb).reshape(N, K)
    per = 4 if dist == "normal" else 1
    draws = mt19937_draws(seed, per * (na + nb))
    if dist == "uniform":
        v = uniform_values(draws)
    elif dist == "integer":
        v = integer_values(draws)
    elif dist == "normal":
        v = normal_values(draws, 1.0 / math.sqrt(N))
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    A = np.ascontiguousarray(v[:na].reshape(M, N))
    B = np.ascontiguousarray(v[na:].reshape(N, K))
    return A, B


def workload_inputs(w: Workload):
    return make_inputs(w.M, w.N, w.K, w.dist, w.seed)
