"""CPU oracle for C[M,K] = A[M,N] x B[N,K] (row-major FP32), in double precision.

TEST INFRASTRUCTURE ONLY. The tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` use it; the product package never imports it
and shares no code with it. The arithmetic lives in ``oracle.c`` (plain C,
built with gcc); this module only builds, loads and marshals.

Functions
    gemm(A, B, threads=0)        -> (C, S)   full product, float64
    gemm_at(A, B, rows, cols)    -> (C, S)   chosen elements, float64
    tolerance(S)                 -> 1e-5 * S + 1e-6 per element

Every function is pinned by ``tests/test_oracle.py`` against the pages' worked
examples, exact rational brute force, numpy's float64 product and identities.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")


def compile_source(src: str, out: str) -> str:
    """gcc -O2 -fopenmp: one C file to a shared library."""
    tmp = out + f".tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so (next to the source) if stale."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        compile_source(_SRC, _LIB)
    return _LIB


class Oracle:
    """Bindings of one build of oracle.c (the default one, or a test's variant)."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        f = ctypes.c_void_p
        i64 = ctypes.c_int64
        lib.oracle_gemm.argtypes = [f, f, i64, i64, i64, f, f, ctypes.c_int]
        lib.oracle_gemm.restype = None
        lib.oracle_gemm_at.argtypes = [f, f, i64, i64, i64, f, f, i64, f, f]
        lib.oracle_gemm_at.restype = i64
        lib.oracle_max_threads.argtypes = []
        lib.oracle_max_threads.restype = ctypes.c_int
        self.path = path
        self._lib = lib

    def gemm(self, A, B, threads: int = 0):
        """Full product in float64: returns (C, S), each of shape (M, K)."""
        A = np.asarray(A)
        B = np.asarray(B)
        if A.ndim != 2 or B.ndim != 2 or A.shape[1] != B.shape[0]:
            raise ValueError(f"shapes {A.shape} x {B.shape} do not chain")
        M, N = A.shape
        K = B.shape[1]
        A = _as_f32(A, M, N, "A")
        B = _as_f32(B, N, K, "B")
        C = np.empty((M, K), dtype=np.float64)
        S = np.empty((M, K), dtype=np.float64)
        self._lib.oracle_gemm(_ptr(A), _ptr(B), M, N, K, _ptr(C), _ptr(S), int(threads))
        return C, S

    def gemm_at(self, A, B, rows, cols):
        """Elements (rows[i], cols[i]) of the product: (C, S) of length len(rows)."""
        A = np.asarray(A)
        B = np.asarray(B)
        if A.ndim != 2 or B.ndim != 2 or A.shape[1] != B.shape[0]:
            raise ValueError(f"shapes {A.shape} x {B.shape} do not chain")
        M, N = A.shape
        K = B.shape[1]
        A = _as_f32(A, M, N, "A")
        B = _as_f32(B, N, K, "B")
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        cols = np.ascontiguousarray(cols, dtype=np.int64)
        if rows.shape != cols.shape:
            raise ValueError("rows and cols differ in length")
        C = np.empty(rows.size, dtype=np.float64)
        S = np.empty(rows.size, dtype=np.float64)
        bad = self._lib.oracle_gemm_at(_ptr(A), _ptr(B), M, N, K, _ptr(rows), _ptr(cols),
                                       rows.size, _ptr(C), _ptr(S))
        if bad:
            raise IndexError(f"{bad} sample coordinates lie outside the {M}x{K} product")
        return C, S

    def max_threads(self) -> int:
        return int(self._lib.oracle_max_threads())


_default = None


def _get() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle(build())
    return _default


def _as_f32(x, rows, cols, name):
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.size != rows * cols:
        raise ValueError(f"{name} has {x.size} elements, expected {rows}*{cols}")
    return x


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def gemm(A, B, threads: int = 0):
    """Full product in float64: returns (C, S), each of shape (M, K)."""
    return _get().gemm(A, B, threads)


def gemm_at(A, B, rows, cols):
    """Elements (rows[i], cols[i]) of the product: returns (C, S) of length len(rows)."""
    return _get().gemm_at(A, B, rows, cols)


def max_threads() -> int:
    return _get().max_threads()


def tolerance(S):
    """Per-element acceptance bound for FP32 results: 1e-5 * S + 1e-6."""
    return 1e-5 * np.asarray(S, dtype=np.float64) + 1e-6
