"""Python binding of the MI355X row-major FP32 GEMM library (libfp32_gemm_row.so).

Argument marshalling only: every step of the product runs in the library's HIP
kernels (C ABI in include/fp32_gemm_row.h). torch provides device memory and
streams. If the built library is missing, importing the functions raises: there
is no fallback.

    solve(A, B, C, M, N, K, stream=None)   C[M,K] = A[M,N] x B[N,K]

A, B, C are float32 CUDA (HIP) tensors, contiguous, with at least M*N, N*K and
M*K elements (raw device addresses as ints are accepted too). `stream` is a
torch.cuda.Stream, a raw hipStream_t int, or None for torch's current stream.
"""

from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libfp32_gemm_row.so")

# Status codes and path / tile values (mirroring include/fp32_gemm_row.h).
OK = 0
ERR_NULL_POINTER = -1
ERR_BAD_DIMS = -2
ERR_MISALIGNED = -3
ERR_ALIAS = -4
ERR_BAD_PATH = -5
ERR_DEVICE = -6
ERR_LAUNCH = -7
ERR_SCRATCH = -8

PATH_AUTO = 0
PATH_MFMA_VEC = 1
PATH_MFMA_SCALAR = 2
PATH_GEMV_VEC = 3
PATH_GEMV_SCALAR = 4
PATH_MFMA_DMA = 5
PATH_MFMA_SPLIT = 6
PATH_MFMA_DMA_TAIL = 7
PATH_MFMA_KSPLIT = 8
PATH_MFMA_KSPLIT_TAIL = 9
PATH_MFMA_SPLITK = 10
PATH_VALU = 11
PATH_MFMA_STRIP = 12
PATH_NAMES = {
    PATH_MFMA_STRIP: "mfma_strip",
    PATH_VALU: "valu",
    PATH_MFMA_SPLITK: "mfma_splitk",
    PATH_MFMA_KSPLIT: "mfma_ksplit",
    PATH_MFMA_KSPLIT_TAIL: "mfma_ksplit_tail",
    PATH_MFMA_DMA_TAIL: "mfma_dma_tail",
    PATH_MFMA_SPLIT: "mfma_split",
    PATH_MFMA_DMA: "mfma_dma",
    PATH_MFMA_VEC: "mfma_vec",
    PATH_MFMA_SCALAR: "mfma_scalar",
    PATH_GEMV_VEC: "gemv_vec",
    PATH_GEMV_SCALAR: "gemv_scalar",
}

TILE_AUTO = 0
TILE_256 = 256
TILE_128 = 128
TILE_64 = 64
TILE_32 = 32
TILE_32X128 = 32128

# Every symbol the header declares.
EXPORTS = (
    "solve",
    "fgr_solve_default",
    "fgr_solve_path",
    "fgr_select_path",
    "fgr_select_tile",
    "fgr_select_parts",
    "fgr_status_string",
    "fgr_version",
    "fgr_variant_count",
    "fgr_variant_name",
    "fgr_solve_variant",
    "fgr_set_workspace_limit",
    "fgr_stream_read",
    "fgr_solve_noalloc",
)


class GemmError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{message} (status {code})")
        self.code = code


_lib = None


def load_library(path: str = LIB_PATH):
    """Load (once) and return the ctypes handle of the HIP library."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is not built; run `python -m fp32_gemm_row_amd.build` "
            "(there is no CPU fallback)"
        )
    lib = ctypes.CDLL(path)
    vp, ci = ctypes.c_void_p, ctypes.c_int
    lib.solve.argtypes = [vp, vp, vp, ci, ci, ci, vp]
    lib.solve.restype = ci
    lib.fgr_solve_default.argtypes = [vp, vp, vp, ci, ci, ci]
    lib.fgr_solve_default.restype = ci
    lib.fgr_solve_path.argtypes = [vp, vp, vp, ci, ci, ci, vp, ci, ci]
    lib.fgr_solve_path.restype = ci
    lib.fgr_select_path.argtypes = [vp, vp, vp, ci, ci, ci]
    lib.fgr_select_path.restype = ci
    lib.fgr_select_tile.argtypes = [vp, vp, vp, ci, ci, ci]
    lib.fgr_select_tile.restype = ci
    lib.fgr_select_parts.argtypes = [vp, vp, vp, ci, ci, ci]
    lib.fgr_select_parts.restype = ci
    lib.fgr_status_string.argtypes = [ci]
    lib.fgr_status_string.restype = ctypes.c_char_p
    lib.fgr_version.argtypes = []
    lib.fgr_version.restype = ci
    lib.fgr_variant_count.argtypes = []
    lib.fgr_variant_count.restype = ci
    lib.fgr_variant_name.argtypes = [ci]
    lib.fgr_variant_name.restype = ctypes.c_char_p
    lib.fgr_solve_variant.argtypes = [vp, vp, vp, ci, ci, ci, vp, ci]
    lib.fgr_solve_variant.restype = ci
    lib.fgr_set_workspace_limit.argtypes = [ctypes.c_longlong]
    lib.fgr_set_workspace_limit.restype = ctypes.c_longlong
    lib.fgr_stream_read.argtypes = [vp, ctypes.c_longlong, vp, ci, vp]
    lib.fgr_stream_read.restype = ci
    lib.fgr_solve_noalloc.argtypes = [vp, vp, vp, ci, ci, ci, vp]
    lib.fgr_solve_noalloc.restype = ci
    _lib = lib
    return lib


def status_string(code: int) -> str:
    return load_library().fgr_status_string(int(code)).decode()


_torch = None


def _torch_module():
    global _torch
    if _torch is None:
        import torch

        _torch = torch
    return _torch


def _address(x, need: int, name: str) -> int:
    """Device address of a float32 GPU tensor (checked) or a raw int address."""
    if isinstance(x, int):
        return x
    torch = _torch_module()
    if not isinstance(x, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor or an int address")
    if x.dtype != torch.float32:
        raise TypeError(f"{name} must be float32, got {x.dtype}")
    if not x.is_cuda:
        raise ValueError(f"{name} must live on the GPU, got {x.device}")
    if not x.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if x.numel() < need:
        raise ValueError(f"{name} has {x.numel()} elements, needs {need}")
    return x.data_ptr()


def _current_stream_handle() -> int:
    """torch's current stream on the current device, as a raw handle. The
    raw accessor costs about 0.1 us per call against 2.8 us for
    torch.cuda.current_stream().cuda_stream (which builds a Stream object);
    the public form serves where the accessor is absent."""
    torch = _torch_module()
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is not None:
        return raw(torch.cuda.current_device())
    return torch.cuda.current_stream().cuda_stream


def _stream_handle(stream) -> int:
    if stream is None:
        return _current_stream_handle()
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(code: int) -> None:
    if code != OK:
        raise GemmError(code, status_string(code))


def _dims(M, N, K):
    M, N, K = int(M), int(N), int(K)
    if M < 1 or N < 1 or K < 1:
        # let the library report it with its own code
        return M, N, K, 0, 0, 0
    return M, N, K, M * N, N * K, M * K


def solve(A, B, C, M: int, N: int, K: int, stream=None) -> None:
    """C[M,K] = A[M,N] x B[N,K] (row-major FP32) on `stream`; asynchronous."""
    lib = load_library()
    M, N, K, na, nb, nc = _dims(M, N, K)
    a = _address(A, na, "A")
    b = _address(B, nb, "B")
    c = _address(C, nc, "C")
    _check(lib.solve(a, b, c, M, N, K, _stream_handle(stream)))


def solve_noalloc(A, B, C, M: int, N: int, K: int, stream=None) -> None:
    """solve() with any workspace taken from the library's static 64 MiB device
    scratch (no allocation); raises GemmError(ERR_SCRATCH) if the plan needs
    more. Calls that overlap on one GPU race on that scratch."""
    lib = load_library()
    M, N, K, na, nb, nc = _dims(M, N, K)
    a = _address(A, na, "A")
    b = _address(B, nb, "B")
    c = _address(C, nc, "C")
    _check(lib.fgr_solve_noalloc(a, b, c, M, N, K, _stream_handle(stream)))


def solve_path(A, B, C, M: int, N: int, K: int, path: int, tile: int = TILE_AUTO, stream=None) -> None:
    """solve() with the kernel path and output tile forced."""
    lib = load_library()
    M, N, K, na, nb, nc = _dims(M, N, K)
    a = _address(A, na, "A")
    b = _address(B, nb, "B")
    c = _address(C, nc, "C")
    _check(lib.fgr_solve_path(a, b, c, M, N, K, _stream_handle(stream), int(path), int(tile)))


def _raw(x) -> int:
    return x if isinstance(x, int) else x.data_ptr()


def select_path(A, B, C, M: int, N: int, K: int) -> int:
    """The FGR path solve() would take on a 256-CU device (host-only; negative = error code)."""
    return int(load_library().fgr_select_path(_raw(A), _raw(B), _raw(C), int(M), int(N), int(K)))


def select_tile(A, B, C, M: int, N: int, K: int) -> int:
    """The output tile solve() would use with that path (host-only; negative = error code)."""
    return int(load_library().fgr_select_tile(_raw(A), _raw(B), _raw(C), int(M), int(N), int(K)))


def select_parts(A, B, C, M: int, N: int, K: int) -> int:
    """Workgroups per tile's reduction on the split path (1 on any other; host-only)."""
    return int(load_library().fgr_select_parts(_raw(A), _raw(B), _raw(C), int(M), int(N), int(K)))


def version() -> int:
    return int(load_library().fgr_version())


def variant_names() -> list:
    """Names of the controlled-comparison kernel variants, in index order."""
    lib = load_library()
    return [lib.fgr_variant_name(i).decode() for i in range(lib.fgr_variant_count())]


def solve_variant(A, B, C, M: int, N: int, K: int, variant: int, stream=None) -> None:
    """solve() with one controlled-comparison kernel variant alone."""
    lib = load_library()
    M, N, K, na, nb, nc = _dims(M, N, K)
    a = _address(A, na, "A")
    b = _address(B, nb, "B")
    c = _address(C, nc, "C")
    _check(lib.fgr_solve_variant(a, b, c, M, N, K, _stream_handle(stream), int(variant)))


def set_workspace_limit(nbytes: int) -> int:
    """Largest workspace one request may take from now on (negative: no
    limit); plans that would need more run their no-workspace form. Returns
    the previous limit."""
    return int(load_library().fgr_set_workspace_limit(int(nbytes)))


def stream_read(X, n: int, out, blocks: int, stream=None) -> None:
    """Measurement hook: read n floats of X once (128-bit loads) on `blocks`
    workgroups, each writing its sum to out[b]; asynchronous."""
    lib = load_library()
    x = _address(X, int(n), "X")
    o = _address(out, int(blocks), "out")
    _check(lib.fgr_stream_read(x, int(n), o, int(blocks), _stream_handle(stream)))
