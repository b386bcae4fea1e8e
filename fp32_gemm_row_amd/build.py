"""Build the HIP library libfp32_gemm_row.so in-tree with hipcc for gfx950.

    python -m fp32_gemm_row_amd.build [--resource-usage]

The library is a plain C-ABI shared object (include/fp32_gemm_row.h); the
Python binding loads it with ctypes. Packed-FP32 VALU instructions are
disabled for the device code (-packed-fp32-ops off).
"""

from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libfp32_gemm_row.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
SOURCES = [os.path.join(CSRC, "solve.hip")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def build(resource_usage: bool = False, verbose: bool = False) -> str:
    """Compile every source into LIB_PATH (always recompiles)."""
    tmp = LIB_PATH + f".tmp{os.getpid()}"
    cmd = [HIPCC, *FLAGS, f"-I{INCLUDE}", f"-I{CSRC}", *SOURCES, "-o", tmp]
    if resource_usage:
        cmd.insert(1, "-Rpass-analysis=kernel-resource-usage")
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    if resource_usage:
        sys.stderr.write(res.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    build(resource_usage="--resource-usage" in sys.argv, verbose=True)
    print(LIB_PATH)
