"""Build tests/shim/liblayout_shim.so (test infrastructure only) with hipcc for
gfx950, from layout_shim.hip and the library's kernel headers."""

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "layout_shim.hip")
LIB = os.path.join(HERE, "liblayout_shim.so")
CSRC = os.path.join(ROOT, "fp32_gemm_row_amd", "csrc")


def build(force: bool = False) -> str:
    deps = [SRC] + [os.path.join(CSRC, n) for n in os.listdir(CSRC) if n.endswith(".hpp")]
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= max(os.path.getmtime(d) for d in deps):
        return LIB
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [os.environ.get("HIPCC", "/opt/rocm/bin/hipcc"), "--offload-arch=gfx950", "-O2", "-std=c++17", "-fPIC",
           "-shared", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", f"-I{CSRC}",
           f"-I{os.path.join(ROOT, 'include')}", SRC, "-o", tmp]
    subprocess.run(cmd, check=True, capture_output=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(force=True))
