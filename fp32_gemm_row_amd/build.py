"""Build the HIP library libfp32_gemm_row.so in-tree with hipcc for gfx950.

    python -m fp32_gemm_row_amd.build [--resource-usage] [--resource-report FILE] [--timestamps]

--timestamps builds the measurement library libfp32_gemm_row_ts.so instead
(FGR_TIMESTAMPS: per-workgroup timestamp records, bench.py --timestamps).

--resource-report writes a markdown table of every kernel's registers, LDS,
occupancy and spills, as the compiler reports them (-Rpass-analysis=
kernel-resource-usage) - the counterpart of the ptxas table of the LeetGPU
write-up's "Controlled Comparison".

The library is a plain C-ABI shared object (include/fp32_gemm_row.h); the
Python binding loads it with ctypes. Packed-FP32 VALU instructions are
disabled for the device code (-packed-fp32-ops off).
"""

from __future__ import annotations

import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libfp32_gemm_row.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
# the measurement build: the same library with per-workgroup timestamps
# (FGR_TIMESTAMPS, csrc/timestamps.hpp, include/fp32_gemm_row_timestamps.h)
TS_LIB_PATH = os.path.join(PKG, "libfp32_gemm_row_ts.so")
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


def resource_table(remarks: str) -> str:
    """Markdown table of the compiler's per-kernel resource remarks."""
    rows, cur = [], None
    for line in remarks.splitlines():
        m = re.search(r"remark:\s+(.*?)\s*\[-Rpass-analysis", line)
        if not m:
            continue
        text = m.group(1)
        if text.startswith("Function Name:"):
            cur = {"name": text.split(":", 1)[1].strip()}
            rows.append(cur)
        elif cur is not None and ":" in text:
            key, val = text.split(":", 1)
            cur[key.strip()] = val.strip()
    demangled = {}
    try:
        out = subprocess.run(["c++filt"], input="\n".join(r["name"] for r in rows),
                             capture_output=True, text=True, check=True).stdout.splitlines()
        demangled = dict(zip((r["name"] for r in rows), out))
    except (OSError, subprocess.CalledProcessError):
        pass
    cols = ["VGPRs", "AGPRs", "Occupancy [waves/SIMD]", "LDS Size [bytes/block]", "VGPRs Spill",
            "ScratchSize [bytes/lane]"]
    lines = ["| kernel | " + " | ".join(cols) + " |", "|---" * (len(cols) + 1) + "|"]
    for r in rows:
        name = demangled.get(r["name"], r["name"]).split("(")[0]
        lines.append(f"| `{name}` | " + " | ".join(r.get(c, "") for c in cols) + " |")
    return "\n".join(lines) + "\n"


def build(resource_usage: bool = False, verbose: bool = False, report: str = "", timestamps: bool = False) -> str:
    """Compile every source into LIB_PATH, or with timestamps into
    TS_LIB_PATH (always recompiles)."""
    out = TS_LIB_PATH if timestamps else LIB_PATH
    tmp = out + f".tmp{os.getpid()}"
    cmd = [HIPCC, *FLAGS, *(["-DFGR_TIMESTAMPS"] if timestamps else []), f"-I{INCLUDE}", f"-I{CSRC}", *SOURCES,
           "-o", tmp]
    if resource_usage or report:
        cmd.insert(1, "-Rpass-analysis=kernel-resource-usage")
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    if resource_usage:
        sys.stderr.write(res.stderr)
    if report:
        with open(report, "w", encoding="utf-8") as fh:
            fh.write("# Kernel resources (hipcc -Rpass-analysis=kernel-resource-usage, gfx950)\n\n")
            fh.write("Command: `python -m fp32_gemm_row_amd.build --resource-report " + os.path.relpath(report, ROOT)
                     + "`\n\n")
            fh.write(resource_table(res.stderr))
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    rep = ""
    if "--resource-report" in sys.argv:
        rep = os.path.abspath(sys.argv[sys.argv.index("--resource-report") + 1])
    print(build(resource_usage="--resource-usage" in sys.argv, verbose=True, report=rep,
                timestamps="--timestamps" in sys.argv))
