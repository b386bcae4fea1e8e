"""Wait states after inline-asm writes, checked in the gfx950 assembly of the library.

The compiler inserts the wait states an MFMA needs after a vector-ALU write of
one of its source registers (two on gfx950; it places an `s_nop 1` after its
own moves), but it does not know what an inline-asm block writes, so it may
leave fewer after one. A move written in asm must therefore carry its own wait
states. This test compiles the library's kernels to assembly (hipcc -S, no GPU
needed) and checks, instruction by instruction, that no MFMA reads a register
written inside an asm block fewer than two wait states later: each instruction
counts one, `s_nop n` counts n + 1. State is dropped at labels and branches,
so only straight-line code is judged; the asm moves and the MFMAs that read
them sit in the same block.
"""
import os
import re
import shutil
import subprocess

import pytest

from fp32_gemm_row_amd import build as fbuild

NEEDED = 2  # wait states between a VALU write and an MFMA read of that register

_VREG = re.compile(r"\bv(\d+)\b|\bv\[(\d+):(\d+)\]")


def _regs(operand):
    """VGPR numbers named by one operand (v7 or v[4:7])."""
    out = set()
    for m in _VREG.finditer(operand):
        if m.group(1) is not None:
            out.add(int(m.group(1)))
        else:
            out.update(range(int(m.group(2)), int(m.group(3)) + 1))
    return out


def _operands(line):
    parts = line.split(None, 1)
    if len(parts) < 2:
        return parts[0], []
    return parts[0], [p.strip() for p in parts[1].split(",")]


def violations(asm_text):
    """(function, line) of every MFMA reading an asm-written VGPR too early."""
    found = []
    func = None
    in_asm = False
    pending = {}  # VGPR -> wait states since its asm write
    for raw in asm_text.splitlines():
        line = raw.split(";", 1)[0].strip() if not raw.strip().startswith(";;#ASM") else raw.strip()
        if raw.startswith("_Z") and ":" in raw:  # a kernel's entry label
            func = raw.split(":", 1)[0]
            pending.clear()
            continue
        if line == ";;#ASMSTART":
            in_asm = True
            continue
        if line == ";;#ASMEND":
            in_asm = False
            continue
        if line.endswith(":"):  # a label: another path may enter here
            pending.clear()
            continue
        if not line or line.startswith("."):  # directives
            continue
        op, ops = _operands(line)
        if in_asm:
            if op == "s_nop":
                n = int(ops[0], 0) + 1
                for r in pending:
                    pending[r] += n
            else:
                for r in pending:
                    pending[r] += 1
                if op.startswith("v_") and ops:
                    for r in _regs(ops[0]):
                        pending[r] = 0
            continue
        if op.startswith("v_mfma") and len(ops) >= 3:
            srcs = _regs(ops[1]) | _regs(ops[2]) | (_regs(ops[3]) if len(ops) > 3 else set())
            for r in srcs:
                if r in pending and pending[r] < NEEDED:
                    found.append((func, raw.strip(), r, pending[r]))
        if op.startswith("s_branch") or op.startswith("s_cbranch") or op == "s_setpc_b64":
            pending.clear()
            continue
        n = int(ops[0], 0) + 1 if op == "s_nop" else 1
        for r in list(pending):
            pending[r] += n
            if pending[r] >= NEEDED:
                del pending[r]
        # a later write of the register by ordinary code ends the asm's hazard
        if op.startswith("v_") and not op.startswith("v_mfma") and ops:
            for r in _regs(ops[0]):
                pending.pop(r, None)
    return found


def test_checker_flags_a_short_gap():
    text = "\n".join([
        "_Zk:",
        "\t;;#ASMSTART",
        "\tv_mov_b32 v1, v38",
        "\t;;#ASMEND",
        "\ts_nop 0",
        "\tv_mfma_f32_32x32x2_f32 a[0:15], v14, v1, a[0:15]",
        "\t;;#ASMSTART",
        "\tv_mov_b32 v2, v39",
        "\ts_nop 1",
        "\t;;#ASMEND",
        "\tv_mfma_f32_32x32x2_f32 a[16:31], v2, v3, a[16:31]",
    ])
    bad = violations(text)
    assert [(b[2], b[3]) for b in bad] == [(1, 1)]


@pytest.mark.skipif(shutil.which(fbuild.HIPCC) is None and not os.path.exists(fbuild.HIPCC),
                    reason="hipcc is not installed")
def test_no_mfma_reads_an_asm_write_too_early(tmp_path):
    out = tmp_path / "solve.s"
    flags = [f for f in fbuild.FLAGS if f not in ("-shared", "-fPIC")]
    cmd = [fbuild.HIPCC, *flags, "--cuda-device-only", "-S", f"-I{fbuild.INCLUDE}", f"-I{fbuild.CSRC}",
           *fbuild.SOURCES, "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    text = out.read_text()
    assert ";;#ASMSTART" in text, "the kernels hold inline asm; the check would be vacuous without it"
    bad = violations(text)
    assert not bad, f"{len(bad)} MFMA reads of asm-written registers within {NEEDED} wait states: {bad[:5]}"
