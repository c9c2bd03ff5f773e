"""Static check of the compiled gfx950 code (CPU: hipcc cross-compiles).

A v_mfma_f32_16x16x16_bf16 that accumulates onto the result of a
v_mfma_f32_16x16x32_bf16 issued less than 8 wait states before it reads a
stale accumulator (measured on MI355X: values of order 1e35 back to back,
exact from 8 wait states on), and this compiler issues such pairs back to
back.  The kernels therefore never chain products of different opcodes
through one accumulator; this test compiles representative instances of the
per-row decay forward and the backward to assembly and
checks that no product reads an accumulator that a product of another
opcode wrote within the previous 16 instructions.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "kernelized_attention_scan_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
WINDOW = 16

ROWS_TU = """#include "la_forward_rows.h"
namespace la {
template __global__ void la_fwd_rows_kernel<bf16, 128, 128, 0, false>(RowArgs);
template __global__ void la_fwd_rows_kernel<bf16, 128, 128, 0, true>(RowArgs);
template __global__ void la_fwd_rows_kernel<bf16, 64, 256, 0, false>(RowArgs);
template __global__ void la_fwd_rows_kernel<bf16, 16, 32, 0, true>(RowArgs);
template __global__ void la_fwd_rows_kernel<bf16, 128, 128, 1, false>(RowArgs);
template __global__ void la_fwd_rows_kernel<bf16, 128, 256, 2, false>(RowArgs);
}
"""


def _regs(tok):
    m = re.match(r"([va])\[(\d+):(\d+)\]", tok)
    if m:
        return {(m.group(1), r) for r in range(int(m.group(2)),
                                               int(m.group(3)) + 1)}
    m = re.match(r"([va])(\d+)$", tok)
    return {(m.group(1), int(m.group(2)))} if m else set()


def mixed_chains(asm: str, window: int = WINDOW):
    """(writer, reader) pairs of products with different opcodes where the
    reader's accumulator input overlaps the writer's result."""
    insts = [s.strip() for s in asm.splitlines()]
    insts = [s for s in insts if s and not s.startswith((";", "."))]
    found = []
    for i, s in enumerate(insts):
        if not s.startswith("v_mfma"):
            continue
        ops = [t.strip() for t in s.split(None, 1)[1].split(",")]
        srcc = _regs(ops[3])
        for p in insts[max(0, i - window):i]:
            if p.startswith("v_mfma") and p.split()[0] != s.split()[0]:
                if _regs(p.split(None, 1)[1].split(",")[0].strip()) & srcc:
                    found.append((p, s))
    return found


def test_checker_finds_a_mixed_chain():
    asm = """
    v_mfma_f32_16x16x32_bf16 a[0:3], v[10:13], v[14:17], a[0:3]
    s_waitcnt lgkmcnt(0)
    v_mfma_f32_16x16x16_bf16 a[0:3], v[20:21], v[22:23], a[0:3]
    v_mfma_f32_16x16x32_bf16 a[4:7], v[10:13], v[14:17], 0
    v_mfma_f32_16x16x32_bf16 a[4:7], v[10:13], v[14:17], a[4:7]
    """
    assert len(mixed_chains(asm)) == 1


def _asm(tmp_path, name, text=None, src=None):
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    if text is not None:
        src = tmp_path / f"{name}.hip"
        src.write_text(text)
    out = tmp_path / f"{name}.s"
    cmd = [HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "-Xclang",
           "-target-feature", "-Xclang", "-packed-fp32-ops", "-I",
           os.path.join(ROOT, "include"), "-I", CSRC, "-S",
           "--cuda-device-only", str(src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return out.read_text()


def test_row_decay_forward_has_no_mixed_chains(tmp_path):
    asm = _asm(tmp_path, "rows", text=ROWS_TU)
    assert "v_mfma_f32_16x16x16_bf16" in asm  # the K = 16 carry is there
    assert mixed_chains(asm) == []


def test_backward_has_no_mixed_chains(tmp_path):
    asm = _asm(tmp_path, "bwd", src=os.path.join(CSRC, "la_backward.hip"))
    assert mixed_chains(asm) == []
