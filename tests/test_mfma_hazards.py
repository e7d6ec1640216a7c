"""The attention kernel issues its MFMAs from inline assembly, where the compiler does not insert
hazard wait states. A VALU instruction that writes a register an MFMA then reads needs two wait
states between them (a nop or any two instructions). The chained S^T steps carry no pad of their
own: their operands come from LDS loads, from the Q registers written once at the start, and
from the accumulator of the previous MFMA. This test compiles the kernel source to gfx950
assembly, exactly as the library build does, and checks every MFMA in it: no VALU write of one
of its source registers may sit within two wait states before it, and an MFMA with no pad must
not directly follow a label (a branch target whose predecessors the scan cannot see).

No GPU is needed: hipcc cross-compiles.
"""

import os
import re
import subprocess
import tempfile

from mla_sparse_top_amd import build as B

KERNEL = os.path.join(B.CSRC, "sfa_kernels.hip")


def _device_asm() -> str:
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "k.s")
        cmd = [B.hipcc_path(), "--offload-arch=gfx950", "--offload-device-only", "-S", "-O3", "-std=c++17",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument",
               "-I", B.INCLUDE, "-I", B.CSRC, KERNEL, "-o", out]
        proc = subprocess.run(cmd, capture_output=True, text=True)
        assert proc.returncode == 0, proc.stderr[-2000:]
        return open(out).read()


_REG = re.compile(r"\b([va])(?:\[(\d+):(\d+)\]|(\d+)(?!\d))")


def _regs(operand: str) -> set:
    out = set()
    for m in _REG.finditer(operand):
        kind = m.group(1)
        if m.group(4) is not None:
            out.add((kind, int(m.group(4))))
        else:
            out.update((kind, r) for r in range(int(m.group(2)), int(m.group(3)) + 1))
    return out


def _operands(line: str) -> list:
    body = line.split(None, 1)[1] if len(line.split(None, 1)) > 1 else ""
    return [o.strip() for o in body.split(",")]


def _valu_dst(line: str) -> set:
    op = line.split()[0]
    if not op.startswith("v_") or op.startswith("v_mfma") or op.startswith("v_cmp") or op.startswith("v_readfirstlane") \
            or op.startswith("v_readlane"):
        return set()
    ops = _operands(line)
    return _regs(ops[0]) if ops else set()


def _nop_states(line: str) -> int:
    m = re.match(r"s_nop\s+(\d+)", line)
    return int(m.group(1)) + 1 if m else 0


def _scan(asm: str):
    lines = [l.split(";")[0].strip() for l in asm.split("\n")]
    lines = [l for l in lines if l and not l.startswith(".") or re.match(r"^\.LBB\d+_\d+:", l or "")]
    problems, n_mfma = [], 0
    for i, line in enumerate(lines):
        if not line.startswith("v_mfma"):
            continue
        n_mfma += 1
        ops = _operands(line)
        srcs = set().union(*(_regs(o) for o in ops[1:]))
        ws, j = 0, i - 1
        while ws < 2 and j >= 0:
            prev = lines[j]
            if re.match(r"^\.LBB\d+_\d+:", prev) or prev.endswith(":"):
                problems.append(f"MFMA {i} reached a label with {ws} wait states: {line}")
                break
            hit = _valu_dst(prev) & srcs
            if hit:
                problems.append(f"MFMA {i} reads {sorted(hit)} written {ws} wait states before by: {prev}")
                break
            ws += _nop_states(prev) or 1
            j -= 1
    return problems, n_mfma


def test_unpadded_mfma_operands_are_not_fresh_valu_results():
    problems, n_mfma = _scan(_device_asm())
    assert n_mfma > 100, "expected the attention kernels' MFMAs in the assembly"
    assert not problems, "\n".join(problems[:20])


def test_scanner_flags_a_planted_hazard():
    asm = "\n".join([
        "_kernel:",
        "  s_nop 7",
        "  v_mov_b32 v12, v3",
        "  v_mfma_f32_32x32x16_bf16 v[0:15], v[12:15], a[0:3], v[0:15]",
        "  s_nop 2",
        "  v_mfma_f32_32x32x16_bf16 v[0:15], v[12:15], a[0:3], v[0:15]",
        "  v_add_f32 v40, v41, v42",
        "  v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], a[0:3], v[0:15]",
        "  v_accvgpr_write_b32 a1, v5",
        "  s_nop 0",
        "  v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], a[0:3], v[0:15]",
    ])
    problems, n = _scan(asm)
    assert n == 4
    assert len(problems) == 2, problems
    assert "v12" in problems[0] or "('v', 12)" in problems[0]
    assert "('a', 1)" in problems[1]
