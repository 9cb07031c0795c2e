"""Matrix-op result hazards in the emitted gfx950 code (no GPU).

The fp8 GEMM writes its matrix ops as inline asm, so the compiler cannot see
that a later instruction reads (or overwrites) a register a matrix op is
still writing.  CDNA3/CDNA4 require a number of wait states between a matrix
op and any non-matrix instruction that touches its destination registers:
passes + 3 (the 16x16x128 fp8 op, 8 passes: 11; the 16x16x32 bf16 op, 4
passes: 7), and the hardware does not check it.  The kernels pay for it
with s_nop padding placed by hand.

This test disassembles our own build (_build/*.o), and from every matrix op
walks every control-flow path forward, counting wait states the way the
hazard rules do (one per instruction issued, n + 1 for s_nop n), until the
required number is reached.  Any other instruction on the way that names one
of the op's destination registers (VGPR or AGPR) is a violation.  Matrix ops
that accumulate into the same registers are the hardware's own dependency
and are left out.  The mutant at the end removes the padding from the
disassembly text and must be caught.
"""
import os
import re
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import test_isa_schedule as isa  # noqa: E402

# wait states a non-matrix instruction must keep from each matrix op that
# writes a register it names (passes + 3); an op not listed fails the test,
# so a new matrix instruction has to be classified before it is audited
REQUIRED = {
    "v_mfma_f32_16x16x128_f8f6f4": 11,
    "v_mfma_scale_f32_16x16x128_f8f6f4": 11,
    "v_mfma_f32_16x16x32_bf16": 7,
}
REG = re.compile(r"(?<![\w.])([va])(?:\[(\d+):(\d+)\]|(\d+))(?![\w\]])")
NOP = re.compile(r"^\s*(0x[0-9a-f]+|\d+)")


def regs(text):
    out = set()
    for m in REG.finditer(text):
        lo, hi = (int(m.group(2)), int(m.group(3))) if m.group(2) else (int(m.group(4)), int(m.group(4)))
        out |= {(m.group(1), r) for r in range(lo, hi + 1)}
    return out


def wait_states(mn, ops):
    if mn == "s_nop":
        return int(NOP.match(ops).group(1), 0) + 1
    return 1


def audit(insns):
    """(matrix ops audited, [violations]) for one kernel."""
    at = {a: i for i, (a, _, _, _) in enumerate(insns)}
    bad, n = [], 0
    for i, (addr, mn, ops, _) in enumerate(insns):
        if not mn.startswith("v_mfma"):
            continue
        assert mn in REQUIRED, f"matrix instruction {mn} has no hazard count"
        need = REQUIRED[mn]
        dst = regs(ops.split(",")[0])
        assert dst, f"{addr:x}: no destination registers in {ops!r}"
        n += 1
        # (index, wait states since the op) on every path until `need`
        stack, seen = [(i + 1, 0)], set()
        while stack:
            j, ws = stack.pop()
            while j < len(insns) and ws < need:
                if (j, ws) in seen:
                    break
                seen.add((j, ws))
                a2, mn2, ops2, tgt = insns[j]
                if not mn2.startswith("v_mfma") and regs(ops2) & dst:
                    bad.append(f"{addr:x} {mn} -> {a2:x} {mn2} {ops2} after {ws} of {need} wait states")
                    break
                ws += wait_states(mn2, ops2)
                if mn2 == "s_endpgm":
                    break
                if mn2 == "s_branch":
                    stack.append((at[tgt], ws))
                    break
                if mn2.startswith("s_cbranch"):
                    stack.append((at[tgt], ws))
                j += 1
    return n, bad


@pytest.fixture(scope="module")
def kernels():
    from dense_matmul_amd import build

    funcs = {}
    for src in ("gemm_a8w8.hip", "gemm_bf16.hip"):
        text = build.disassemble(src)
        funcs.update({s: v for s, v in isa.parse(text).items() if "gemm" in s and "kernel" in s})
    assert funcs
    return funcs


def test_register_parser():
    assert regs("v[12:15], v20, a[0:3], s[4:7], vcc, off offset:16") == (
        {("v", r) for r in range(12, 16)} | {("v", 20)} | {("a", r) for r in range(4)})
    assert regs("v5, v100, v6 row_newbcast:1") == {("v", 5), ("v", 100), ("v", 6)}
    assert wait_states("s_nop", "7") == 8 and wait_states("s_nop", "0x3") == 4
    assert wait_states("v_fmac_f32_e32", "v1, v2, v3") == 1


def test_every_matrix_op_result_is_left_alone_long_enough(kernels):
    total = 0
    for sym, insns in sorted(kernels.items()):
        n, bad = audit(insns)
        assert not bad, f"{sym}: " + "; ".join(bad[:5])
        total += n
    assert total > 1000, "the audit saw the kernels' matrix ops"


def test_audit_catches_missing_padding(kernels):
    # drop every s_nop from one blockscale kernel: the fold reads its
    # products too soon
    sym = isa.fp8_symbol(1, 0)
    stripped = [x for x in kernels[sym] if x[1] != "s_nop"]
    _, bad = audit(stripped)
    assert bad
