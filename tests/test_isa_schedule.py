"""The emitted gfx950 code against the proven schedule (no GPU).

tests/test_schedule_and_layout.py proves the K pipeline on an event model
(``program``: per wave, the order of the A-tile DMAs, the B-event loads, the
waits with kpipe.h's counts, and the barriers).  This test ties that model to
the machine code the build produced: it disassembles the device code object
of _build/gemm_a8w8.hip.o and _build/gemm_bf16.hip.o (our own build), walks
every path of each kernel's control-flow graph, and cuts each path at its
s_barrier instructions into windows.  A window is the text between two
barriers, reduced to its vector-memory loads in issue order (D: a
``buffer_load ... lds`` DMA, L: any other buffer load), plus two facts at its
closing barrier:

* ``eff``, the tightest bound the path's s_waitcnt instructions put on the
  wave's outstanding loads there (a wait vmcnt(c) bounds them by c, and every
  load issued after it raises the bound by one; stores only ever make the
  counter larger, so leaving them out is safe, as in kpipe.h);
* whether an lgkmcnt(0) wait follows the window's last LDS read.

For each pair of consecutive windows (a wait covers a DMA issued at most one
window back) the load strings must be a pair the model produces for the
kernel's K case, and ``eff`` must not exceed the model's count for it: then
every wave's code issues its loads exactly as the model orders them and
waits at least as strictly, so the model's proof (RAW: every LDS read follows
a barrier that covers its tile's DMAs in every wave; WAR: every DMA follows a
barrier after which no wave still reads the stage) holds for the code.  The
branches of the graph are taken both ways, so the walk also visits paths no
launch takes; the check holds on those too.  Every model pair must appear in
the code as well, so the check can never pass vacuously.

Loads of the gathered mode's ready flags (global_load) have to be waited for
(vmcnt(0)) before any further load or barrier, which then completes every
load before them.  A loop the compiler builds over the distinct values of an
operand it cannot prove uniform (readfirstlane / exec-mask loops around a
load) fails the audit: every buffer descriptor is uniform by construction.

The mutants at the end edit the disassembly text and must be caught: a DMA
moved across its barrier, a window whose waits are all relaxed to vmcnt(63)
(the pages' bare barrier), a barrier whose lgkmcnt(0) is dropped, a barrier
removed.
"""
import os
import re
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import test_schedule_and_layout as model  # noqa: E402

FUNC = re.compile(r"^([0-9a-f]+) <(\S+)>:\s*$")
INSN = re.compile(r"^\s+([a-z_0-9]+)\b(.*?)//\s*([0-9A-F]+):")
TARGET = re.compile(r"<\S+\+0x([0-9a-f]+)>\s*$")
VMCNT = re.compile(r"vmcnt\((\d+)\)")
LGKMCNT = re.compile(r"lgkmcnt\((\d+)\)")
VMCNT_MAX = 63
MAX_WINDOW = 256  # far more loads than any window of the schedule has


def parse(text):
    """{symbol: [(address, mnemonic, operands, branch target or None)]}"""
    funcs, cur, base = {}, None, 0
    for line in text.splitlines():
        m = FUNC.match(line)
        if m:
            base = int(m.group(1), 16)
            cur = funcs.setdefault(m.group(2), [])
            continue
        if cur is None:
            continue
        m = INSN.match(line)
        if m:
            t = TARGET.search(line)
            cur.append((int(m.group(3), 16), m.group(1), m.group(2).strip(), base + int(t.group(1), 16) if t else None))
    return funcs


def windows(insns):
    """Walk every path of one kernel; returns ({(prev loads or None, loads):
    [(eff, lgkm_ok)]}, [violations])."""
    at = {a: i for i, (a, _, _, _) in enumerate(insns)}
    joins = {at[t] for _, _, _, t in insns if t is not None}  # block starts that branches reach
    out, bad = {}, []
    seen = set()
    stack = [(0, None, "", VMCNT_MAX, True, False)]
    while stack:
        i, prev, loads, eff, lgkm_ok, poll = stack.pop()
        while i < len(insns):
            if i in joins or i == 0:
                # one walk per (block, state): paths that merge with equal
                # state are walked once from here
                key = (i, prev, loads, eff, lgkm_ok, poll)
                if key in seen:
                    break
                seen.add(key)
            addr, mn, ops, tgt = insns[i]
            if mn.startswith("buffer_load"):
                if poll:
                    bad.append(f"{addr:x}: a load follows a flag load that was not waited for")
                loads += "D" if re.search(r"\blds\b", ops) else "L"
                eff = min(eff + 1, VMCNT_MAX)
            elif mn.startswith(("global_load", "flat_load")):
                poll = True
                eff = min(eff + 1, VMCNT_MAX)
            elif mn == "s_waitcnt":
                v, k = VMCNT.search(ops), LGKMCNT.search(ops)
                if v:
                    eff = min(eff, int(v.group(1)))
                    if int(v.group(1)) == 0:
                        poll = False
                if k and int(k.group(1)) == 0:
                    lgkm_ok = True
            elif mn.startswith("ds_read") or mn.startswith("ds_load"):
                lgkm_ok = False
            elif mn == "s_barrier":
                if poll:
                    bad.append(f"{addr:x}: barrier with a flag load outstanding")
                out.setdefault((prev, loads), set()).add((eff, lgkm_ok))
                prev, loads, lgkm_ok = loads, "", True
            if len(loads) > MAX_WINDOW:
                bad.append(f"{addr:x}: more than {MAX_WINDOW} loads without a barrier (a loop of loads)")
                break
            if mn == "s_endpgm":
                break
            if mn == "s_cbranch_execnz" and tgt <= addr and insns[i - 1][1] == "s_xor_b64" \
                    and insns[i - 1][2].startswith("exec, exec"):
                # a loop over the distinct values of a VGPR held in the wave's
                # lanes (s_and_saveexec ... s_xor exec ... back): the compiler
                # could not prove an operand uniform
                bad.append(f"{addr:x}: loop over the lanes' values of a non-uniform operand")
            elif mn == "s_branch":
                stack.append((at[tgt], prev, loads, eff, lgkm_ok, poll))
                break
            elif mn.startswith("s_cbranch"):
                stack.append((at[tgt], prev, loads, eff, lgkm_ok, poll))
            i += 1
    return out, bad


def model_windows(events):
    """The same reduction of a model event list: {(prev, loads): count}."""
    segs, loads, c = [], "", None
    for e in events:
        if e[0] == "load":
            loads += ("L" if e[1] == "B" else "D") * e[3]
        elif e[0] == "wait":
            c = e[1]
        elif e[0] == "barrier":
            segs.append((loads, c))
            loads, c = "", None
    out, prev = {}, None
    for loads, c in segs:
        out[(prev, loads)] = min(out.get((prev, loads), VMCNT_MAX), c)
        prev = loads
    return out


def audit(found, want):
    """Violations of the code's windows against the model's."""
    bad = []
    for key, facts in found.items():
        if key not in want:
            bad.append(f"load order {key} is not one the schedule has")
            continue
        for eff, lgkm_ok in facts:
            if eff > want[key]:
                bad.append(f"{key}: up to {eff} loads outstanding at the barrier, the proof allows {want[key]}")
            if not lgkm_ok:
                bad.append(f"{key}: LDS reads not retired (lgkmcnt(0)) before the barrier")
    for key in want:
        if key not in found:
            bad.append(f"the code never issues {key}")
    return bad


# ------------------------------------------------------------------ inputs
@pytest.fixture(scope="module")
def L():
    return model.compile_shim(tempfile.mkdtemp())


@pytest.fixture(scope="module")
def fp8_text():
    from dense_matmul_amd import build

    return build.disassemble("gemm_a8w8.hip")


@pytest.fixture(scope="module")
def fp8(fp8_text):
    return parse(fp8_text)


@pytest.fixture(scope="module")
def bf16():
    from dense_matmul_amd import build

    return parse(build.disassemble("gemm_bf16.hip"))


def fp8_symbol(mode, case):
    return f"_ZN3dmm16gemm_a8w8_kernelILi{mode}ELi{case}EEEvNS_8GemmArgsE"


def fp8_model(L, mode_name, case, events=None):
    NA, NB, NSC = model.MODES[mode_name]
    want = {}
    for KI in range(1, 41):
        if L.case_of(KI) != case:
            continue
        for ntiles in range(1, 6):
            ev = (events or model.program)(L, KI, ntiles, NA, NB, NSC)
            for k, c in model_windows(ev).items():
                want[k] = min(want.get(k, VMCNT_MAX), c)
    return want


CASES = [0, 1, 2, 3, 4]


# ------------------------------------------------------------------- tests
@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("mode_name", sorted(model.MODE_IDS))
def test_fp8_kernel_code_follows_the_proven_schedule(L, fp8, mode_name, case):
    sym = fp8_symbol(model.MODE_IDS[mode_name], case)
    assert sym in fp8, f"{sym} not in the code object"
    found, bad = windows(fp8[sym])
    bad += audit(found, fp8_model(L, mode_name, case))
    assert not bad, f"{mode_name} case {case}: {bad[:4]}"


@pytest.mark.parametrize("tile", sorted(model.BF16_RINGS))
def test_bf16_kernel_code_follows_the_proven_ring(L, bf16, tile):
    NS, NL = model.BF16_RINGS[tile]
    bm = tile.split("x")[0]
    sym = next(s for s in bf16 if re.search(rf"gemm_bf16_kernelILi{bm}ELi{bm}E", s))
    want = {}
    for KT in range(1, 40):
        for k, c in model_windows(model.program_bf16(L, KT, NS, NL)).items():
            want[k] = min(want.get(k, VMCNT_MAX), c)
    found, bad = windows(bf16[sym])
    bad += audit(found, want)
    assert not bad, f"bf16 {tile}: {bad[:4]}"


# ----------------------------------------------------------------- mutants
def mutate(text, sym, edit):
    """Apply edit(lines of the kernel's body) -> lines, return parsed insns."""
    lines = text.splitlines()
    start = next(i for i, l in enumerate(lines) if l.endswith(f"<{sym}>:"))
    end = next((i for i in range(start + 1, len(lines)) if FUNC.match(lines[i])), len(lines))
    body = edit(lines[start + 1:end])
    return parse("\n".join([lines[start]] + body))[sym]


def barrier_lines(body):
    return [i for i, l in enumerate(body) if "\ts_barrier" in l or " s_barrier " in l]


MUTANT_KERNEL = ("ptpc", 2)


def _check(L, insns):
    found, bad = windows(insns)
    return bad + audit(found, fp8_model(L, *MUTANT_KERNEL))


def test_unmutated_kernel_passes(L, fp8_text):
    sym = fp8_symbol(model.MODE_IDS[MUTANT_KERNEL[0]], MUTANT_KERNEL[1])
    assert _check(L, mutate(fp8_text, sym, lambda b: b)) == []


def test_audit_catches_a_dma_moved_before_its_barrier(L, fp8_text):
    sym = fp8_symbol(model.MODE_IDS[MUTANT_KERNEL[0]], MUTANT_KERNEL[1])

    def edit(body):
        b = barrier_lines(body)[3]
        d = next(i for i in range(b + 1, len(body)) if "buffer_load" in body[i] and " lds" in body[i])
        return body[:b] + [body[d]] + body[b:d] + body[d + 1:]

    assert _check(L, mutate(fp8_text, sym, edit))


def test_audit_catches_a_bare_barrier(L, fp8_text):
    """Every vmcnt in the window before one barrier relaxed to 63."""
    sym = fp8_symbol(model.MODE_IDS[MUTANT_KERNEL[0]], MUTANT_KERNEL[1])

    def edit(body):
        bl = barrier_lines(body)
        lo, hi = bl[3], bl[4]
        return body[:lo] + [VMCNT.sub("vmcnt(63)", l) for l in body[lo:hi]] + body[hi:]

    assert _check(L, mutate(fp8_text, sym, edit))


def test_audit_catches_unretired_lds_reads(L, fp8_text):
    sym = fp8_symbol(model.MODE_IDS[MUTANT_KERNEL[0]], MUTANT_KERNEL[1])

    def edit(body):
        bl = barrier_lines(body)
        lo, hi = bl[3], bl[4]
        return body[:lo] + [LGKMCNT.sub("lgkmcnt(1)", l) for l in body[lo:hi]] + body[hi:]

    assert _check(L, mutate(fp8_text, sym, edit))


def test_audit_catches_a_missing_barrier(L, fp8_text):
    sym = fp8_symbol(model.MODE_IDS[MUTANT_KERNEL[0]], MUTANT_KERNEL[1])

    def edit(body):
        b = barrier_lines(body)[4]
        return body[:b] + body[b + 1:]

    assert _check(L, mutate(fp8_text, sym, edit))


def test_audit_catches_a_model_count_below_the_code(L, fp8_text):
    """A schedule that claims stricter waits than the code has: every count
    of the model one load lower."""
    sym = fp8_symbol(model.MODE_IDS[MUTANT_KERNEL[0]], MUTANT_KERNEL[1])
    NA, NB, NSC = model.MODES[MUTANT_KERNEL[0]]

    def events(L_, KI, ntiles, *_):
        return model.program(L_, KI, ntiles, NA, NB, NSC,
                             wait_fn=lambda s, k: L_.wait_at(s, k, KI, NA, NB, NSC) - 8)

    found, bad = windows(mutate(fp8_text, sym, lambda b: b))
    assert audit(found, fp8_model(L, MUTANT_KERNEL[0], MUTANT_KERNEL[1], events=events))


def test_audit_catches_a_loop_over_lane_values():
    """The compiler's loop over the distinct values of a VGPR operand
    (readfirstlane, s_and_saveexec, the load, s_xor exec, back) is rejected."""
    insns = [(0x0, "s_mov_b64", "s[2:3], exec", None),
             (0x4, "v_readfirstlane_b32", "s4, v10", None),
             (0x8, "s_and_saveexec_b64", "s[0:1], s[0:1]", None),
             (0xc, "buffer_load_dwordx4", "v3, s[4:7], 0 offen lds", None),
             (0x14, "s_xor_b64", "exec, exec, s[0:1]", None),
             (0x18, "s_cbranch_execnz", "65530", 0x4),
             (0x1c, "s_endpgm", "", None)]
    _, bad = windows(insns)
    assert any("non-uniform" in b for b in bad)
