"""CPU proofs for the fp8 GEMM's pipeline (no GPU).

The kernel takes every wait count from ``kpipe.h`` and every LDS address from
``lds_layout.h``; this test compiles those two headers into a host shim with
g++ and checks, exhaustively over the shapes that matter:

* the schedule: for every K-tile count KI in 1..40 and 1..5 output tiles per
  workgroup, each LDS read of stream K tile j happens after a wait + barrier
  that covers the DMA of tile j in every wave (RAW), each DMA into a stage
  happens after a barrier that every wave passed only after its reads of the
  stage's previous tile retired (WAR), and every count is exactly the number
  of loads issued after the covered DMA (the loosest safe value, capped at
  the 6-bit field).  This is the property the pages' tail fix restores
  (mori PR 785, sections Problem and Fix): no LDS read of a K tile -- in the
  main loop, the peeled tail, or a K = 256 tile with no main loop at all --
  can run ahead of that tile's producers.
* the layout: the DMA lanes together write every (row, chunk) of a stage
  exactly once, each fragment read finds the (row, chunk) it needs, and each
  16-lane read phase touches 16 distinct 16-byte bank groups (64 banks).
The mutants at the end show the checker has teeth.
"""
import ctypes
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "dense_matmul_amd", "csrc")

SHIM = r"""
#include "b_layout.h"
#include "kpipe.h"
#include "lds_layout.h"
using namespace dmm;
extern "C" {
int prologue_wait(int NA) { return sched::prologue_wait(NA); }
int wait_at(int s, int k, int KI, int NA, int NB, int NSC) { return sched::wait_at(s, k, KI, NA, NB, NSC); }
int stage_of(int j) { return sched::stage_of(j); }
int refill_stage(int s) { return sched::refill_stage(s); }
int dma_ahead_tile(int k, int KI) { return sched::dma_ahead_tile(k, KI); }
int dma_ahead_kt(int k, int KI) { return sched::dma_ahead_kt(k, KI); }
int case_of(int KI) { return sched::case_of(KI); }
int phase_advance(int CASE) { return sched::phase_advance(CASE); }
int dma_lds_byte(int b, int l) { return lds::dma_lds_byte(b, l); }
int dma_row(int b, int l, int MB) { return lds::dma_row(b, l, MB); }
int dma_chunk(int b, int l, int MB) { return lds::dma_chunk(b, l, MB); }
int frag_byte(int i, int g, int mb, int half, int MB) { return lds::frag_byte(i, g, mb, half, MB); }
int bf16_chunk_pos(int r, int c) { return lds::bf16_chunk_pos(r, c); }
int bf16_prologue_wait(int NS, int NL) { return sched::bf16_prologue_wait(NS, NL); }
int bf16_mid_wait(int NS, int NL) { return sched::bf16_mid_wait(NS, NL); }
int frag_col(int nb, int r, int p) { return bl::frag_col(nb, r, p); }
int group_blocks(int G, int nblocks) { return bl::group_blocks(G, nblocks); }
int shape_field(int mode, int f) {
    const sched::Shape sh = sched::shape_of(mode);
    const int v[6] = {sh.MB, sh.NBW, sh.WAVES, sh.NA, sh.NB, sh.NSC};
    return v[f];
}
}
"""


SHIM_FUNCS = ("prologue_wait", "wait_at", "stage_of", "refill_stage", "dma_lds_byte", "dma_row", "dma_chunk",
              "frag_byte", "dma_ahead_tile", "dma_ahead_kt", "case_of", "phase_advance", "bf16_chunk_pos",
              "shape_field", "bf16_prologue_wait", "bf16_mid_wait", "frag_col", "group_blocks")


def compile_shim(d):
    """The host shim over kpipe.h, lds_layout.h and b_layout.h, built with
    g++ into directory d."""
    src = os.path.join(str(d), "shim.cpp")
    with open(src, "w") as f:
        f.write(SHIM)
    lib = os.path.join(str(d), "libshim.so")
    subprocess.run(["g++", "-std=c++17", "-O1", "-shared", "-fPIC", "-I", CSRC, src, "-o", lib], check=True)
    L = ctypes.CDLL(lib)
    for f in SHIM_FUNCS:
        getattr(L, f).restype = ctypes.c_int
    return L


@pytest.fixture(scope="module")
def shim(tmp_path_factory):
    return compile_shim(tmp_path_factory.mktemp("shim"))


# ---------------------------------------------------------------- schedule
# the kernel's modes (kpipe.h, shape_of): name -> mode id
MODE_IDS = {"ptpc": 0, "blockscale": 1, "mxfp8": 2, "ptpc_128x256": 3, "ptpc_gathered": 4, "mxfp8_256x128": 5,
            "blockscale_128x128": 6, "ptpc_128x128": 7}


def _shapes():
    """NA, NB, NSC per wave for every mode, read from kpipe.h through the
    shim (the numbers the kernel's waits are built from)."""
    import tempfile

    L = compile_shim(tempfile.mkdtemp())
    return {name: tuple(L.shape_field(mid, f) for f in (3, 4, 5)) for name, mid in MODE_IDS.items()}


MODES = _shapes()  # NA, NB, NSC per wave


def test_mode_shapes_are_the_documented_loads():
    """The counts the proof runs on, as kpipe.h states them: per K tile NA
    = 2 MB / waves A DMAs and NB = 2 NBW B fragment halves (+ 3 scale loads
    for mxfp8 and blockscale); the ptpc tiles add 2 epilogue-scale DMAs."""
    assert MODES == {"ptpc": (8, 8, 2), "blockscale": (2, 7, 0), "mxfp8": (8, 11, 0), "ptpc_128x256": (2, 4, 2),
                     "ptpc_gathered": (8, 8, 2), "mxfp8_256x128": (8, 7, 0), "blockscale_128x128": (4, 7, 0),
                     "ptpc_128x128": (4, 4, 2)}


def program(L, KI, ntiles, NA, NB, NSC, wait_fn=None):
    """One wave's event list for a workgroup stream, as the kernel issues it:
    ("load", kind, index, n), ("store", n), ("wait", c), ("barrier",),
    ("read", stream tile), ("read_done",) -- the same for every wave."""
    wait_fn = wait_fn or (lambda s, k: L.wait_at(s, k, KI, NA, NB, NSC))
    S = KI * ntiles
    ev = [("load", "B", 0, NB)]
    if KI > 1 and NSC:
        ev.append(("load", "E", 0, NSC))  # tile 0's epilogue scales
    ev += [("load", "A", 0, NA), ("load", "A", 1, NA), ("load", "A", 2, NA),
           ("wait", L.prologue_wait(NA)), ("barrier",), ("read", 0)]
    for s in range(S):
        k = s % KI
        if k == 0 and s > 0:
            ev.append(("store", 16 if KI > 1 else 32))  # (part of) the previous tile
        ev.append(("load", "B", s + 1, NB))
        if KI == 1 and NSC:
            ev.append(("load", "E", s, NSC))  # this tile's, before the wait
        ev.append(("read", s))  # first half of the row blocks
        ev.append(("wait", wait_fn(s, k)))
        ev.append(("barrier",))
        if k == KI - 1 and KI > 1 and NSC:
            ev.append(("load", "E", s // KI + 1, NSC))  # the next tile's, after the wait
        ev.append(("load", "A", s + 3, NA))
        ev.append(("read", s))  # second half
        ev.append(("read", s + 1))  # the next tile's first two fragments
        if k == KI - 1 and KI > 1:
            ev.append(("store", 16))  # row blocks 0..7 of this tile
    return ev


def check_program(ev, L):
    """Returns a list of violations (empty when the schedule is proven).

    Loads complete in issue order, so a wait vmcnt(c) completes every load
    except the last c issued (stores are not counted: they can only delay a
    wait).  All waves run the same program and pass a barrier only after
    their own wait, so what one wave has completed at a barrier every wave
    has; the lgkmcnt(0) in every wait retires the wave's LDS reads."""
    bad = []
    n_loads = 0
    last_instr = {}  # A tile -> index of its last DMA instruction
    complete_upto = 0  # loads with index < complete_upto are complete
    covered = -1  # watermark at the latest barrier
    unretired = set()  # tiles read since the latest barrier
    for e in ev:
        kind = e[0]
        if kind == "load":
            _, what, idx, n = e
            if what == "A" and (idx - 4) in unretired:
                bad.append(f"DMA of tile {idx} into stage {L.stage_of(idx)} while tile {idx - 4} may still be read")
            n_loads += n
            if what == "A":
                last_instr[idx] = n_loads - 1
        elif kind == "wait":
            complete_upto = max(complete_upto, n_loads - e[1])
        elif kind == "barrier":
            covered = complete_upto
            unretired.clear()
        elif kind == "read":
            t = e[1]
            if t not in last_instr or last_instr[t] >= covered:
                bad.append(f"read of tile {t} before a barrier covering its DMA in every wave")
            unretired.add(t)
    return bad


def tight(L, KI, ntiles, NA, NB, NSC):
    """Every wait count equals the number of loads issued after the covered
    DMA (capped at 63): no count is stricter than it needs to be."""
    ev = program(L, KI, ntiles, NA, NB, NSC)
    issued, s = [], -1
    out = []
    for e in ev:
        if e[0] == "load":
            issued += [(e[1], e[2])] * e[3]
        elif e[0] == "wait":
            target = 0 if s < 0 else s + 1
            last = max(p for p, x in enumerate(issued) if x == ("A", target))
            after = len(issued) - 1 - last
            out.append((e[1], min(after, 63)))
        if e[0] == "barrier":
            s += 1
    return out


@pytest.mark.parametrize("mode", sorted(MODES))
def test_every_lds_read_is_covered(shim, mode):
    NA, NB, NSC = MODES[mode]
    for KI in range(1, 41):
        for ntiles in range(1, 6):
            bad = check_program(program(shim, KI, ntiles, NA, NB, NSC), shim)
            assert not bad, f"{mode} KI={KI} tiles={ntiles}: {bad[:3]}"


@pytest.mark.parametrize("mode", sorted(MODES))
def test_counts_are_exact(shim, mode):
    NA, NB, NSC = MODES[mode]
    for KI in range(1, 21):
        for ntiles in range(1, 4):
            for got, want in tight(shim, KI, ntiles, NA, NB, NSC):
                assert got == want, f"{mode} KI={KI} tiles={ntiles}: wait {got}, loads after target {want}"


def test_lookahead_dma_targets_stream_step_plus_three(shim):
    """The A DMA of K step k lands on stream step s + 3: tile d ahead, K tile
    kt, with d * KI + kt = k + 3.  The kernel holds the next two tiles; only
    K = 128 (KI = 1, every step the first and last of its tile) reaches the
    third, which the kernel computes separately."""
    for KI in range(1, 41):
        for k in range(KI):
            d, kt = shim.dma_ahead_tile(k, KI), shim.dma_ahead_kt(k, KI)
            assert 0 <= kt < KI and d * KI + kt == k + 3, (KI, k, d, kt)
            assert (d == 3) == (KI == 1), (KI, k, d)


def test_tile_phase_matches_stream_stage(shim):
    """The kernel compiles one variant per CASE and gives tile j of a
    workgroup the stage phase (phase_advance(CASE) * j) % 4; that must be the
    stage of the tile's first K tile, stream step j * KI."""
    for KI in range(1, 41):
        adv = shim.phase_advance(shim.case_of(KI))
        for j in range(12):
            assert (adv * j) % 4 == shim.stage_of(j * KI), (KI, j)


def test_k256_runs_the_tail_only_and_is_covered(shim):
    """K = 256: two K tiles per output tile, no middle steps at all."""
    NA, NB, NSC = MODES["ptpc"]
    ev = program(shim, 2, 3, NA, NB, NSC)
    assert check_program(ev, shim) == []


def test_checker_catches_a_bare_barrier(shim):
    """Mutant: the tail's wait replaced by vmcnt(63) -- the 'bare barrier'
    of the pages -- must be flagged for K = 256 and for long K."""
    NA, NB, NSC = MODES["ptpc"]
    for KI in (2, 14):
        def wf(s, k, KI=KI):
            return 63 if k == KI - 1 else shim.wait_at(s, k, KI, NA, NB, NSC)
        assert check_program(program(shim, KI, 2, NA, NB, NSC, wf), shim), KI


def test_checker_catches_a_count_one_too_high(shim):
    NA, NB, NSC = MODES["mxfp8"]
    for KI in (2, 3, 14):
        def wf(s, k, KI=KI):
            return shim.wait_at(s, k, KI, NA, NB, NSC) + NA
        assert check_program(program(shim, KI, 2, NA, NB, NSC, wf), shim), KI


def test_checker_catches_a_missing_war_barrier(shim):
    """Mutant: the DMA issued before the barrier instead of after it."""
    NA, NB, NSC = MODES["ptpc"]
    out = program(shim, 6, 1, NA, NB, NSC)
    # move each step's DMA in front of its wait + barrier
    mutated = []
    i = 0
    while i < len(out):
        if out[i][0] == "wait" and i + 2 < len(out) and out[i + 2][0] == "load" and out[i + 2][1] == "A" \
                and out[i + 1][0] == "barrier":
            mutated += [out[i + 2], out[i], out[i + 1]]
            i += 3
        else:
            mutated.append(out[i])
            i += 1
    assert check_program(mutated, shim)


# ------------------------------------------------------------------ layout
# (row blocks per stage / 16, waves): ptpc and mxfp8, the 8-wave 128-row tiles, blockscale 128 x 128
LAYOUTS = [(16, 4), (8, 8), (8, 4)]


def dma_blocks(MB, waves):
    NA = 2 * MB // waves
    return [(w, j, NA * w + j) for w in range(waves) for j in range(NA)]


@pytest.mark.parametrize("MB,waves", LAYOUTS)
def test_dma_writes_every_row_chunk_once(shim, MB, waves):
    seen = {}
    for w, j, b in dma_blocks(MB, waves):
        for l in range(64):
            addr = shim.dma_lds_byte(b, l)
            assert addr % 16 == 0 and 0 <= addr < 16 * MB * 128
            assert addr not in seen
            seen[addr] = (shim.dma_row(b, l, MB), shim.dma_chunk(b, l, MB))
    assert sorted(seen.values()) == [(r, c) for r in range(16 * MB) for c in range(8)]
    # every lane group of 8 fetches one whole 128-byte row (coalesced)
    for w, j, b in dma_blocks(MB, waves):
        for q in range(8):
            rows = {shim.dma_row(b, 8 * q + t, MB) for t in range(8)}
            chunks = {shim.dma_chunk(b, 8 * q + t, MB) for t in range(8)}
            assert len(rows) == 1 and chunks == set(range(8))


@pytest.mark.parametrize("MB,waves", LAYOUTS)
def test_fragment_reads_find_their_data(shim, MB, waves):
    where = {}
    for w, j, b in dma_blocks(MB, waves):
        for l in range(64):
            where[shim.dma_lds_byte(b, l)] = (shim.dma_row(b, l, MB), shim.dma_chunk(b, l, MB))
    for l in range(64):
        i, g = l % 16, l // 16
        for mb in range(MB):
            for half in (0, 1):
                addr = shim.frag_byte(i, g, mb, half, MB)
                assert where.get(addr) == (MB * i + mb, 4 * half + g), (MB, l, mb, half)


@pytest.mark.parametrize("MB", [16, 8])
def test_fragment_reads_are_bank_conflict_free(shim, MB):
    """64 banks x 4 bytes: the 16 lanes of each read phase hit 16 distinct
    16-byte bank groups."""
    for mb in range(MB):
        for half in (0, 1):
            for phase in range(4):
                groups = {(shim.frag_byte(l % 16, l // 16, mb, half, MB) // 16) % 16 for l in range(16 * phase, 16 * phase + 16)}
                assert len(groups) == 16, (MB, mb, half, phase, sorted(groups))


# ------------------------------------------------------------ bf16 layout
def test_bf16_layout_is_a_permutation_and_conflict_free(shim):
    """bf16 GEMM stages (lds::bf16_chunk_pos): every row's 8 chunks land on 8
    distinct positions, and each 16-lane phase of a fragment read (rows
    16 q + i, one chunk) hits 16 distinct 16-byte bank groups."""
    for r in range(128):
        assert sorted(shim.bf16_chunk_pos(r, c) for c in range(8)) == list(range(8))
    for q in range(8):
        for c in range(8):
            groups = {((16 * q + i) * 128 + shim.bf16_chunk_pos(16 * q + i, c) * 16) // 16 % 16 for i in range(16)}
            assert len(groups) == 16, (q, c, sorted(groups))


def test_bf16_old_swizzle_would_conflict():
    """The r & 7 swizzle puts rows i and i + 8 on the same bank group: the
    check above would reject it."""
    groups = {(i * 128 + ((0 ^ (i & 7)) * 16)) // 16 % 16 for i in range(16)}
    assert len(groups) == 8


# ------------------------------------------------------- the bf16 GEMM's ring
BF16_RINGS = {"128x128": (4, 8), "64x64": (3, 4)}  # NS, NL (DMAs per wave per K tile) of each tile shape


def program_bf16(L, KT, NS, NL, prologue=None, mid=None, refill_before_barrier=False):
    """One wave's events in the bf16 GEMM (kpipe.h, the bf16 ring): DMA j
    writes stage j % NS; R(t) reads K tile t's stage."""
    prologue = L.bf16_prologue_wait(NS, NL) if prologue is None else prologue
    mid = L.bf16_mid_wait(NS, NL) if mid is None else mid
    ev = [("load", "A", j, NL) for j in range(NS)]
    ev += [("wait", prologue), ("barrier",), ("read", 0)]
    for kt in range(KT):
        ev.append(("read", kt))
        if refill_before_barrier:
            ev.append(("load", "A", kt + NS, NL))
        ev += [("wait", mid), ("barrier",)]
        if not refill_before_barrier:
            ev.append(("load", "A", kt + NS, NL))
        ev.append(("read", kt + 1))
    return ev


def check_ring(ev, NS):
    """RAW: a read of tile t follows a barrier whose waits (in every wave)
    covered t's DMAs.  WAR: a DMA of tile j into stage j % NS comes after a
    barrier that every wave passed with its reads of the stage's previous
    tile (j - NS) retired (the lgkmcnt(0) in each wait)."""
    bad, n_loads, last_instr, complete_upto, covered = [], 0, {}, 0, -1
    unretired, retired_at_barrier = set(), set()
    for e in ev:
        if e[0] == "load":
            _, _, j, n = e
            if j - NS >= 0 and (j - NS) not in retired_at_barrier:
                bad.append(f"DMA of tile {j} while tile {j - NS} may still be read")
            n_loads += n
            last_instr[j] = n_loads - 1
        elif e[0] == "wait":
            complete_upto = max(complete_upto, n_loads - e[1])
        elif e[0] == "barrier":
            covered = complete_upto
            retired_at_barrier |= unretired
            unretired = set()
        elif e[0] == "read":
            t = e[1]
            if t not in last_instr or last_instr[t] >= covered:
                bad.append(f"read of tile {t} before a barrier covering its DMA")
            unretired.add(t)
            retired_at_barrier.discard(t)
    return bad


@pytest.mark.parametrize("tile", sorted(BF16_RINGS))
def test_bf16_ring_is_covered_for_every_k(shim, tile):
    NS, NL = BF16_RINGS[tile]
    for KT in range(1, 40):
        assert check_ring(program_bf16(shim, KT, NS, NL), NS) == [], (tile, KT)


def test_bf16_ring_counts_are_the_loosest_safe_ones(shim):
    """One more outstanding DMA at either wait breaks coverage."""
    for NS, NL in BF16_RINGS.values():
        for KT in (1, 2, 5, 16):
            assert check_ring(program_bf16(shim, KT, NS, NL, prologue=shim.bf16_prologue_wait(NS, NL) + 1), NS)
            if KT >= 2:
                assert check_ring(program_bf16(shim, KT, NS, NL, mid=shim.bf16_mid_wait(NS, NL) + 1), NS)


def test_bf16_ring_catches_a_refill_before_the_barrier(shim):
    for NS, NL in BF16_RINGS.values():
        assert check_ring(program_bf16(shim, 8, NS, NL, refill_before_barrier=True), NS)


def test_bf16_ring_shapes_match_the_kernel():
    """NS and NL as gemm_bf16.hip derives them: 4 stages of a 128 x 128 tile
    (A and B 16 KiB each per K tile of 64 = 8 KiB per wave), 3 of 64 x 64."""
    src = open(os.path.join(CSRC, "gemm_bf16.hip")).read()
    assert "static constexpr int NS = BM == 128 ? 4 : 3;" in src
    for bm, (NS, NL) in ((128, BF16_RINGS["128x128"]), (64, BF16_RINGS["64x64"])):
        assert NL == 2 * (bm * 64 * 2 // 1024 // 4)


# ------------------------------------------------------------- B row order
def test_b_layout_is_a_permutation_of_each_group(shim):
    """Every group of p blocks (p = 1..4) sends its 16 p fragment rows to its
    16 p output columns exactly once."""
    for p in range(1, 5):
        cols = sorted(shim.frag_col(nb, r, p) for nb in range(p) for r in range(16))
        assert cols == list(range(16 * p)), p


def test_b_layout_gives_each_lane_two_runs_of_eight_columns(shim):
    """Lane (i, g) holds B-operand rows 4g .. 4g+3 of each block in its
    accumulators: in a full group its blocks 0-1 cover columns 8g .. 8g+7
    and blocks 2-3 columns 32+8g .. 32+8g+7, in register order; a pair in a
    partial group covers 8g .. 8g+7 the same way; a lone block covers
    16 nb + 4g .. + 3."""
    for p in range(1, 5):
        for g in range(4):
            for pair in range(p // 2):
                run = [shim.frag_col(2 * pair + h, 4 * g + v, p) for h in range(2) for v in range(4)]
                assert run == list(range(32 * pair + 8 * g, 32 * pair + 8 * g + 8)), (p, g, pair)
            if p % 2:
                nb = p - 1
                assert [shim.frag_col(nb, 4 * g + v, p) for v in range(4)] == [16 * nb + 4 * g + v for v in range(4)]


def test_group_blocks_counts_the_last_partial_group(shim):
    assert [shim.group_blocks(G, 393) for G in (0, 97, 98, 99)] == [4, 4, 1, 0]  # N = 6288
    assert [shim.group_blocks(G, 3) for G in (0, 1)] == [3, 0]                  # N = 48
