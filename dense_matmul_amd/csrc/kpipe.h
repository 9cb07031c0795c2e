// kpipe.h -- the issue schedule of the fp8 GEMM's K pipeline and the vmcnt
// value of every wait in it.  Plain constexpr C++ so that the kernel and a
// host-side checker evaluate the very same functions.
//
// The race the pages study (mori PR 785 "fix(gemm-ar): drain the peeled
// tail's producers instead of tightening the loop", sections Problem and Why
// the existing A+B-1 did not fix it; aiter PR 6539, Technical Details) is an
// LDS read that a barrier lets through before every wave's global->LDS copy of
// that tile has landed.  Here each wait names exactly which copy it covers.
//
// A workgroup walks a stream of K tiles: all K tiles of its first output
// tile, then all of the next, and so on (s = stream position, k = K tile
// within the output tile, KI = K / 128).  Per wave, in issue order:
//   prologue : Bev(0), [E(tile 0) if KI >= 2,] A(0), A(1), A(2);
//              wait vmcnt(prologue_wait) lgkmcnt(0); s_barrier
//   step s   : top : Bev(s+1) [, E(this tile) if KI == 1]
//              mid : wait vmcnt(c(s)) lgkmcnt(0); s_barrier;
//                    [E(next tile) if k == KI-1 and KI >= 2;]
//                    A(s+3) into LDS stage (s+3) % 4
//              stores of an output tile are spread over its step k == KI-1
//              and the next tile's step k == 0 (all in k == 0 if KI == 1)
// A(j) is the global->LDS DMA of stream K tile j (NA loads per wave), Bev(j)
// the direct-to-register loads of its B fragments plus any per-K-tile scales
// (NB loads), E the ptpc epilogue's scale loads (NSC loads).  E is read at
// the top of the step that starts storing its tile, so with KI >= 2 a
// tile's last step loads the next tile's (the prologue tile 0's); with
// KI == 1 each step loads its own tile's and stores the previous one.  Every step
// issues its loads unconditionally: a position past the end of the stream
// goes through a zero-length buffer descriptor, moves no data and still
// counts in vmcnt.  So the counts below depend only on where a step sits in
// its output tile, never on K or on the stream's length: the peeled tail,
// K = 256 (two steps per tile) and K = 128 (one) run the same rule.
//
// A wait vmcnt(c) leaves at most the c most recently issued vector-memory
// operations outstanding.  Loads complete in issue order, so a wait covers a
// load exactly when c is at most the number of LOADS issued after it; stores
// (the epilogue's) are left out of that number on purpose -- they only make
// the counter larger, so a wait that ignores them is still sufficient even
// if stores and loads complete out of order with respect to each other.
// The functions return that number (the loosest count that still covers
// the load), capped at the 6-bit field.  The barrier after the wait extends
// the guarantee from this wave's share of the tile to every wave's; the
// lgkmcnt(0) before the same barrier retires this wave's LDS reads of stage
// (s+3) % 4 (K tile s-1) before any wave refills it.
#pragma once

namespace dmm {
namespace sched {

constexpr int kStages = 4;  // LDS stages of the A tile

// The kernel's modes and the shape each gives a workgroup (the kernel's Cfg
// reads these, and so does the host-side checker):
//   0 ptpc, 256 x 256, 4 waves         3 ptpc, 128 x 256, 8 waves
//   1 blockscale, 128 x 256, 8 waves   4 ptpc over a gathered A, 256 x 256
//   2 mxfp8, 256 x 256, 4 waves        5 mxfp8, 256 x 128, 4 waves
//   6 blockscale, 128 x 128, 4 waves   7 ptpc, 128 x 128, 4 waves
// Each wave owns MB 16-row blocks (all rows of the tile) and NBW 16-column
// blocks.  Per K tile a wave issues NA A-tile DMAs (1 KiB each: the 16 MB x
// 128-byte tile split over the waves) and NB vector loads of its B event
// (2 NBW fragment halves plus the mode's per-K-tile scales: mxfp8 a 16-byte
// window and a dword of A scales and a dword of B scales, blockscale two
// 16-byte A-scale loads and a dword of B scale); ptpc tiles load their
// epilogue scales with NSC = 2 more DMAs per tile.
struct Shape {
    int MB, NBW, WAVES, NA, NB, NSC;
};
constexpr Shape shape_of(int mode) {
    const bool narrow = mode == 1 || mode == 3, slim = mode == 5, square = mode == 6 || mode == 7;
    const bool ptpc = mode == 0 || mode == 3 || mode == 4 || mode == 7;
    const int MB = narrow || square ? 8 : 16, NBW = narrow || slim || square ? 2 : 4, WAVES = narrow ? 8 : 4;
    return Shape{MB, NBW, WAVES, 2 * MB / WAVES, ptpc ? 2 * NBW : 2 * NBW + 3, ptpc ? 2 : 0};
}
constexpr int kVmcntMax = 63;

constexpr int cap(int c) { return c > kVmcntMax ? kVmcntMax : c; }

// Prologue wait: covers A(0); A(1) and A(2) were issued after it.
constexpr int prologue_wait(int NA) { return 2 * NA; }

// Mid-step wait of the stream's first step: A(1) is followed by A(2) and
// Bev(1) (plus E if the first output tile has a single K tile).
constexpr int first_mid_wait(int NA, int NB) { return NA + NB; }

// Mid-step wait of step s >= 1: A(s+1) (issued at step s-2, or in the
// prologue for s = 1) is followed by Bev(s), A(s+2) and Bev(s+1), plus NSC
// for each E issued in between: KI == 1, the E of steps s-1 and s;
// otherwise the one of step s-1 when it closed its output tile (k == 0) --
// an E of step s-2 precedes that step's A DMAs.
constexpr int mid_wait(int NA, int NB) { return 2 * NB + NA; }

// The full rule, as the kernel applies it.
constexpr int wait_at(int s, int k, int KI, int NA, int NB, int NSC) {
    const int extra = KI == 1 ? 1 + (s > 0 ? 1 : 0) : (s > 0 && k == 0 ? 1 : 0);
    return cap((s == 0 ? first_mid_wait(NA, NB) : mid_wait(NA, NB)) + extra * NSC);
}

// Target of the A DMA issued in K step k of a tile (KI K tiles per tile):
// stream step s + 3, i.e. K tile dma_ahead_kt of the tile dma_ahead_tile
// places further down the workgroup's list.  The kernel keeps the next two
// tiles at hand; only K = 128 (KI = 1) reaches three tiles ahead.
constexpr int dma_ahead_tile(int k, int KI) {
    return k + 3 < KI ? 0 : k + 3 < 2 * KI ? 1 : k + 3 < 3 * KI ? 2 : 3;
}
constexpr int dma_ahead_kt(int k, int KI) { return k + 3 - KI * dma_ahead_tile(k, KI); }

// The kernel is compiled per CASE = KI % 4 for KI >= 2 and CASE = 4 for
// KI = 1 (every step both the first and the last of its tile).  Tile j's
// first K tile is stream step j KI, in stage (j KI) % 4: the stage advances
// by phase_advance(CASE) = KI % 4 per tile.
constexpr int case_of(int KI) { return KI == 1 ? 4 : KI % 4; }
constexpr int phase_advance(int CASE) { return CASE == 4 ? 1 : CASE; }

// LDS stage holding stream K tile j, and the stage step s refills.
constexpr int stage_of(int j) { return j % kStages; }
constexpr int refill_stage(int s) { return (s + 3) % kStages; }

// The bf16 GEMM (gemm_bf16.hip) runs a simpler ring: NS stages, one output
// tile per workgroup, NL DMAs per wave per K tile (A and B both through LDS).
//   prologue: D(0) .. D(NS-1) into stages 0 .. NS-1;
//             wait vmcnt(bf16_prologue_wait) lgkmcnt(0); s_barrier; R(0, half 0)
//   step kt : R(kt, half 1); wait vmcnt(bf16_mid_wait) lgkmcnt(0); s_barrier;
//             D(kt + NS) into stage kt % NS; R(kt + 1, half 0)
// D(j) past the last K tile goes through an empty descriptor (counted, no
// data).  The prologue wait covers D(0) (NS - 1 tiles' DMAs after it); the
// mid wait of step kt covers D(kt + 1), after which D(kt + 2) .. D(kt + NS -
// 1) were issued.
constexpr int bf16_prologue_wait(int NS, int NL) { return cap((NS - 1) * NL); }
constexpr int bf16_mid_wait(int NS, int NL) { return cap((NS - 2) * NL); }

}  // namespace sched
}  // namespace dmm
