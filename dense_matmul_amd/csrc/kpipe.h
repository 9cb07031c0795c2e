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
// Per wave, in issue order (KI = K / 128 tiles, NA / NB instructions):
//   prologue : Bev(0), A(0), A(1), A(2);
//              wait vmcnt(prologue_wait) lgkmcnt(0); s_barrier
//   step k   : top : Bev(k+1)
//              mid : wait vmcnt(mid_wait(k)) lgkmcnt(0); s_barrier;
//                    A(k+3) into LDS stage (k+3) % 4
// A(j) is the global->LDS DMA of K tile j (NA instructions per wave), Bev(j)
// the direct-to-register loads of tile j's B fragments plus any per-tile scale
// loads (NB instructions per wave).  Every step issues both, always: a load
// of a tile index >= KI goes through a zero-length buffer descriptor, so it
// moves no data but still counts in vmcnt.  The counts therefore never depend
// on K, and the tail -- including K = 256, where no step refills anything
// real -- runs exactly the same waits as the middle of a long K loop.
//
// A wait vmcnt(c) leaves at most the c most recently issued vector-memory
// instructions outstanding, and they complete in issue order, so the wait
// covers a DMA exactly when c is at most the number of instructions issued
// after it.  The functions return that number (the loosest count that still
// covers the DMA); the barrier that follows extends the guarantee from this
// wave's share of the tile to every wave's.  The lgkmcnt(0) before the same
// barrier retires this wave's LDS reads of stage (k+3) % 4 (tile k-1) before
// any wave refills it.
#pragma once

namespace dmm {
namespace sched {

constexpr int kStages = 4;  // LDS stages of the A tile

// Prologue wait: covers A(0); A(1) and A(2) were issued after it.
constexpr int prologue_wait(int NA) { return 2 * NA; }

// Mid-step wait of step k: covers A(k+1).
//   k == 0: A(1) is followed by A(2) and Bev(1).
//   k >= 1: A(k+1) is followed by Bev(k), A(k+2) and Bev(k+1).
constexpr int mid_wait(int k, int NA, int NB) { return k == 0 ? NA + NB : 2 * NB + NA; }

// Which issues of step k move real data (the rest are zero-length).
constexpr bool b_valid(int k, int KI) { return k + 1 < KI; }
constexpr bool a_valid(int k, int KI) { return k + 3 < KI; }

// LDS stage holding K tile j, and the stage step k refills.
constexpr int stage_of(int j) { return j % kStages; }
constexpr int refill_stage(int k) { return (k + 3) % kStages; }

}  // namespace sched
}  // namespace dmm
