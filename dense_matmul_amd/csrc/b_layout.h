// b_layout.h -- which output column each row of a preshuffled B fragment
// feeds.  Plain constexpr C++ shared by preshuffle_b, the fp8 GEMM (epilogue
// store columns, ptpc and mxfp8 scale columns) and a host-side checker.
//
// B's N rows (one per output column) come in 16-row blocks, one matrix-op
// operand each, and the blocks in groups of four: 64 output columns, one
// wave's share of a 256-wide tile (a 32-column wave takes two blocks of a
// group).  Fragment row r (0..15) of block nb of a group holds output column
// frag_col(nb, r, p) of the group, where p is the group's block count: 4, or
// 1..3 for the last group when N % 64 != 0.
//
// The matrix op's output puts B-operand rows 4g .. 4g + 3 in the four
// accumulators of lane (i, g) (i = lane % 16, g = lane / 16), so with
// frag_col a lane ends a row block holding columns 8g .. 8g + 7 (blocks 0
// and 1) and 32 + 8g .. 32 + 8g + 7 (blocks 2 and 3): two runs of 8 adjacent
// columns, each one 16-byte store, and four lanes together cover 64
// contiguous bytes of a row -- no lane exchange before the stores.  A block
// without a partner (the last block of a group with an odd count) keeps its
// rows in order: lane g then holds columns 16 nb + 4g .. 16 nb + 4g + 3.
#pragma once

namespace dmm {
namespace bl {

// blocks in group G of a B with nblocks 16-row blocks (0 past the end)
constexpr int group_blocks(int G, int nblocks) {
    const int p = nblocks - 4 * G;
    return p < 0 ? 0 : p > 4 ? 4 : p;
}

// block nb of a group of p blocks has no partner
constexpr bool lone(int nb, int p) { return (p & 1) != 0 && nb == p - 1; }

// output column (within the group) fed by fragment row r of block nb
constexpr int frag_col(int nb, int r, int p) {
    return lone(nb, p) ? 16 * nb + r : 32 * (nb >> 1) + 8 * (r >> 2) + 4 * (nb & 1) + (r & 3);
}

}  // namespace bl
}  // namespace dmm
