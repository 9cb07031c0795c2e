// tile_order.h -- which output tiles each workgroup of the persistent fp8
// GEMM computes, and in what order.  Plain constexpr C++ so that the kernel
// and host-side tests evaluate the very same functions.
//
// A workgroup computes positions first, first + stride, ... (n of them) of a
// linear tile order; a position maps to a (row tile, column tile) pair.
#pragma once

namespace dmm {
namespace order {

constexpr int kXcds = 8;   // the dispatcher deals workgroups to the XCDs in turn
constexpr int kGroup = 4;  // row tiles that sweep the column tiles together

struct List {
    int first, stride, n;
};

constexpr List make_list(int first, int stride, int end) {
    return List{first, stride, first < end ? (end - first + stride - 1) / stride : 0};
}

// Default order: workgroup wg runs on XCD wg % 8; XCD x owns a contiguous
// eighth of the positions and its workgroups stride through it, so the
// tiles in flight on one XCD at any time are neighbours in the order.
constexpr List xcd_list(int wg, int grid, int T) {
    const int x = wg % kXcds, per = T / kXcds, rem = T % kXcds;
    const int start = x * per + (x < rem ? x : rem);
    const int count = per + (x < rem ? 1 : 0);
    const int slots = (grid - x + kXcds - 1) / kXcds;  // workgroups on XCD x
    return make_list(start + wg / kXcds, slots, start + count);
}

// Time-ordered: round j of the grid covers positions [j grid, (j+1) grid),
// so the whole grid works through the order front to back; within a round
// XCD x takes a contiguous chunk (its workgroups' slots), keeping its tiles
// neighbours.  Used when the rows of later tiles arrive later.
constexpr List round_list(int wg, int grid, int T) {
    const int x = wg % kXcds;
    int off = 0;
    for (int y = 0; y < x; ++y) off += (grid - y + kXcds - 1) / kXcds;
    return make_list(off + wg / kXcds, grid, T);
}

// Position t -> (row tile, column tile) within a block of rows_t row tiles:
// kGroup row tiles sweep all column tiles, so tiles close in the order share
// A rows and B columns.
constexpr void coords(int t, int rows_t, int tiles_n, int& tm, int& tn) {
    const int group = t / (kGroup * tiles_n);
    const int first = group * kGroup;
    const int gsize = rows_t - first < kGroup ? rows_t - first : kGroup;
    const int within = t - group * kGroup * tiles_n;
    tm = first + within % gsize;
    tn = within / gsize;
}

// Gathered operand (the GEMM half of an all-gather + GEMM; mori PR 809,
// How it works: tile order and the wait).  A is nsrc source slabs of bt row
// tiles each, slab s = rows [s bt 256, (s+1) bt 256); slab `own` is resident
// from the start and every other slab arrives in nchunks chunks of
// bt / nchunks row tiles, chunk c of slab s guarded by band s nchunks + c.
// The order: the own slab first (no wait); then for each chunk c, the
// sources own+1, own+2, ... (mod nsrc), each chunk's tiles in the coords
// order.  Sets band to the band a tile waits for, or -1.
constexpr void gathered_coords(int u, int bt, int nsrc, int nchunks, int own, int tiles_n, int& tm, int& tn,
                               int& band) {
    const int own_tiles = bt * tiles_n;
    if (u < own_tiles) {
        coords(u, bt, tiles_n, tm, tn);
        tm += own * bt;
        band = -1;
        return;
    }
    const int ct = bt / nchunks;        // row tiles per chunk
    const int per = ct * tiles_n;       // tiles per (chunk, source)
    const int v = u - own_tiles;
    const int idx = v / per;            // (chunk, source) in order
    const int c = idx / (nsrc - 1);
    const int src = (own + 1 + idx % (nsrc - 1)) % nsrc;
    coords(v - idx * per, ct, tiles_n, tm, tn);
    tm += src * bt + c * ct;
    band = src * nchunks + c;
}

}  // namespace order
}  // namespace dmm
