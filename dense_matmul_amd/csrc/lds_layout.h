// lds_layout.h -- where the fp8 GEMM's A tile lives in LDS.  Plain constexpr
// C++ shared by the kernel and a host-side checker.
//
// A stage holds 16 * MB rows of 128 bytes (one 128-wide K tile of fp8
// codes).  Row r sits in row slot r ^ h(r), h(r) = (r >> HB) & 1 with
// HB = log2(8 MB), i.e. the upper half of the rows swaps slot parity; inside
// a row, 16-byte chunk c sits at position c ^ ((r / MB) & 7).
//
// An A fragment (16 rows x 128 K for the 16x16x128 matrix-core op) is read
// by lane (i, g) = (l % 16, l / 16) from row MB i + mb, chunks g and 4 + g.
// For 64 LDS banks of 4 bytes, the 16 lanes of one read phase then cover
// 256 distinct bytes of bank space: rows i and i + 8 differ in slot parity
// and within a parity the eight chunk positions differ.
//
// The global -> LDS DMA writes 16 bytes per lane at consecutive addresses
// (lane l of a 1 KiB instruction writes slot 8 q + l / 8, position l % 8), so
// the permutation is applied on the global side: that lane fetches the row
// and chunk that belong there.
#pragma once

namespace dmm {
namespace lds {

constexpr int log2i(int v) { return v <= 1 ? 0 : 1 + log2i(v / 2); }
constexpr int half_bit(int MB) { return log2i(8 * MB); }

// slot <-> row (an involution)
constexpr int slot_of_row(int r, int MB) { return r ^ ((r >> half_bit(MB)) & 1); }
constexpr int row_of_slot(int q, int MB) { return slot_of_row(q, MB); }

// position of chunk c of row r inside its slot (an involution in c)
constexpr int chunk_pos(int r, int c, int MB) { return c ^ ((r / MB) & 7); }

// The stage is written by 2 MB DMA instructions of 1 KiB; instruction j of
// wave w is block b = NA w + j (NA = 2 MB / waves per wave).  Lane l of
// block b: the LDS byte it writes and the (row, chunk) it must fetch.
constexpr int dma_lds_byte(int b, int l) { return b * 1024 + 16 * l; }
constexpr int dma_row(int b, int l, int MB) { return row_of_slot(8 * b + (l >> 3), MB); }
constexpr int dma_chunk(int b, int l, int MB) { return chunk_pos(dma_row(b, l, MB), l & 7, MB); }

// Fragment read of row block mb by lane (i, g), half 0 (chunk g) or 1
// (chunk 4 + g): base[mb & 1][half] + 128 mb.  With h = (i >> 3) & 1 the
// slot of row MB i + mb is MB i + mb + h for even mb, MB i + mb - h for odd.
constexpr int frag_base(int i, int g, int odd_mb, int half, int MB) {
    const int h = ((MB * i) >> half_bit(MB)) & 1;
    const int r0 = MB * i;
    return (r0 + (odd_mb ? -h : h)) * 128 + chunk_pos(r0, half * 4 + g, MB) * 16;
}
constexpr int frag_byte(int i, int g, int mb, int half, int MB) { return frag_base(i, g, mb & 1, half, MB) + 128 * mb; }

// The bf16 GEMM's stages: rows of 128 bytes (64 bf16 of one K tile), 16-byte
// chunk c of row r at position c ^ ((r >> 1) & 7).  Its fragment reads take
// rows 16 q + i (i = 0..15) and one chunk for all 16 lanes of a phase; rows
// i and i + 1 differ in 128-byte parity (the two halves of the 256 bytes of
// bank space) and, within a parity, (i >> 1) & 7 takes all eight values, so
// the phase touches 16 distinct 16-byte bank groups.  (Swizzling by r & 7
// would put rows i and i + 8 on the same banks.)  The DMA writes lane l of
// a 1 KiB instruction at row 8 q + l / 8, position l % 8, and fetches the
// chunk that belongs there.
constexpr int bf16_chunk_pos(int r, int c) { return c ^ ((r >> 1) & 7); }

}  // namespace lds
}  // namespace dmm
