// gemm_a8w8.hip -- fp8 (OCP E4M3) a8w8 GEMM for gfx950 with bf16 output, in
// the three scaling modes of mori PR 785 ("fix(gemm-ar): drain the peeled
// tail's producers instead of tightening the loop", section Cost): ptpc,
// 1x128 / 128x128 blockscale and mxfp8.
//
//   C[m, n] = bf16( sum_k A[m, k] sa(m, k) * B[n, k] sb(n, k) ),  fp32 accumulate
//
// Structure (persistent: one workgroup per CU, each walking its list of
// output tiles as one continuous stream of K tiles, so the loads of the next
// tile overlap the end of the current one and its stores):
//   * Output tile 16*MB x 256: 256 x 256 with 4 waves for ptpc and mxfp8,
//     128 x 256 with 8 waves for blockscale and the narrow ptpc tile.  Wave
//     w owns all tile rows and the WN = 256 / waves columns [WN w, WN w + WN).
//   * Tile order (tile_order.h): XCD-aware groups of row tiles sweeping the
//     column tiles; the gathered-operand mode walks its own slab first and
//     polls an arrival flag before it loads a remote band's rows.
//   * A (row-major codes) streams global -> LDS with direct-to-LDS buffer
//     loads (16 B per lane) through a 4-stage ring of separate LDS arrays,
//     refilled three K tiles ahead.  Rows sit 128 B apart; the 16-byte
//     chunks are XOR-swizzled by (row / MB) & 7 and rows 128..255 swap slot
//     parity, so a fragment read by 16 lanes touches all 64 banks once.
//   * B comes pre-shuffled (preshuffle_b) into the matrix-core operand order,
//     so every wave loads its fragments straight into registers with fully
//     coalesced 1 KiB loads, one K tile ahead (register double buffer).
//   * v_mfma_scale_f32_16x16x128_f8f6f4: src0 = 16 B rows (output columns),
//     src1 = 16 A rows (output rows).  Lane l holds row l % 16 and, in bytes
//     0-15 / 16-31, K values 16(l/16)+[0,16) / 64+16(l/16)+[0,16) of the
//     128-wide K tile (the instruction's operand layout on gfx950).  mxfp8
//     passes the E8M0 scales to the instruction (lane 16q + i carries the
//     scale of row i, K group q); ptpc applies both scales in the epilogue;
//     blockscale folds one scale per 128-K tile into fp32 accumulators.
//   * Every LDS read of a K tile follows "s_waitcnt vmcnt(c) lgkmcnt(0);
//     s_barrier" where c comes from kpipe.h and covers that tile's DMA in
//     every wave.  Every step issues its loads unconditionally (positions
//     past the end go through a zero-length buffer descriptor), so the
//     counts never depend on K: the tail, K = 256 and K = 128 run the same
//     rule as the middle of a long K loop.
//   * Epilogue: preshuffle_b orders B's rows within each group of 64 output
//     columns (b_layout.h) so that every lane ends a row block with two runs
//     of 8 adjacent columns: the bf16 tile leaves in 16-byte stores, four
//     lanes covering 64 contiguous bytes of a row, with no lane exchange;
//     rows past M and runs past N fall outside the C descriptor and are
//     dropped.  ptpc and mxfp8 spread it over a tile's last K step and the
//     next tile's first.
#include "b_layout.h"
#include "common.h"
#include "kpipe.h"
#include "lds_layout.h"
#include "tile_order.h"

#include <type_traits>

namespace dmm {

// MODE_PTPC_N: ptpc on the 128 x 256 tile of eight waves (see Cfg);
// MODE_PTPC_G: ptpc over a gathered A (Gather), 256 x 256 tiles;
// MODE_MXFP8_N: mxfp8 on the 256 x 128 tile of four waves;
// MODE_BLOCKSCALE_N: blockscale on a 128 x 128 tile of four waves;
// MODE_PTPC_Q: ptpc on a 128 x 128 tile of four waves.
enum {
    MODE_PTPC = 0,
    MODE_BLOCKSCALE = 1,
    MODE_MXFP8 = 2,
    MODE_PTPC_N = 3,
    MODE_PTPC_G = 4,
    MODE_MXFP8_N = 5,
    MODE_BLOCKSCALE_N = 6,
    MODE_PTPC_Q = 7
};

template <int MODE>
constexpr bool kWidePtpc = MODE == MODE_PTPC || MODE == MODE_PTPC_G;
// ptpc on 32-column waves with VGPR accumulators (128 x 256 and 128 x 128)
template <int MODE>
constexpr bool kNarrowPtpc = MODE == MODE_PTPC_N || MODE == MODE_PTPC_Q;
template <int MODE>
constexpr bool kPtpc = kWidePtpc<MODE> || kNarrowPtpc<MODE>;
template <int MODE>
constexpr bool kMx = MODE == MODE_MXFP8 || MODE == MODE_MXFP8_N;
template <int MODE>
constexpr bool kBlock = MODE == MODE_BLOCKSCALE || MODE == MODE_BLOCKSCALE_N;

constexpr int BK = 128;

// The LDS ring: four distinct arrays so that the compiler can tell the
// stages apart (its own LDS-DMA dependency tracking is per object).
constexpr int kMaxStageBytes = 256 * BK;
__shared__ __attribute__((aligned(1024))) char g_lds_a0[kMaxStageBytes];
__shared__ __attribute__((aligned(1024))) char g_lds_a1[kMaxStageBytes];
__shared__ __attribute__((aligned(1024))) char g_lds_a2[kMaxStageBytes];
__shared__ __attribute__((aligned(1024))) char g_lds_a3[kMaxStageBytes];
// ptpc epilogue scales: per wave (up to eight) 1 KiB of a_scale (the tile's
// rows, up to 256) and 1 KiB of b_scale (the tile's 256 columns)
__shared__ __attribute__((aligned(1024))) char g_lds_scale[8 * 2048];

// The kernel body takes the four stage addresses and carries them in its
// context (the host compilation pass only accepts references to the LDS
// arrays there); after inlining they are constants again.
struct Stages {
    lds_char* p[4];
    lds_char* scale;
};

template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

// DPP control of a row broadcast.
constexpr int kDppRowNewBcast = 0x150;  // + k: lane k of each 16-lane row to the whole row

// Cache-policy bits of the 256-wide tiles' C stores (a lane's two 16-byte
// runs cover 64 bytes of each 128-byte line; the other half comes from the
// same wave's next store).  Non-temporal (nt) keeps C from displacing the A
// and B panels in the L2, which pays when K is long; with short K the C
// write dominates and device scope (sc1) on top of nt writes the lines out
// faster (measured, nt + sc1 vs nt: 4096 x 7168 x 256 14.3 vs 20.7 us,
// 32768 x 7168 x 1792 318.6 vs 319.0 us, 32768 x 6288 x 7168 1082 vs 1011 us).
constexpr int kStoreNt = 2;
constexpr int kStoreNtSc1 = 18;
constexpr int kLongK = 4096;  // K at or above which the stores are nt only

// Gathered operand (order::gathered_coords): band b's rows of A and
// a_scale may be read once flags[b] has reached epoch (wrap-safe compare).
struct Gather {
    const uint32_t* flags;  // null: A is resident, default order
    int bt, nsrc, nchunks, own;
    uint32_t epoch;
    long long spin_limit;   // polls per band before giving up
    int* status;            // set to 1 + band (the largest) when a wait gave up
};

struct GemmArgs {
    const uint8_t* a;
    const uint8_t* b;
    const void* sa;
    const void* sb;
    uint16_t* c;
    int m, n, k;
    int tiles_m, tiles_n;
    Gather gather;  // MODE_PTPC_G only
};

// The C stores' policy for a GEMM of depth k (kStoreNt / kStoreNtSc1).
constexpr bool store_nt_only(int k) { return k >= kLongK; }

// Tile shape per mode.  Each of the WAVES waves owns NBW 16-column blocks
// side by side and all MB 16-row blocks of the tile.  ptpc and mxfp8 keep
// their 256 x 256 tile in the 256 accumulation registers of 4 waves (one per
// SIMD).  Blockscale folds every K tile's products into VGPR accumulators
// with its scales, so each of its waves owns 128 x 32 (64 accumulators per
// lane) and 8 waves, two per SIMD, share a 128 x 256 tile: each SIMD then
// has a second wave to issue matrix ops while one waits.  MODE_PTPC_N runs
// ptpc on that narrow tile (matrix ops straight into VGPR accumulators),
// which doubles the tile count of small problems.  MODE_MXFP8_N runs mxfp8
// on a 256 x 128 tile of four waves, each owning all 256 rows and 32
// columns (128 AGPR accumulators): A, the operand that goes through LDS, is
// twice the size of B in each K tile.
// MODE_BLOCKSCALE_N runs the blockscale waves four to a 128 x 128 tile (one
// per SIMD), which doubles the tile count of grids that would leave CUs
// idle; MODE_PTPC_Q does the same for the narrow ptpc waves.
template <int MODE>
struct Cfg {
    static constexpr sched::Shape S = sched::shape_of(MODE);  // kpipe.h
    static constexpr int MB = S.MB;        // 16-row blocks per wave
    static constexpr int NBW = S.NBW;      // 16-column blocks per wave
    static constexpr int WAVES = S.WAVES;  // waves per workgroup
    static constexpr int NTHREADS = 64 * WAVES;
    static constexpr int BM = 16 * MB;     // tile rows
    static constexpr int WN = 16 * NBW;    // columns per wave
    static constexpr int BN = WAVES * WN;  // tile columns
    static constexpr int NA = S.NA;        // DMA instructions per wave per K tile
    // vector-memory instructions of one B event: 2 NBW fragment loads plus scales
    static constexpr int NB = S.NB;
    // vector-memory instructions of the ptpc epilogue's scale loads (two
    // 1 KiB DMAs per wave)
    static constexpr int NSC = S.NSC;
    static_assert(NA == 2 * MB / WAVES && NB == (kPtpc<MODE> ? 2 * NBW : 2 * NBW + 3) && NSC == (kPtpc<MODE> ? 2 : 0),
                  "the counts kpipe.h gives the mode are the loads the kernel issues");
    static_assert(2 * NB + NA <= 63, "vmcnt range");
};

// Whether a tile's epilogue is deferred into the next tile's first K step
// (the 256 x 256 tiles), and whether the accumulators are pinned to AGPRs
// (those and the 256 x 128 mxfp8 tile: 128 accumulators per lane there, which
// leave the VGPRs to the operands, so the compiler never has to move an
// accumulator that an asm matrix op may still be writing).
template <int MODE>
constexpr bool kDeferEpilogue = Cfg<MODE>::NBW == 4;
template <int MODE>
constexpr bool kAgprAcc = kDeferEpilogue<MODE> || MODE == MODE_MXFP8_N;

// Tile order of the persistent grid: tile_order.h (order::xcd_list, or
// order::round_list with the gathered order).

// One output tile of a workgroup's list: its origin and the byte offsets of
// its A rows and preshuffled B blocks.  Loads go through descriptors that
// end where A or B ends (a_rsrc, b_rsrc), so rows past M and column blocks
// past N fall outside them and read as zero.  Past the end of the list m0 =
// -1: the descriptors of such loads are empty, so they move no data but
// still count in vmcnt.
struct TileRef {
    int m0, n0;
    int a_off, b_off;
};

// What the epilogue of one tile needs besides the accumulators.
struct Epi {
    v4f eas[4], ebs[4];  // ptpc: a_scale of this lane's rows, b_scale of its columns
    // byte offsets into C, for row block 0, of this lane's two 16-byte runs
    // (columns 8g .. 8g + 7 of blocks 0-1, and of blocks 2-3, b_layout.h) and
    // of its 8-byte run in a lone block; a run that does not exist carries
    // 2^31 on top (all real offsets are below 2^31), which puts it past the C
    // descriptor, so the hardware drops the store without a branch
    uint32_t o16[2], o8;
    int lone;  // the wave's group ends in a lone block among this wave's (uniform)
};

template <int MODE>
struct Ctx {
    using C = Cfg<MODE>;
    Stages lds;
    const uint8_t* a;
    const uint8_t* b;
    const void* sa;
    const void* sb;
    uint16_t* c;
    int M, N, K, KI, tiles_m, tiles_n;
    bool nt_only;  // store_nt_only(K)
    order::List tl;
    int ntiles;
    Gather gather;             // MODE_PTPC_G only
    unsigned long long ready;  // MODE_PTPC_G: bands seen complete
    int w, lane, i, g;
    int dma_lds;        // byte offset of this wave's DMA slots in a stage
    int voff_a[C::NA];  // per-lane byte offsets of the DMA rows, relative to the tile's first row
    int voff_b[C::NBW]; // per-lane byte offsets of the B fragments, relative to the tile's first column
    int rd[2][2];       // LDS byte offsets of the two 16-byte halves of an A fragment, for even / odd mb
    v4f acc[C::MB][C::NBW];
    v8i bq[2][C::NBW];  // B fragments, double buffered across K tiles
    v8i pre[2];         // first two A fragments of the next K tile
    // mxfp8: E8M0 bytes for A (a 16-byte window plus one word to realign) and B (one per block)
    v4i sxa[2];
    int sxa_tail[2];
    int sxa_shift[2];
    int sxb_raw[2];      // B scale bytes of 4 columns as loaded, per K tile
    int sxb[C::NBW];     // B scale of this lane's fragment row in each block (byte 0), current step
    // blockscale: A scales of this lane's MB rows and the wave's B block scale;
    // the products of the last two row blocks, before they are scaled in
    v4f sfa[2][C::MB / 4];
    float sfb[2];
    v4f bp[2][C::NBW];
    // the epilogue of the tile being stored (ptpc, mxfp8)
    Epi ep;

    // Tile j of this workgroup's list with the buffer descriptors its loads
    // use (see TileRef).
    __device__ __forceinline__ TileRef ref(int j);
};

// Wait until band b of a gathered A has arrived: poll its flag with
// system-scope loads (every wave of the workgroup polls for itself, before
// any of its loads of the band's rows), then an acquire fence, so that the
// loads that follow see the band's rows and scales.  After spin_limit polls
// the wait gives up, records the band in status and goes on: the kernel
// always finishes.
__device__ __forceinline__ void await_band(const Gather& gth, int b) {
    long long polls = 0;
    for (;;) {
        const uint32_t f = __builtin_amdgcn_readfirstlane(
            __hip_atomic_load(gth.flags + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM));
        if ((int32_t)(f - gth.epoch) >= 0) break;
        if (++polls > gth.spin_limit) {
            if (threadIdx.x == 0) atomicMax(gth.status, b + 1);
            break;
        }
        __builtin_amdgcn_s_sleep(8);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "");
}

template <int MODE>
__device__ __forceinline__ TileRef Ctx<MODE>::ref(int j) {
    if (j >= ntiles) return TileRef{-1, -1, 0, 0};
    const int u = tl.first + j * tl.stride;
    int tm, tn;
    if constexpr (MODE == MODE_PTPC_G) {
        int band;
        order::gathered_coords(u, gather.bt, gather.nsrc, gather.nchunks, gather.own, tiles_n, tm, tn, band);
        if (band >= 0 && !((ready >> band) & 1ull)) {
            await_band(gather, band);
            ready |= 1ull << band;
        }
    } else {
        order::coords(u, tiles_m, tiles_n, tm, tn);
    }
    const int m0 = tm * C::BM, n0 = tn * C::BN;
    return TileRef{m0, n0, m0 * K, (n0 / 16) * KI * 2048};
}

// Descriptors over A (B) from a tile's first row (first column block) to the
// end of the operand, or empty for a tile past the list.  Within the tile a
// lane's offset (its row or fragment, loop-invariant) is the instruction's
// VGPR offset and the K tile's the scalar offset, so no step spends vector
// instructions on addresses.  The range check, on the VGPR part (the scalar
// offset stays below K either way), still drops rows past M and column
// blocks past N: their offsets reach past the shortened extent.
// Blockscale keeps descriptors over the whole operand and adds the tile's
// offset to the VGPR offset instead: its two waves per SIMD share the scalar
// unit, where the per-step descriptor arithmetic cost it more than the
// vector additions it saves (16384 x 7168 x 2048: 241.5 against 237.5 us;
// ptpc and mxfp8 gain 1.3-2.4 %).
template <int MODE>
constexpr bool kTileRsrc = !kBlock<MODE>;

template <int MODE>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t a_rsrc(const Ctx<MODE>& x, int a_off, bool valid) {
    const uint32_t o = kTileRsrc<MODE> ? (uint32_t)__builtin_amdgcn_readfirstlane(a_off) : 0u;
    return make_rsrc(x.a + o, valid ? (uint32_t)x.M * (uint32_t)x.K - o : 0u);
}
template <int MODE>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t b_rsrc(const Ctx<MODE>& x, int b_off, bool valid) {
    const uint32_t o = kTileRsrc<MODE> ? (uint32_t)__builtin_amdgcn_readfirstlane(b_off) : 0u;
    return make_rsrc(x.b + o, valid ? (uint32_t)x.N * (uint32_t)x.K - o : 0u);
}

// ---------------------------------------------------------------- issue
// B event of one K tile: the B fragments (8 x 1 KiB loads per wave) plus
// the per-K-tile scales of the mode.  A step spreads the fragment loads over
// its first row blocks, one or two between consecutive groups of matrix ops.
//
// Fragment load Q (0..2 NBW-1): half Q % 2 of column block Q / 2; b_off =
// the tile's B offset (where rb starts, see b_rsrc), kbase = 2048 kt for K
// tile kt.
template <int MODE, int T, int Q>
__device__ __forceinline__ void b_piece(Ctx<MODE>& x, __amdgpu_buffer_rsrc_t rb, int b_off, int kbase) {
    const int voff = x.voff_b[Q / 2] + (Q % 2) * 1024;
    const v4i v = kTileRsrc<MODE>
                      ? __builtin_amdgcn_raw_buffer_load_b128(rb, voff, __builtin_amdgcn_readfirstlane(kbase), 0)
                      : __builtin_amdgcn_raw_buffer_load_b128(rb, voff + b_off + kbase, 0, 0);
    v8i& d = x.bq[T][Q / 2];
    constexpr int h = 4 * (Q % 2);
    d[h + 0] = v[0];
    d[h + 1] = v[1];
    d[h + 2] = v[2];
    d[h + 3] = v[3];
}

// The mode's per-K-tile scales of a B event (none for ptpc).
template <int MODE, int T>
__device__ __forceinline__ void b_scales(Ctx<MODE>& x, TileRef r, int kt) {
    using C = Cfg<MODE>;
    const bool valid = r.m0 >= 0;
    const int n0 = valid ? r.n0 : 0, m0 = valid ? r.m0 : 0;
    if constexpr (kMx<MODE>) {
        const __amdgpu_buffer_rsrc_t rsa = make_rsrc(x.sa, valid ? (uint32_t)(x.K / 32) * (uint32_t)x.M : 0u);
        const __amdgpu_buffer_rsrc_t rsb = make_rsrc(x.sb, valid ? (uint32_t)(x.K / 32) * (uint32_t)x.N : 0u);
        // A: 16 consecutive E8M0 bytes (rows 16i .. 16i+15 of the tile) of K
        // group 4kt + g; the row stride M need not be a multiple of 4, so
        // load the dword-aligned window and realign in registers
        const int off = (4 * kt + x.g) * x.M + m0 + 16 * x.i;
        const int base = off & ~3;
        x.sxa[T] = __builtin_amdgcn_raw_buffer_load_b128(rsa, base, 0, 0);
        x.sxa_tail[T] = __builtin_amdgcn_raw_buffer_load_b32(rsa, base + 16, 0, 0);
        x.sxa_shift[T] = off & 3;
        // B: lane (i, g) loads the dword of columns c .. c+3 of the wave's WN
        // for K group 4kt + g (N is a multiple of 16), c = 4i; the step that
        // uses them hands each lane the bytes of the columns its fragment rows
        // feed (realign_mx; with WN = 32, lanes i >= 8 load a neighbour's
        // columns, unused).  The step's broadcasts give bank q of block j the
        // dword of lane 8 (j/2) + j%2 + 2q, which holds columns 32 (j/2) +
        // 4 (j%2) + 8q .. + 3 of a paired block (b_layout.h).  A lone block
        // j (the last of a group with an odd block count, rows in order; a
        // wave's block 0 or 2, or block 0 of a 32-column wave) needs columns
        // 16 j + 4q there instead: its four source lanes 4j + 2q load
        // column c = 2i + 8j, so that every step uses the same broadcasts.
        const int p = bl::group_blocks((n0 + C::WN * x.w) >> 6, x.N >> 4);
        const int lone = C::NBW == 4 ? ((p & 1) ? p - 1 : -1) : (2 * (x.w & 1) + 1 == p ? 0 : -1);
        const bool remap = lone >= 0 && (x.i & 1) == 0 && (x.i >> 3) == (lone >> 1);
        const int col = remap ? 2 * x.i + 8 * lone : 4 * x.i;
        const int boff = (4 * kt + x.g) * x.N + n0 + C::WN * x.w + col;
        x.sxb_raw[T] = __builtin_amdgcn_raw_buffer_load_b32(rsb, boff, 0, 0);
    } else if constexpr (kBlock<MODE>) {
        const __amdgpu_buffer_rsrc_t rsa = make_rsrc(x.sa, valid ? (uint32_t)x.KI * (uint32_t)x.M * 4u : 0u);
        const __amdgpu_buffer_rsrc_t rsb =
            make_rsrc(x.sb, valid ? (uint32_t)((x.N + 127) / 128) * (uint32_t)x.KI * 4u : 0u);
        // the MB consecutive rows MB i .. MB i + MB-1 of this lane: two
        // 16-byte loads (rows past M read the next K block's scales or, at
        // the end, zeros; their output is dropped)
        static_assert(C::MB == 8, "two 16-byte loads of A scales per lane");
        const int aoff = (kt * x.M + m0 + C::MB * x.i) * 4;
        x.sfa[T][0] = __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(rsa, aoff, 0, 0));
        x.sfa[T][1] = __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(rsa, aoff + 16, 0, 0));
        x.sfb[T] = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(rsb, (((n0 + C::WN * x.w) / 128) * x.KI + kt) * 4, 0, 0));
    }
}

// A whole B event at once (the prologue's).
template <int MODE, int T>
__device__ __forceinline__ void issue_b(Ctx<MODE>& x, TileRef r, int kt) {
    const __amdgpu_buffer_rsrc_t rb = b_rsrc(x, r.b_off, r.m0 >= 0);
    static_for<0, 2 * Cfg<MODE>::NBW>([&](auto Qc) { b_piece<MODE, T, decltype(Qc)::value>(x, rb, r.b_off, kt * 2048); });
    b_scales<MODE, T>(x, r, kt);
}

// ptpc epilogue scales of tile t: NSC = 2 DMAs per wave into the wave's own
// 2 KiB of g_lds_scale (a_scale of rows m0 .. m0+255, then b_scale of
// columns n0 .. n0+255; entries past M or N read as zero, and a tile past
// the end of the list moves nothing).
template <int MODE>
__device__ __forceinline__ void issue_epilogue_scales(Ctx<MODE>& x, TileRef t) {
    if constexpr (kPtpc<MODE>) {
        const bool valid = t.m0 >= 0;
        const int m0 = valid ? t.m0 : 0, n0 = valid ? t.n0 : 0;
        const __amdgpu_buffer_rsrc_t rsa = make_rsrc(x.sa, valid ? (uint32_t)x.M * 4u : 0u);
        const __amdgpu_buffer_rsrc_t rsb = make_rsrc(x.sb, valid ? (uint32_t)x.N * 4u : 0u);
        lds_char* dst = x.lds.scale + x.w * 2048;
        lds_dma16(rsa, dst, 4 * m0 + 16 * x.lane);
        lds_dma16(rsb, dst + 1024, 4 * n0 + 16 * x.lane);
    }
}

// Global -> LDS DMA of one A K tile: NA instructions per wave; instruction
// j moves 1 KiB (8 rows x 128 bytes).  a_off = the tile's A offset (where ra
// starts, see a_rsrc), kbase = 128 kt for K tile kt; rows past M fall
// outside the descriptor and read as zero.
template <int MODE>
__device__ __forceinline__ void a_piece(Ctx<MODE>& x, lds_char* stage, __amdgpu_buffer_rsrc_t ra, int a_off, int kbase,
                                        int j) {
    if constexpr (kTileRsrc<MODE>)
        lds_dma16(ra, stage + x.dma_lds + j * 1024, x.voff_a[j], __builtin_amdgcn_readfirstlane(kbase));
    else
        lds_dma16(ra, stage + x.dma_lds + j * 1024, x.voff_a[j] + a_off + kbase);
}

template <int MODE>
__device__ __forceinline__ void issue_a(Ctx<MODE>& x, lds_char* stage, TileRef r, int kt) {
    const __amdgpu_buffer_rsrc_t ra = a_rsrc(x, r.a_off, r.m0 >= 0);
#pragma unroll
    for (int j = 0; j < Cfg<MODE>::NA; ++j) a_piece<MODE>(x, stage, ra, r.a_off, kt * BK, j);
}

template <int MODE, int S>
__device__ __forceinline__ v8i read_a(const Ctx<MODE>& x, int mb) {
    const lds_char* st = x.lds.p[S];
    typedef __attribute__((address_space(3))) const v4i lds_v4i;
    v4i lo = *(lds_v4i*)(st + x.rd[mb & 1][0] + mb * 128);
    v4i hi = *(lds_v4i*)(st + x.rd[mb & 1][1] + mb * 128);
    return (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// ------------------------------------------------------------- compute
// The accumulators are pinned to AGPRs through inline asm: with all 256 of
// them in the 256 accumulation registers, the allocator has no reason to
// shuttle tuples through VGPRs.  Because the compiler cannot see that these
// statements are matrix ops, the two hazards they create are handled here:
// the first K tile of an output tile uses the zero-accumulator form (no
// register writes precede it), and the epilogue waits out the pipeline
// (mfma_drain) before it reads the results.
template <bool ZERO>
__device__ __forceinline__ void mfma_acc(v4f& acc, const v8i& b, const v8i& a) {
    if constexpr (ZERO) asm volatile("v_mfma_f32_16x16x128_f8f6f4 %0, %1, %2, 0" : "+a"(acc) : "v"(b), "v"(a));
    else asm volatile("v_mfma_f32_16x16x128_f8f6f4 %0, %1, %2, %0" : "+a"(acc) : "v"(b), "v"(a));
}

// The same with the accumulator in VGPRs (MODE_PTPC_N, MODE_PTPC_Q).
template <bool ZERO>
__device__ __forceinline__ void mfma_vacc(v4f& acc, const v8i& b, const v8i& a) {
    if constexpr (ZERO) asm volatile("v_mfma_f32_16x16x128_f8f6f4 %0, %1, %2, 0" : "=&v"(acc) : "v"(b), "v"(a));
    else asm volatile("v_mfma_f32_16x16x128_f8f6f4 %0, %1, %2, %0" : "+v"(acc) : "v"(b), "v"(a));
}

template <bool ZERO, int OA, int OB>
__device__ __forceinline__ void mfma_scaled_acc(v4f& acc, const v8i& b, const v8i& a, int sb, int sa) {
    if constexpr (ZERO)
        asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, 0, %3, %4 op_sel:[%5,%6,0] op_sel_hi:[%7,%8,0]"
                     : "+a"(acc)
                     : "v"(b), "v"(a), "v"(sb), "v"(sa), "n"(OA & 1), "n"(OB & 1), "n"(OA >> 1), "n"(OB >> 1));
    else
        asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel:[%5,%6,0] op_sel_hi:[%7,%8,0]"
                     : "+a"(acc)
                     : "v"(b), "v"(a), "v"(sb), "v"(sa), "n"(OA & 1), "n"(OB & 1), "n"(OA >> 1), "n"(OB >> 1));
}

// blockscale: acc[r][nb] (+)= bp[r % 2][nb] * s, s = sa(row, kt) * sb(block,
// kt).  The fp8 16x16x128 matrix op has 8 passes, so a VALU access to its
// result needs 11 wait states, which the compiler cannot see across the asm
// statements.  Column block nb of row block r is folded right after the
// matrix op (r + 1, nb), so that the four additions sit between matrix ops;
// PAD wait states of s_nop go in front, where the instructions counted
// since the matrix op that wrote the products fall short of 11 (mfma_row).
template <int PAD>
__device__ __forceinline__ void pad_wait_states() {
    static_assert(PAD >= 0 && PAD <= 16, "one or two s_nop");
    if constexpr (PAD > 8) asm volatile("s_nop 7\n\ts_nop %0" ::"n"(PAD - 9));
    else if constexpr (PAD > 0) asm volatile("s_nop %0" ::"n"(PAD - 1));
}

template <int MODE, int T, int r>
__device__ __forceinline__ float fold_scale(const Ctx<MODE>& x) {
    return x.sfa[T][r / 4][r % 4] * x.sfb[T];
}

template <int MODE, int r, int nb, bool FIRST, int PAD>
__device__ __forceinline__ void fold_block(Ctx<MODE>& x, float s) {
    v4f& c = x.acc[r][nb];
    const v4f p = x.bp[r & 1][nb];
    pad_wait_states<PAD>();
    if constexpr (FIRST)
        asm volatile("v_mul_f32 %0, %4, %8\n\tv_mul_f32 %1, %5, %8\n\tv_mul_f32 %2, %6, %8\n\tv_mul_f32 %3, %7, %8"
                     : "=&v"(c[0]), "=&v"(c[1]), "=&v"(c[2]), "=&v"(c[3])
                     : "v"(p[0]), "v"(p[1]), "v"(p[2]), "v"(p[3]), "v"(s));
    else
        asm volatile("v_fmac_f32 %0, %4, %8\n\tv_fmac_f32 %1, %5, %8\n\tv_fmac_f32 %2, %6, %8\n\tv_fmac_f32 %3, %7, %8"
                     : "+v"(c[0]), "+v"(c[1]), "+v"(c[2]), "+v"(c[3])
                     : "v"(p[0]), "v"(p[1]), "v"(p[2]), "v"(p[3]), "v"(s));
}

// Block (mb, nb) of a K tile, ptpc / mxfp8 (AGPR accumulators).
template <int MODE, int T, int mb, int nb, bool FIRST>
__device__ __forceinline__ void mfma_block(Ctx<MODE>& x, const v8i& a) {
    if constexpr (kWidePtpc<MODE>) {
        mfma_acc<FIRST>(x.acc[mb][nb], x.bq[T][nb], a);
    } else if constexpr (MODE == MODE_MXFP8) {
        // src1 (A) scale: byte mb % 4 of word mb / 4 of the realigned bytes;
        // src0 (B) scale: byte 0 of the block's register
        mfma_scaled_acc<FIRST, 0, mb % 4>(x.acc[mb][nb], x.bq[T][nb], a, x.sxb[nb], x.sxa[T][mb / 4]);
    } else {
        static_assert(MODE == MODE_MXFP8_N, "blockscale issues its row blocks as a whole");
        mfma_scaled_acc<FIRST, 0, mb % 4>(x.acc[mb][nb], x.bq[T][nb], a, x.sxb[nb], x.sxa[T][mb / 4]);
    }
}

template <int MODE, int T, int mb, bool FIRST>
__device__ __forceinline__ void mfma_row(Ctx<MODE>& x, const v8i& a) {
    if constexpr (kWidePtpc<MODE> || kMx<MODE>) {
        static_for<0, Cfg<MODE>::NBW>([&](auto NBc) { mfma_block<MODE, T, mb, decltype(NBc)::value, FIRST>(x, a); });
    } else if constexpr (kNarrowPtpc<MODE>) {
        // each accumulator is rewritten once per K tile, 2 MB - 1 matrix ops
        // after its last write: far past the result latency
        mfma_vacc<FIRST>(x.acc[mb][0], x.bq[T][0], a);
        mfma_vacc<FIRST>(x.acc[mb][1], x.bq[T][1], a);
    } else {
        // blockscale: one fp32 scale per (row, 128-wide K tile) times the
        // B block's scale multiplies each K tile's products before they are
        // added to the VGPR accumulators.  The products of row block mb go
        // to bp[mb % 2]; column block nb of row block mb - 1 is scaled in
        // right behind the matrix op (mb, nb), the last row block's after
        // its own.  Wait states from the matrix op (r, nb) to the fold (r,
        // nb), one per instruction in between plus the fold's own padding:
        //   fold (0, 0): two matrix ops + 9 = 11;
        //   fold (r, 0), r >= 1: fold (r-1, 0) (padding >= 1, four
        //     additions), a matrix op, fold (r-1, 1) (4), a matrix op, + 1
        //     = 12 or more;
        //   fold (r, 1): fold (r-1, 1) (4; none for r = 0), a matrix op,
        //     fold (r, 0) (1 + 4 or 9 + 4), a matrix op = 11 or more;
        //   last row block: fold (7, 0) 5 + 1 + 4 + 1 = 11, fold (7, 1)
        //     4 + 5 + 2 = 11.
        // Anything the compiler puts in between only adds to these
        // (tests/test_isa_hazards.py audits the emitted code).
        static_assert(Cfg<MODE>::NBW == 2, "two column blocks per wave");
        constexpr int MB = Cfg<MODE>::MB;
        asm volatile("v_mfma_f32_16x16x128_f8f6f4 %0, %1, %2, 0" : "=&v"(x.bp[mb & 1][0]) : "v"(x.bq[T][0]), "v"(a));
        if constexpr (mb > 0) fold_block<MODE, mb - 1, 0, FIRST, mb == 1 ? 9 : 1>(x, fold_scale<MODE, T, mb - 1>(x));
        asm volatile("v_mfma_f32_16x16x128_f8f6f4 %0, %1, %2, 0" : "=&v"(x.bp[mb & 1][1]) : "v"(x.bq[T][1]), "v"(a));
        if constexpr (mb > 0) fold_block<MODE, mb - 1, 1, FIRST, 0>(x, fold_scale<MODE, T, mb - 1>(x));
        if constexpr (mb == MB - 1) {
            fold_block<MODE, mb, 0, FIRST, 1>(x, fold_scale<MODE, T, mb>(x));
            fold_block<MODE, mb, 1, FIRST, 2>(x, fold_scale<MODE, T, mb>(x));
        }
    }
}

// Before the epilogue reads accumulators written by the asm matrix ops:
// 32 wait states cover the longest result latency of the 16x16x128 op, and
// the empty asm statements (ordered after the wait like all volatile asm)
// make every later read of an accumulator depend on it.
template <int MODE>
__device__ __forceinline__ void mfma_drain(Ctx<MODE>& x) {
    if constexpr (!kBlock<MODE>) {
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
        for (int mb = 0; mb < Cfg<MODE>::MB; ++mb)
#pragma unroll
            for (int nb = 0; nb < Cfg<MODE>::NBW; ++nb) {
                if constexpr (kAgprAcc<MODE>) asm volatile("" : "+a"(x.acc[mb][nb]));
                else asm volatile("" : "+v"(x.acc[mb][nb]));
            }
    }
}

// Within each 16-lane row, lane 4q + t (bank q) receives the value of lane
// src(q): four row broadcasts, each written to one bank of four lanes.
template <int S0, int S1, int S2, int S3>
__device__ __forceinline__ int row_gather4(int src) {
    int x = 0;
    x = __builtin_amdgcn_update_dpp(x, src, kDppRowNewBcast + S0, 0xF, 0x1, false);
    x = __builtin_amdgcn_update_dpp(x, src, kDppRowNewBcast + S1, 0xF, 0x2, false);
    x = __builtin_amdgcn_update_dpp(x, src, kDppRowNewBcast + S2, 0xF, 0x4, false);
    x = __builtin_amdgcn_update_dpp(x, src, kDppRowNewBcast + S3, 0xF, 0x8, false);
    return x;
}

// Start of a step's mxfp8 scales: realign the 20 loaded A-scale bytes so word
// q holds the bytes of rows 4q..4q+3, and give lane (i, g) the B-scale byte
// of the column its fragment row i feeds in each block (b_layout.h), which
// lane (src, g) loaded as byte i % 4 of its dword: for the wave's block j and
// bank q = i / 4, src = 8 (j / 2) + 2q + j % 2 (b_scales chose what each
// source lane loads, lone blocks included).  DPP row broadcasts: vector ops,
// where an LDS crossbar permute would cost matrix time.
template <int MODE, int T>
__device__ __forceinline__ void realign_mx(Ctx<MODE>& x) {
    if constexpr (kMx<MODE>) {
        const int sh = x.sxa_shift[T];
        if (sh) {
            const v4i w = x.sxa[T];
            const int t = x.sxa_tail[T];
            // alignbyte(hi, lo, s) = bytes s..s+3 of the 64-bit hi:lo
            x.sxa[T] = (v4i){(int)__builtin_amdgcn_alignbyte(w[1], w[0], sh), (int)__builtin_amdgcn_alignbyte(w[2], w[1], sh),
                             (int)__builtin_amdgcn_alignbyte(w[3], w[2], sh), (int)__builtin_amdgcn_alignbyte(t, w[3], sh)};
        }
        const int byte = 8 * (x.i & 3);
        const int raw = x.sxb_raw[T];
        static_for<0, Cfg<MODE>::NBW>([&](auto Jc) {
            constexpr int j = decltype(Jc)::value;
            constexpr int b = 8 * (j / 2) + (j % 2);
            x.sxb[j] = (int)((uint32_t)row_gather4<b, b + 2, b + 4, b + 6>(raw) >> byte);
        });
    }
}

// ------------------------------------------------------------ epilogue
// Result lane l, register v of block (mb, nb) holds row MB (l % 16) + mb of
// the tile and the output column that B-fragment row 4 (l / 16) + v of the
// block feeds (b_layout.h): in a full group, lane (i, g) holds columns
// 8g .. 8g + 7 of its wave's 64 in blocks 0-1 and 32 + 8g .. 32 + 8g + 7 in
// blocks 2-3 (a 32-column wave: 8g .. 8g + 7 in its two blocks), so after the
// bf16 conversion each run is one 16-byte store and the four lanes of a row
// write 64 contiguous bytes.  A lone block (the odd last block of the last
// group when N % 64 is 16 or 48) holds columns 16 nb + 4g .. + 3 and leaves
// in an 8-byte store.  Rows at or past M fall outside the C descriptor;
// runs at or past N carry 2^31 on their offset and fall outside it too.
//
// ptpc and mxfp8 (accumulators in AGPRs) spread a tile's epilogue over two
// K steps, so that its conversion work and its stores overlap matrix ops
// instead of piling up between them.  With two or more K tiles per tile:
//   * the tile's last K step stores row blocks 0..7, each as soon as its
//     final matrix ops are done: row block r in eight phases, one after each
//     matrix op of row blocks 2r+1 and 2r+2 (row block 7's second half after
//     the step's last matrix op);
//   * the next tile's first K step stores row blocks 8..15, each before
//     that step's matrix ops overwrite its accumulators: row block r after
//     the matrix ops of row blocks 2(r-8) and 2(r-8)+1.
// With one K tile per tile both halves would land in the same step, so
// there the whole tile is stored in the next tile's first step, each row
// block just ahead of the matrix ops that overwrite it.  The workgroup's
// last rows are stored after its loop.  Blockscale and the other 32-column
// waves store each tile at its end.

constexpr uint32_t kDrop = 0x80000000u;

// Start the epilogue of the tile at (m0, n0): the store offsets and, for
// ptpc, the scales.  ptpc reads its scales from this wave's LDS region,
// where the scale DMAs (issue_epilogue_scales) put them: in the previous
// tile's last step or the prologue, or, with one K tile per tile, earlier in
// the same or the previous step.  Every such DMA was followed by at least
// the NA A-tile DMAs of a step (and possibly by stores), so vmcnt(NA) covers
// it; each wave reads only the region it filled.  The reads are written out
// so that the compiler, which cannot tell the A-tile DMAs still in flight
// from writes to this region, does not drain the whole prefetch pipeline
// (vmcnt(0)) before them.
template <int MODE>
__device__ __forceinline__ Epi epi_begin(Ctx<MODE>& x, int m0, int n0) {
    using C = Cfg<MODE>;
    Epi e;
    // the wave's first column, its group's block count, and the byte
    // offset of row MB i (this lane's row in row block 0) at that column
    const int wc = n0 + C::WN * x.w;
    const int p = bl::group_blocks(wc >> 6, x.N >> 4);
    const uint32_t base = (uint32_t)(((m0 + C::MB * x.i) * x.N + wc) * 2);
    if constexpr (C::NBW == 4) {
        e.o16[0] = base + 16 * x.g + (p >= 2 ? 0u : kDrop);       // blocks 0-1: columns 8g ..
        e.o16[1] = base + 64 + 16 * x.g + (p == 4 ? 0u : kDrop);  // blocks 2-3: columns 32 + 8g ..
        e.lone = p & 1;                                           // block p - 1 is lone
        e.o8 = base + 32 * (p - 1) + 8 * x.g + (p & 1 ? 0u : kDrop);
    } else {
        // the wave holds blocks 2 (w % 2) and 2 (w % 2) + 1 of its group
        const int first = 2 * (x.w & 1);
        e.o16[0] = base + 16 * x.g + (first + 2 <= p ? 0u : kDrop);
        e.o16[1] = kDrop;
        e.lone = first + 1 == p;
        e.o8 = base + 8 * x.g + (first + 1 == p ? 0u : kDrop);
    }
    if constexpr (kNarrowPtpc<MODE>) {
        // rows MB i .. MB i + 7; columns 8g + 4j + v of the wave's 32 (a lone
        // block: 4g + v)
        static_assert(C::MB == 8 && C::NBW == 2, "two A- and two B-scale vectors");
        wait_vm<C::NA>();
        const uint32_t sc = (uint32_t)(uintptr_t)(x.lds.scale + x.w * 2048);
        const uint32_t pa = sc + C::MB * x.i * 4;
        const uint32_t pb = sc + 1024 + (C::WN * x.w + (e.lone ? 4 : 8) * x.g) * 4;
        asm volatile(
            "ds_read_b128 %0, %4\n"
            "ds_read_b128 %1, %4 offset:16\n"
            "ds_read_b128 %2, %5\n"
            "ds_read_b128 %3, %5 offset:16\n"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(e.eas[0]), "=&v"(e.eas[1]), "=&v"(e.ebs[0]), "=&v"(e.ebs[1])
            : "v"(pa), "v"(pb)
            : "memory");
    }
    if constexpr (kWidePtpc<MODE>) {
        // rows MB i .. MB i + 15; block nb's columns 8g + {0, 4, 32, 36}[nb] + v
        // of the wave's 64 (a lone block nb: 16 nb + 4g + v)
        static_assert(C::MB == 16 && C::NBW == 4, "ptpc epilogue reads four A- and four B-scale vectors");
        wait_vm<C::NA>();
        const uint32_t sc = (uint32_t)(uintptr_t)(x.lds.scale + x.w * 2048);
        const uint32_t pa = sc + C::MB * x.i * 4, pb = sc + 1024 + (C::WN * x.w + 8 * x.g) * 4;
        const uint32_t pl = sc + 1024 + (C::WN * x.w + 16 * (p - 1) + 4 * x.g) * 4;
        v4f lone;
        asm volatile(
            "ds_read_b128 %0, %9\n"
            "ds_read_b128 %1, %9 offset:16\n"
            "ds_read_b128 %2, %9 offset:32\n"
            "ds_read_b128 %3, %9 offset:48\n"
            "ds_read_b128 %4, %10\n"
            "ds_read_b128 %5, %10 offset:16\n"
            "ds_read_b128 %6, %10 offset:128\n"
            "ds_read_b128 %7, %10 offset:144\n"
            "ds_read_b128 %8, %11\n"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(e.eas[0]), "=&v"(e.eas[1]), "=&v"(e.eas[2]), "=&v"(e.eas[3]), "=&v"(e.ebs[0]),
              "=&v"(e.ebs[1]), "=&v"(e.ebs[2]), "=&v"(e.ebs[3]), "=&v"(lone)
            : "v"(pa), "v"(pb), "v"(p > 0 ? pl : pb)
            : "memory");
        // a lone block (p odd) is block 0 or 2
        if (p == 1) e.ebs[0] = lone;
        if (p == 3) e.ebs[2] = lone;
    }
    return e;
}

// One row block's epilogue (ptpc, mxfp8) in eight phases, so that it can be
// spread over eight matrix ops:
//   0, 1  read the accumulators of column-block pair 0 / 1
//   2..5  ptpc scaling, pair (PH - 2) / 2, first / second block of the pair
//   6     bf16 conversion of both pairs
//   7     the stores
struct EpiRow {
    v4f u[2], v[2];
    v4i d[2];
};

template <int MODE, int r, int PH>
__device__ __forceinline__ void epi_phase(Ctx<MODE>& x, const Epi& e, EpiRow& q) {
    using C = Cfg<MODE>;
    static_assert(kDeferEpilogue<MODE> && C::NBW == 4, "AGPR accumulators, two block pairs per wave");
    if constexpr (PH < 2) {
        // explicit reads, so that the register allocator keeps each
        // accumulator where the next tile's matrix ops will write it
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(q.u[PH][c]) : "a"(x.acc[r][2 * PH][c]));
            asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(q.v[PH][c]) : "a"(x.acc[r][2 * PH + 1][c]));
        }
    } else if constexpr (PH < 6) {
        if constexpr (kWidePtpc<MODE>) {
            constexpr int pair = (PH - 2) / 2;
            const float sa = e.eas[r / 4][r % 4];
            if constexpr (PH % 2 == 0) q.u[pair] = q.u[pair] * sa * e.ebs[2 * pair];
            else q.v[pair] = q.v[pair] * sa * e.ebs[2 * pair + 1];
        }
    } else if constexpr (PH == 6) {
#pragma unroll
        for (int pair = 0; pair < 2; ++pair)
            q.d[pair] = (v4i){pack_bf16(q.u[pair][0], q.u[pair][1]), pack_bf16(q.u[pair][2], q.u[pair][3]),
                              pack_bf16(q.v[pair][0], q.v[pair][1]), pack_bf16(q.v[pair][2], q.v[pair][3])};
    } else {
        // C is written once and never read back: non-temporal stores, with
        // device scope as well when K is short (kStoreNt, kStoreNtSc1)
        const __amdgpu_buffer_rsrc_t rc = make_rsrc(x.c, (uint32_t)x.M * (uint32_t)x.N * 2u);
        const uint32_t ro = (uint32_t)(r * x.N * 2);
        // the lone block is block 0 (then run 0 is dropped) or block 2
        const v4i& d = e.o16[0] < kDrop ? q.d[1] : q.d[0];
        if (x.nt_only) {
            __builtin_amdgcn_raw_buffer_store_b128(q.d[0], rc, e.o16[0] + ro, 0, kStoreNt);
            __builtin_amdgcn_raw_buffer_store_b128(q.d[1], rc, e.o16[1] + ro, 0, kStoreNt);
            if (e.lone) __builtin_amdgcn_raw_buffer_store_b64((v2i){d[0], d[1]}, rc, e.o8 + ro, 0, kStoreNt);
        } else {
            __builtin_amdgcn_raw_buffer_store_b128(q.d[0], rc, e.o16[0] + ro, 0, kStoreNtSc1);
            __builtin_amdgcn_raw_buffer_store_b128(q.d[1], rc, e.o16[1] + ro, 0, kStoreNtSc1);
            if (e.lone) __builtin_amdgcn_raw_buffer_store_b64((v2i){d[0], d[1]}, rc, e.o8 + ro, 0, kStoreNtSc1);
        }
    }
}

template <int MODE, int r, int PH = 0>
__device__ __forceinline__ void epi_phases(Ctx<MODE>& x, const Epi& e, EpiRow& q) {
    if constexpr (PH < 8) {
        epi_phase<MODE, r, PH>(x, e, q);
        epi_phases<MODE, r, PH + 1>(x, e, q);
    }
}

// Scale, convert and store row block mb of the tile whose accumulators are
// live.
template <int MODE, int mb>
__device__ __forceinline__ void epi_row(Ctx<MODE>& x, const Epi& e) {
    using C = Cfg<MODE>;
    if constexpr (kDeferEpilogue<MODE>) {
        EpiRow q;
        epi_phases<MODE, mb>(x, e, q);
    } else {
        // blockscale, narrow ptpc: one block pair per wave, accumulators
        // in VGPRs
        static_assert(C::NBW == 2, "one block pair per wave");
        const __amdgpu_buffer_rsrc_t rc = make_rsrc(x.c, (uint32_t)x.M * (uint32_t)x.N * 2u);
        v4f u = x.acc[mb][0], v = x.acc[mb][1];
        if constexpr (kNarrowPtpc<MODE>) {
            const float sa = e.eas[mb / 4][mb % 4];
            u = u * sa * e.ebs[0];
            v = v * sa * e.ebs[1];
        }
        // the wave's two blocks (columns 8g .. 8g + 7), or its lone block 0
        // (columns 4g .. 4g + 3); the neighbouring wave writes the other
        // half of each 128-byte segment, so these stores go through the L2,
        // which merges the halves
        const v4i d = (v4i){pack_bf16(u[0], u[1]), pack_bf16(u[2], u[3]), pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
        const uint32_t ro = (uint32_t)(mb * x.N * 2);
        __builtin_amdgcn_raw_buffer_store_b128(d, rc, e.o16[0] + ro, 0, 0);
        if (e.lone) __builtin_amdgcn_raw_buffer_store_b64((v2i){d[0], d[1]}, rc, e.o8 + ro, 0, 0);
    }
}

// The whole epilogue of a tile at once.
template <int MODE, int mb = 0>
__device__ __forceinline__ void epi_rows(Ctx<MODE>& x, const Epi& e) {
    if constexpr (mb < Cfg<MODE>::MB) {
        epi_row<MODE, mb>(x, e);
        // keep the scheduler from hoisting every accumulator read of the
        // epilogue at once (the next tile's loads are live here)
        if constexpr ((mb & 1) == 1) __builtin_amdgcn_sched_barrier(0);
        epi_rows<MODE, mb + 1>(x, e);
    }
}

template <int MODE>
__device__ __forceinline__ void store_tile(Ctx<MODE>& x, int m0, int n0) {
    epi_rows<MODE>(x, epi_begin<MODE>(x, m0, n0));
}


// ---------------------------------------------------------------- step
// Origins and operand extents of tiles j, j+1, j+2 of the list, rotated as
// the stream advances: loads run up to two tiles ahead of the one computed.
struct Ring {
    TileRef t0, t1, t2;
};

// Where one stream step's loads go: the B event of step s+1 and the A DMA of
// step s+3 (K tile k+3 of this tile or of one of the next two).
struct StepLoads {
    __amdgpu_buffer_rsrc_t rb, ra;
    int bbase, abase;  // K-tile byte offsets of the B event and the A DMA within their tiles
    int boff, aoff;    // their tiles' B and A offsets
    int bkt;           // K tile of the B event (for the mode's scales)
    TileRef bref;
    TileRef enext;     // the next tile, whose epilogue scales a tile's last step loads
};

// The middle of a step.  RAW: K tile s+1 has landed in every wave's share of
// LDS.  WAR: every wave's reads of stage (S+3)%4 (stream step s-1) have
// retired, so the A DMAs that follow may refill it.  The count is
// sched::wait_at(s, k, KI, ...), specialised (FIRST && LAST is KI == 1):
// only the stream's very first step (HEAD: the first K step of the
// workgroup's first tile, s = 0) differs from the rest of its kind.  Every
// count is a compile-time constant, so each barrier has exactly one wait in
// front of it on every path through the code.
template <int MODE, int S, bool FIRST, bool LAST, bool HEAD>
__device__ __forceinline__ void mid_step() {
    using C = Cfg<MODE>;
    constexpr int NA = C::NA, NB = C::NB, NSC = C::NSC;
    constexpr int XT = FIRST && LAST ? 2 : FIRST ? 1 : 0;
    static_assert(!HEAD || FIRST, "the stream starts with a tile's first K step");
    if constexpr (HEAD) wait_vm_lgkm0<sched::cap(sched::first_mid_wait(NA, NB) + (LAST ? NSC : 0))>();
    else wait_vm_lgkm0<sched::cap(sched::mid_wait(NA, NB) + XT * NSC)>();
    __builtin_amdgcn_s_barrier();
}

// The four matrix ops of row block mb, each followed by one phase of the
// epilogue of row block r (phases PH0 .. PH0+3).  With R0 (the first phase
// of a row block whose final matrix ops ran earlier in this step) the
// accumulator reads wait out the matrix-op result latency: the compiler
// cannot see that hazard across the asm statements.
template <int MODE, int T, int mb, bool FIRST, int r, int PH0, bool R0>
__device__ __forceinline__ void mfma_row_epi(Ctx<MODE>& x, const v8i& a, EpiRow& q) {
    static_for<0, 4>([&](auto NBc) {
        constexpr int nb = decltype(NBc)::value;
        mfma_block<MODE, T, mb, nb, FIRST>(x, a);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (R0 && nb == 0) asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" ::: "memory");
        epi_phase<MODE, r, PH0 + nb>(x, x.ep, q);
        __builtin_amdgcn_sched_barrier(0);
    });
}

// Row blocks mb .. MB-1 of a step; each row block's four matrix ops are
// separated by at most a few other instructions:
// - A fragments run two row blocks ahead through a three-deep register ring
//   (f0, f1, f2 hold fragments = 0, 1, 2 mod 3): fragment mb + 2 is read
//   while mb's matrix ops run.  Reads of this step's stage S need no barrier
//   (the previous step's covered its tile); the next stage's first two
//   fragments, read in the last two row blocks, come after this step's
//   barrier.
// - The next B event is spread over the first half (2 NBW / (MB/2) fragment
//   loads per row block, then the mode's scales and, with one K tile per
//   tile, this tile's epilogue scale DMAs); the wait + barrier sits at MB/2,
//   followed in a tile's last step (two or more K tiles per tile) by the
//   next tile's epilogue scale DMAs; the NA A DMAs of step s+3 follow,
//   spread evenly over the second half.  The order of the loads relative to
//   the wait is the one sched::wait_at counts.
// - EPM, the epilogue carried by the step (ptpc, mxfp8): 0 none; 1 the whole
//   previous tile, each row block just ahead of its matrix ops (one K tile
//   per tile); 2 row blocks 8..15 of the previous tile (first K step);
//   3 row blocks 0..7 of this tile (last K step).
template <int MODE, int S, bool FIRST, bool LAST, bool HEAD, int EPM, int mb>
__device__ __forceinline__ void step_rows(Ctx<MODE>& x, TileRef cur, StepLoads L, EpiRow& q, v8i& f0, v8i& f1,
                                          v8i& f2) {
    using C = Cfg<MODE>;
    if constexpr (mb < C::MB) {
        constexpr int T = S & 1;
        constexpr int SR = (S + 3) & 3;  // stage refilled by this step (tile k-1's)
        constexpr int SN = (S + 1) & 3;  // stage of the next K tile
        constexpr int HALF = C::MB / 2;
        // the 2 NBW B fragment loads of the event, spread over the first
        // half: BPR per row block, or one per BSTRIDE row blocks
        constexpr int NBL = 2 * C::NBW;
        constexpr int BPR = NBL >= HALF ? NBL / HALF : 1;
        constexpr int BSTRIDE = NBL >= HALF ? 1 : HALF / NBL;
        static_assert((BPR == 1 || BPR == 2) && BPR * HALF == NBL * BSTRIDE,
                      "every B fragment load of the event, spread over the first half");
        constexpr int nxt = mb + 2;
        if constexpr (mb < HALF) {
            if constexpr (mb % BSTRIDE == 0) {
                b_piece<MODE, T ^ 1, mb / BSTRIDE * BPR>(x, L.rb, L.boff, L.bbase);
                if constexpr (BPR == 2) b_piece<MODE, T ^ 1, mb * BPR + 1>(x, L.rb, L.boff, L.bbase);
            }
            if constexpr (mb == HALF - 1) {
                b_scales<MODE, T ^ 1>(x, L.bref, L.bkt);
                if constexpr (FIRST && LAST && kPtpc<MODE>) {
                    // after the whole B event, as the wait counts assume
                    __builtin_amdgcn_sched_barrier(0);
                    issue_epilogue_scales<MODE>(x, cur);
                }
            }
        }
        if constexpr (mb == HALF) {
            mid_step<MODE, S, FIRST, LAST, HEAD>();
            if constexpr (LAST && !FIRST) issue_epilogue_scales<MODE>(x, L.enext);
        }
        // NA DMAs spread over the second half, the first at mb = HALF
        static_assert(C::NA <= HALF && HALF % C::NA == 0, "A DMAs spread evenly over the second half");
        constexpr int DSTRIDE = HALF / C::NA;
        if constexpr (mb >= HALF && (mb - HALF) % DSTRIDE == 0)
            a_piece<MODE>(x, x.lds.p[SR], L.ra, L.aoff, L.abase, (mb - HALF) / DSTRIDE);
        if constexpr (nxt < C::MB) {
            v8i fr = read_a<MODE, S>(x, nxt);
            if constexpr (nxt % 3 == 0) f0 = fr;
            else if constexpr (nxt % 3 == 1) f1 = fr;
            else f2 = fr;
        } else {
            x.pre[nxt - C::MB] = read_a<MODE, SN>(x, nxt - C::MB);
        }
        const v8i& fa = mb % 3 == 0 ? f0 : mb % 3 == 1 ? f1 : f2;
        if constexpr (EPM == 1) {
            // the previous tile's row block mb, read out before this step's
            // matrix ops overwrite its accumulators (the fences keep the
            // reads ahead of them and this row block's work together)
            __builtin_amdgcn_sched_barrier(0);
            epi_row<MODE, mb>(x, x.ep);
            __builtin_amdgcn_sched_barrier(0);
            mfma_row<MODE, T, mb, FIRST>(x, fa);
        } else if constexpr (EPM == 2) {
            // row block 8 + mb/2 of the previous tile: its reads (phases
            // 0, 1) come before this step's matrix ops of that row block
            mfma_row_epi<MODE, T, mb, FIRST, 8 + mb / 2, 4 * (mb % 2), false>(x, fa, q);
        } else if constexpr (EPM == 3 && mb > 0) {
            // row block (mb-1)/2 of this tile, final since row block
            // (mb-1)/2's matrix ops earlier in this step
            mfma_row_epi<MODE, T, mb, FIRST, (mb - 1) / 2, 4 * (1 - mb % 2), mb % 2 == 1>(x, fa, q);
        } else {
            mfma_row<MODE, T, mb, FIRST>(x, fa);
        }
        step_rows<MODE, S, FIRST, LAST, HEAD, EPM, mb + 1>(x, cur, L, q, f0, f1, f2);
    } else if constexpr (EPM == 3) {
        // the second half of row block 7 (MB = 16)
        static_assert(Cfg<MODE>::MB == 16, "row blocks 0..7 of 16 in the last K step");
        __builtin_amdgcn_sched_barrier(0);
        epi_phase<MODE, 7, 4>(x, x.ep, q);
        epi_phase<MODE, 7, 5>(x, x.ep, q);
        epi_phase<MODE, 7, 6>(x, x.ep, q);
        epi_phase<MODE, 7, 7>(x, x.ep, q);
    }
}

// Stream step s = K tile k of tile j.  S = s % 4 is the LDS stage of the
// tile, T = s % 2 the B register buffer.  FIRST / LAST: k == 0 / k == KI-1
// (both for KI == 1).  PREV: a tile precedes this one in the workgroup's
// list, so a first K step also stores (part of) it.  HEAD: s == 0.
template <int MODE, int S, bool FIRST, bool LAST, bool PREV = false, bool HEAD = false>
__device__ __forceinline__ void kstep(Ctx<MODE>& x, int s, int k, Ring g, TileRef prev = TileRef{}) {
    static_assert(!PREV || FIRST, "the previous tile's epilogue runs in the first K step");
    static_assert(!(PREV && HEAD), "the stream's first tile has no predecessor");
    constexpr int EPM = !kDeferEpilogue<MODE> ? 0
                        : FIRST && LAST       ? (PREV ? 1 : 0)
                        : FIRST               ? (PREV ? 2 : 0)
                        : LAST                ? 3
                                              : 0;
    constexpr int T = S & 1;
    const int KI = x.KI;
    StepLoads L;
    // B event of stream step s+1: the next K tile, or the next tile's first
    L.bref = LAST ? g.t1 : g.t0;
    L.bkt = LAST ? 0 : k + 1;
    L.rb = b_rsrc(x, L.bref.b_off, L.bref.m0 >= 0);
    L.boff = L.bref.b_off;
    L.bbase = L.bkt * 2048;
    L.enext = g.t1;
    // A DMA of stream step s+3: K tile k+3 of this tile or of one of the next
    // two (selected without branches) -- or, when K = 128 (every step both
    // the first and the last of its tile, s = j), K tile 0 of tile j + 3
    int a_off, a_m0, akt;
    if constexpr (FIRST && LAST) {
        const TileRef t3 = x.ref(s + 3);
        a_off = t3.a_off;
        a_m0 = t3.m0;
        akt = 0;
    } else {
        // sched::dma_ahead_tile(k, KI) (0, 1 or 2 for KI >= 2) and
        // sched::dma_ahead_kt(k, KI), as two comparisons and selects
        const int kk = k + 3;
        const bool in0 = kk < KI, in1 = kk < 2 * KI;
        a_off = g.t2.a_off;
        a_m0 = g.t2.m0;
        akt = kk - 2 * KI;
        a_off = in1 ? g.t1.a_off : a_off;
        a_m0 = in1 ? g.t1.m0 : a_m0;
        akt = in1 ? kk - KI : akt;
        a_off = in0 ? g.t0.a_off : a_off;
        a_m0 = in0 ? g.t0.m0 : a_m0;
        akt = in0 ? kk : akt;
    }
    L.ra = a_rsrc(x, a_off, a_m0 >= 0);
    L.aoff = a_off;
    L.abase = akt * BK;
    if constexpr (EPM == 1) x.ep = epi_begin<MODE>(x, prev.m0, prev.n0);
    // the tile's scales leave LDS before this step's wait lets the next
    // tile's scale DMAs in (the narrow tile stores at the end of the step)
    if constexpr (EPM == 3 || (kNarrowPtpc<MODE> && LAST && !FIRST)) x.ep = epi_begin<MODE>(x, g.t0.m0, g.t0.n0);
    realign_mx<MODE, T>(x);
    v8i f0 = x.pre[0], f1 = x.pre[1], f2;
    EpiRow q;
    step_rows<MODE, S, FIRST, LAST, HEAD, EPM, 0>(x, g.t0, L, q, f0, f1, f2);
}

// All K tiles of tile j, whose first K tile sits in stage P.  CASE = KI % 4
// for KI >= 2, or 4 for KI == 1, is a compile-time constant of the kernel:
// the first and last steps are peeled, the KI - 2 middle steps run as whole
// groups of four plus exactly (CASE - 2) & 3 more, so every stage index and
// every wait count is a constant.  PREV: the first step also stores tile
// j - 1 (prev); without a deferred epilogue the tile stores itself at its end.
// HEAD: the workgroup's first tile (s0 = 0).
template <int MODE, int P, int CASE, bool PREV, bool HEAD>
__device__ __forceinline__ void tile_body(Ctx<MODE>& x, int s0, Ring g, TileRef prev) {
    const int KI = x.KI;
    if constexpr (CASE == 4) {
        kstep<MODE, P, true, true, PREV, HEAD>(x, s0, 0, g, prev);
    } else {
        constexpr int REM = (CASE - 2) & 3;  // (KI - 2) % 4
        kstep<MODE, P, true, false, PREV, HEAD>(x, s0, 0, g, prev);
        int k = 1;
        for (; k + 4 <= KI - 1; k += 4) {
            kstep<MODE, (P + 1) & 3, false, false>(x, s0 + k, k, g);
            kstep<MODE, (P + 2) & 3, false, false>(x, s0 + k + 1, k + 1, g);
            kstep<MODE, (P + 3) & 3, false, false>(x, s0 + k + 2, k + 2, g);
            kstep<MODE, (P + 0) & 3, false, false>(x, s0 + k + 3, k + 3, g);
        }
        if constexpr (REM >= 1) kstep<MODE, (P + 1) & 3, false, false>(x, s0 + k, k, g);
        if constexpr (REM >= 2) kstep<MODE, (P + 2) & 3, false, false>(x, s0 + k + 1, k + 1, g);
        if constexpr (REM >= 3) kstep<MODE, (P + 3) & 3, false, false>(x, s0 + k + 2, k + 2, g);
        kstep<MODE, (P + CASE - 1) & 3, false, true>(x, s0 + KI - 1, KI - 1, g);
    }
    if constexpr (!kDeferEpilogue<MODE>) {
        mfma_drain<MODE>(x);
        if constexpr (kNarrowPtpc<MODE> && CASE != 4) epi_rows<MODE>(x, x.ep);
        else store_tile<MODE>(x, g.t0.m0, g.t0.n0);
    }
}

template <int MODE, int P, int CASE, bool PREV>
__device__ __forceinline__ void run_tile(Ctx<MODE>& x, int j, Ring& g, TileRef& prev) {
    tile_body<MODE, P, CASE, PREV && kDeferEpilogue<MODE>, !PREV>(x, j * x.KI, g, prev);
    prev = g.t0;
    g = Ring{g.t1, g.t2, x.ref(j + 3)};
}

// -------------------------------------------------------------- kernel
// CASE = (K / 128) % 4 (4 when K == 128): the LDS stage of a tile's first K
// tile advances by KI % 4 from one tile to the next, so tiles come in
// cycles of 1, 2 or 4 phases.
template <int MODE, int CASE>
__global__ void __launch_bounds__(Cfg<MODE>::NTHREADS, 1) gemm_a8w8_kernel(GemmArgs p) {
    using C = Cfg<MODE>;
    Ctx<MODE> x;
    x.lds = Stages{{(lds_char*)g_lds_a0, (lds_char*)g_lds_a1, (lds_char*)g_lds_a2, (lds_char*)g_lds_a3},
                   (lds_char*)g_lds_scale};
    x.a = p.a;
    x.b = p.b;
    x.sa = p.sa;
    x.sb = p.sb;
    x.c = p.c;
    x.M = p.m;
    x.N = p.n;
    x.K = p.k;
    x.KI = p.k / BK;
    x.nt_only = store_nt_only(p.k);
    x.tiles_m = p.tiles_m;
    x.tiles_n = p.tiles_n;
    if constexpr (MODE == MODE_PTPC_G) {
        x.gather = p.gather;
        x.ready = 0;
        x.tl = order::round_list(blockIdx.x, gridDim.x, p.tiles_m * p.tiles_n);
    } else {
        x.tl = order::xcd_list(blockIdx.x, gridDim.x, p.tiles_m * p.tiles_n);
    }
    x.ntiles = x.tl.n;
    if (x.ntiles == 0) return;
    x.w = wave_id();
    x.lane = lane_id();
    x.i = x.lane & 15;
    x.g = x.lane >> 4;

    // A tile placement in LDS (lds_layout.h): the DMA lane fetches the row
    // and chunk that belong at the address it writes; a fragment read by 16
    // lanes touches every one of the 64 banks once.
    x.dma_lds = lds::dma_lds_byte(C::NA * x.w, 0);
#pragma unroll
    for (int j = 0; j < C::NA; ++j)
        x.voff_a[j] = lds::dma_row(C::NA * x.w + j, x.lane, C::MB) * x.K + lds::dma_chunk(C::NA * x.w + j, x.lane, C::MB) * 16;
#pragma unroll
    for (int odd = 0; odd < 2; ++odd)
#pragma unroll
        for (int half = 0; half < 2; ++half) x.rd[odd][half] = lds::frag_base(x.i, x.g, odd, half, C::MB);
    // B fragments: 16-column block NBW w + nb of the tile, K tile kt at
    // (block * KI + kt) * 2048; lane l reads 16 bytes at 16 l of each half.
#pragma unroll
    for (int nb = 0; nb < C::NBW; ++nb) x.voff_b[nb] = ((C::NBW * x.w + nb) * x.KI) * 2048 + 16 * x.lane;


    Ring g{x.ref(0), x.ref(1), x.ref(2)};

    // prologue: Bev(0), [E(0),] A(0), A(1), A(2) of the stream
    {
        const int KI = x.KI;
        issue_b<MODE, 0>(x, g.t0, 0);
        // with two or more K tiles per tile, the epilogue scales of a tile
        // are loaded a tile ahead: tile 0's here
        if constexpr (CASE != 4) issue_epilogue_scales<MODE>(x, g.t0);
        auto pos = [&](int sidx, int& kt) {
            if (sidx < KI) { kt = sidx; return g.t0; }
            if (sidx < 2 * KI) { kt = sidx - KI; return g.t1; }
            kt = sidx - 2 * KI;
            return g.t2;
        };
        int kt0, kt1, kt2;
        const TileRef r0 = pos(0, kt0), r1 = pos(1, kt1), r2 = pos(2, kt2);
        issue_a<MODE>(x, x.lds.p[0], r0, kt0);
        issue_a<MODE>(x, x.lds.p[1], r1, kt1);
        issue_a<MODE>(x, x.lds.p[2], r2, kt2);
    }
    wait_vm_lgkm0<sched::prologue_wait(C::NA)>();
    __builtin_amdgcn_s_barrier();
    x.pre[0] = read_a<MODE, 0>(x, 0);
    x.pre[1] = read_a<MODE, 0>(x, 1);

    constexpr int R = sched::phase_advance(CASE);  // KI % 4
    constexpr int CYCLE = R == 0 ? 1 : R == 2 ? 2 : 4;
    // tile j's first K tile sits in stage (R j) % 4; the first cycle is
    // peeled because its first tile has no predecessor to store
    TileRef prev{};
    run_tile<MODE, 0, CASE, false>(x, 0, g, prev);
    if constexpr (CYCLE >= 2) {
        if (1 < x.ntiles) run_tile<MODE, (R * 1) & 3, CASE, true>(x, 1, g, prev);
    }
    if constexpr (CYCLE == 4) {
        if (2 < x.ntiles) run_tile<MODE, (R * 2) & 3, CASE, true>(x, 2, g, prev);
        if (3 < x.ntiles) run_tile<MODE, (R * 3) & 3, CASE, true>(x, 3, g, prev);
    }
    for (int j = CYCLE; j < x.ntiles; j += CYCLE) {
        run_tile<MODE, 0, CASE, true>(x, j, g, prev);
        if constexpr (CYCLE >= 2) {
            if (j + 1 < x.ntiles) run_tile<MODE, (R * 1) & 3, CASE, true>(x, j + 1, g, prev);
        }
        if constexpr (CYCLE == 4) {
            if (j + 2 < x.ntiles) run_tile<MODE, (R * 2) & 3, CASE, true>(x, j + 2, g, prev);
            if (j + 3 < x.ntiles) run_tile<MODE, (R * 3) & 3, CASE, true>(x, j + 3, g, prev);
        }
    }
    if constexpr (kDeferEpilogue<MODE>) {
        // the last tile's epilogue (its row blocks 8..15 with two or more K
        // tiles per tile: the last K step stored the others)
        mfma_drain<MODE>(x);
        if constexpr (CASE == 4) store_tile<MODE>(x, prev.m0, prev.n0);
        else epi_rows<MODE, 8>(x, x.ep);
    }
}

// -------------------------------------------------------------- launch
static int device_cus() {
    static int cus[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cus[dev] = n;
    }
    return cus[dev];
}

template <int MODE>
static hipError_t launch_gemm(const GemmArgs& base, hipStream_t stream) {
    GemmArgs p = base;
    p.tiles_m = (p.m + Cfg<MODE>::BM - 1) / Cfg<MODE>::BM;
    p.tiles_n = (p.n + Cfg<MODE>::BN - 1) / Cfg<MODE>::BN;
    const int tiles = p.tiles_m * p.tiles_n;
    const int grid = tiles < device_cus() ? tiles : device_cus();
    const int ki = p.k / BK;
    switch (sched::case_of(ki)) {
        case 4: hipLaunchKernelGGL((gemm_a8w8_kernel<MODE, 4>), dim3(grid), dim3(Cfg<MODE>::NTHREADS), 0, stream, p); break;
        case 0: hipLaunchKernelGGL((gemm_a8w8_kernel<MODE, 0>), dim3(grid), dim3(Cfg<MODE>::NTHREADS), 0, stream, p); break;
        case 1: hipLaunchKernelGGL((gemm_a8w8_kernel<MODE, 1>), dim3(grid), dim3(Cfg<MODE>::NTHREADS), 0, stream, p); break;
        case 2: hipLaunchKernelGGL((gemm_a8w8_kernel<MODE, 2>), dim3(grid), dim3(Cfg<MODE>::NTHREADS), 0, stream, p); break;
        default: hipLaunchKernelGGL((gemm_a8w8_kernel<MODE, 3>), dim3(grid), dim3(Cfg<MODE>::NTHREADS), 0, stream, p); break;
    }
    return hipGetLastError();
}

// Tile choice.  The persistent grid gives each CU ceil(T / CUs) tiles at
// most, so a launch takes about ceil(T / CUs) tile times.  The 256 x 256 tile
// moves the fewest bytes per matrix op; a half-size tile (128 x 256 for
// ptpc, 256 x 128 for mxfp8) takes `half_cost` of a wide tile's time (more
// than one half: it reads the same LDS fragments for half the matrix ops;
// ptpc also has a quarter-size tile, below).
// The half tile is chosen when its waves cost less, which happens where the
// wide grid leaves many CUs idle in its last wave (at most half the CUs
// busy, or a last wave well short of full).
static bool half_tile_wins(long wide_tiles, long half_tiles, double half_cost) {
    const long cus = device_cus();
    const long wide_waves = (wide_tiles + cus - 1) / cus, half_waves = (half_tiles + cus - 1) / cus;
    return (double)half_waves * half_cost < (double)wide_waves;
}

// ptpc, three tiles: 256 x 256 (1), 128 x 256 of eight waves (2) and
// 128 x 128 of four waves (3), each costing a measured fraction of a wide
// tile's time (the 128 x 128 tile: 28 waves 206 us against 7 waves of wide
// tiles 162 us at 16384 x 7168 x 1792, 56 against 14 waves 434 against
// 319 us at 32768 x 7168 x 1792).  The launch takes the tile whose waves
// over the CUs cost least; the smaller tiles pay off only where the wide
// grid leaves CUs idle.
constexpr double kPtpcHalfCost = 0.625, kPtpcQuarterCost = 0.34;
int ptpc_tile_for(int m, int n) {
    const long cus = device_cus();
    auto waves = [cus](long tiles) { return (double)((tiles + cus - 1) / cus); };
    const double wide = waves((long)((m + 255) / 256) * ((n + 255) / 256));
    const double half = kPtpcHalfCost * waves((long)((m + 127) / 128) * ((n + 255) / 256));
    const double quarter = kPtpcQuarterCost * waves((long)((m + 127) / 128) * ((n + 127) / 128));
    return quarter < half && quarter < wide ? 3 : half < wide ? 2 : 1;
}

// mxfp8: the 256 x 128 tile of four waves.
constexpr double kMxfp8HalfCost = 0.625;
int mxfp8_tile_for(int m, int n) {
    const long wide = (long)((m + 255) / 256) * ((n + 255) / 256);
    const long half = (long)((m + 255) / 256) * ((n + 127) / 128);
    return half_tile_wins(wide, half, kMxfp8HalfCost) ? 2 : 1;
}

// blockscale: the 128 x 128 tile of four waves (one per SIMD, so no second
// wave fills the gaps of its instruction stream) costs 0.59 of a 128 x 256
// tile (measured at 16384 x 7168 x 2048: 28 waves of the small tile 282 us,
// 14 waves of the wide one 239 us).
constexpr double kBlockscaleHalfCost = 0.59;
int blockscale_tile_for(int m, int n) {
    const long wide = (long)((m + 127) / 128) * ((n + 255) / 256);
    const long half = (long)((m + 127) / 128) * ((n + 127) / 128);
    return half_tile_wins(wide, half, kBlockscaleHalfCost) ? 2 : 1;
}

hipError_t launch_gemm_a8w8(int mode, int tile, const uint8_t* a, const uint8_t* b, const void* sa, const void* sb,
                            uint16_t* c, int m, int n, int k, hipStream_t stream) {
    GemmArgs p{a, b, sa, sb, c, m, n, k, 0, 0};
    if (mode == MODE_PTPC) {
        const int t = tile == 0 ? ptpc_tile_for(m, n) : tile;
        if (t == 2) return launch_gemm<MODE_PTPC_N>(p, stream);
        if (t == 3) return launch_gemm<MODE_PTPC_Q>(p, stream);
        return launch_gemm<MODE_PTPC>(p, stream);
    }
    if (mode == MODE_MXFP8 && (tile == 0 ? mxfp8_tile_for(m, n) : tile) == 2) mode = MODE_MXFP8_N;
    if (mode == MODE_MXFP8) return launch_gemm<MODE_MXFP8>(p, stream);
    if (mode == MODE_MXFP8_N) return launch_gemm<MODE_MXFP8_N>(p, stream);
    if ((tile == 0 ? blockscale_tile_for(m, n) : tile) == 2) return launch_gemm<MODE_BLOCKSCALE_N>(p, stream);
    return launch_gemm<MODE_BLOCKSCALE>(p, stream);
}

// ptpc over a gathered A (256 x 256 tiles, time-ordered grid): src_rows rows
// per source slab, nchunks arrival bands per slab (the host checks that
// every band is a whole number of 256-row tiles).
hipError_t launch_gemm_a8w8_gathered(const uint8_t* a, const uint8_t* b, const float* sa, const float* sb,
                                     uint16_t* c, int m, int n, int k, const uint32_t* flags, int src_rows,
                                     int nchunks, int own, uint32_t epoch, long long spin_limit, int* status,
                                     hipStream_t stream) {
    GemmArgs p{a, b, sa, sb, c, m, n, k, 0, 0};
    p.gather = Gather{flags, src_rows / 256, m / src_rows, nchunks, own, epoch, spin_limit, status};
    return launch_gemm<MODE_PTPC_G>(p, stream);
}

}  // namespace dmm
