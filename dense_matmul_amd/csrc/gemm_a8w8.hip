// gemm_a8w8.hip -- fp8 (OCP E4M3) a8w8 GEMM for gfx950 with bf16 output, in
// the three scaling modes of mori PR 785 ("fix(gemm-ar): drain the peeled
// tail's producers instead of tightening the loop", section Cost): ptpc,
// 1x128 / 128x128 blockscale and mxfp8.
//
//   C[m, n] = bf16( sum_k A[m, k] sa(m, k) * B[n, k] sb(n, k) ),  fp32 accumulate
//
// Structure (one 256-thread workgroup = 4 waves per output tile):
//   * Output tile 16*MB x 256 (MB = 16 for ptpc / mxfp8, 8 for blockscale).
//     Wave w owns all tile rows and the 64 columns [64w, 64w + 64).
//   * A (row-major codes) streams global -> LDS with direct-to-LDS buffer
//     loads (16 B per lane) through a 4-stage ring of separate LDS arrays,
//     refilled three K tiles ahead.  Rows are stored 128 B apart with the
//     16-byte chunks XOR-swizzled by (row / MB) & 7 so that fragment reads
//     are bank-conflict free.
//   * B comes pre-shuffled (preshuffle_b) into the matrix-core operand order,
//     so every wave loads its fragments straight into registers with fully
//     coalesced 1 KiB loads, one K tile ahead (register double buffer).
//   * v_mfma_scale_f32_16x16x128_f8f6f4: src0 = 16 B rows (output columns),
//     src1 = 16 A rows (output rows).  Lane l holds row l%16 and, in bytes
//     0-15 / 16-31, K values 16(l/16)+[0,16) / 64+16(l/16)+[0,16) of the
//     128-wide K tile; the result lane l holds C rows for column... see
//     store_tile.  mxfp8 passes the E8M0 scales to the instruction (lane
//     16q + i carries the scale of row i, K group q); ptpc applies both
//     scales in the epilogue; blockscale folds one scale per 128-K tile into
//     fp32 accumulators in VGPRs.
//   * Every LDS read of a K tile follows "s_waitcnt vmcnt(c) lgkmcnt(0);
//     s_barrier" where c comes from kpipe.h and covers that tile's DMA in
//     every wave.  Every step issues its loads unconditionally (tiles past
//     the end go through a zero-length buffer descriptor), so the counts are
//     constants and the tail -- the last three K tiles, all of K = 256 --
//     runs the same waits as the middle of the loop.
#include "common.h"
#include "kpipe.h"

#include <type_traits>

namespace dmm {

enum { MODE_PTPC = 0, MODE_BLOCKSCALE = 1, MODE_MXFP8 = 2 };

constexpr int BN = 256, BK = 128, NTHREADS = 256;

// The LDS ring: four distinct arrays so that the compiler can tell the
// stages apart (its own LDS-DMA dependency tracking is per object).
constexpr int kMaxStageBytes = 256 * BK;
__shared__ __attribute__((aligned(1024))) char g_lds_a0[kMaxStageBytes];
__shared__ __attribute__((aligned(1024))) char g_lds_a1[kMaxStageBytes];
__shared__ __attribute__((aligned(1024))) char g_lds_a2[kMaxStageBytes];
__shared__ __attribute__((aligned(1024))) char g_lds_a3[kMaxStageBytes];

template <int S>
__device__ __forceinline__ char* stage_ptr() {
    if constexpr (S == 0) return g_lds_a0;
    else if constexpr (S == 1) return g_lds_a1;
    else if constexpr (S == 2) return g_lds_a2;
    else return g_lds_a3;
}

template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

struct GemmArgs {
    const uint8_t* a;
    const uint8_t* b;
    const void* sa;
    const void* sb;
    uint16_t* c;
    int m, n, k;
    int tiles_m, tiles_n;
};

template <int MODE>
struct Cfg {
    static constexpr int MB = MODE == MODE_BLOCKSCALE ? 8 : 16;  // 16-row blocks per wave
    static constexpr int BM = 16 * MB;                            // tile rows
    static constexpr int NA = MB / 2;                             // DMA instructions per wave per K tile
    // vector-memory instructions of one B event: 8 fragment loads plus scales
    static constexpr int NB = MODE == MODE_PTPC ? 8 : MODE == MODE_MXFP8 ? 8 + 2 + 4 : 8 + MB + 1;
    static_assert(2 * NB + NA <= 63, "vmcnt range");
};

// Workgroup -> output tile.  The dispatcher hands consecutive workgroups to
// the 8 XCDs in turn, so workgroup w runs on XCD w % 8; each XCD is given a
// contiguous range of the tile order, which walks GROUP row tiles across all
// column tiles so that concurrently running tiles share A and B in that
// XCD's L2.
__device__ __forceinline__ void tile_of(int wg, int tiles_m, int tiles_n, int& tm, int& tn) {
    constexpr int GROUP = 4;
    const int T = tiles_m * tiles_n;
    const int x = wg & 7, s = wg >> 3, per = T >> 3, rem = T & 7;
    const int t = x * per + (x < rem ? x : rem) + s;
    const int group = t / (GROUP * tiles_n);
    const int first = group * GROUP;
    const int gsize = tiles_m - first < GROUP ? tiles_m - first : GROUP;
    const int within = t - group * GROUP * tiles_n;
    tm = first + within % gsize;
    tn = within / gsize;
}

template <int MODE>
struct Ctx {
    using C = Cfg<MODE>;
    // buffer descriptors are built at each use from (base, bytes) in SGPRs
    const void *pa, *pb, *psa, *psb;
    uint32_t na, nb, nsa, nsb;
    int KI, M, N, K, m0, n0, w, lane, i, g;
    int dma_lds;                   // byte offset of this wave's DMA slots in a stage
    int voff_a[C::NA];             // per-lane global byte offsets of the DMA rows
    int voff_b[4];                 // per-lane global byte offsets of the B fragments
    int rd0, rd1;                  // per-lane LDS byte offsets of the two 16-B halves
    int voff_sa[Cfg<MODE>::MB];    // blockscale: per-row A scale offsets (row clamped to M-1)
    int voff_sb;                   // B scale offset (mode dependent)
    v4f acc[C::MB][4];
    v8i bq[2][4];                  // B fragments, double buffered across K tiles
    v8i pre[2];                    // first two A fragments of the next K tile
    // mxfp8: E8M0 bytes for A (16 rows, 4 words + spill word) and B (4 columns)
    v4i sxa[2];
    int sxa_tail[2];
    int sxb[2][4];
    // blockscale: A scales of this lane's MB rows and the wave's B block scale
    v4f sfa[2][C::MB / 4];
    float sfb[2];
};

// ---------------------------------------------------------------- issue
template <int MODE, int T>
__device__ __forceinline__ void issue_b(Ctx<MODE>& x, int kt, bool valid) {
    using C = Cfg<MODE>;
    // a tile past the end is loaded through zero-length descriptors: no data
    // moves, but the instructions still count in vmcnt
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(x.pb, valid ? x.nb : 0u);
    const __amdgpu_buffer_rsrc_t rsa = make_rsrc(x.psa, valid ? x.nsa : 0u);
    const __amdgpu_buffer_rsrc_t rsb = make_rsrc(x.psb, valid ? x.nsb : 0u);
    // B fragments: 2 KiB per (16-column block, K tile), lane l at byte 16 l
    // of each 1 KiB half.
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
        v4i lo = __builtin_amdgcn_raw_buffer_load_b128(rb, x.voff_b[nb] + kt * 2048, 0, 0);
        v4i hi = __builtin_amdgcn_raw_buffer_load_b128(rb, x.voff_b[nb] + kt * 2048 + 1024, 0, 0);
        x.bq[T][nb] = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
    if constexpr (MODE == MODE_MXFP8) {
        // A: 16 consecutive E8M0 bytes (rows 16i .. 16i+15 of the tile) of K
        // group 4kt + g; the row stride M need not be a multiple of 4, so
        // load the dword-aligned window and realign in registers.
        const int off = (4 * kt + x.g) * x.M + x.m0 + 16 * x.i;
        const int base = off & ~3;
        x.sxa[T] = __builtin_amdgcn_raw_buffer_load_b128(rsa, base, 0, 0);
        x.sxa_tail[T] = __builtin_amdgcn_raw_buffer_load_b32(rsa, base + 16, 0, 0);
        // B: the byte of column 16 nb + i of the wave's 64, K group 4kt + g
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
            x.sxb[T][nb] = __builtin_amdgcn_raw_buffer_load_b8(rsb, x.voff_sb + (4 * kt) * x.N + nb * 16, 0, 0);
    } else if constexpr (MODE == MODE_BLOCKSCALE) {
        // one dword per row; rows past M read row M-1 (their output is dropped)
#pragma unroll
        for (int r = 0; r < C::MB; ++r)
            x.sfa[T][r / 4][r % 4] = __builtin_bit_cast(
                float, __builtin_amdgcn_raw_buffer_load_b32(rsa, x.voff_sa[r] + kt * x.M * 4, 0, 0));
        x.sfb[T] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsb, x.voff_sb + kt * 4, 0, 0));
    }
}

template <int MODE>
__device__ __forceinline__ void dma_a_tile(Ctx<MODE>& x, char* stage, int kt, bool valid) {
    using C = Cfg<MODE>;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(x.pa, valid ? x.na : 0u);
    char* dst = stage + x.dma_lds;
#pragma unroll
    for (int j = 0; j < C::NA; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(dst + j * 1024), 16, x.voff_a[j] + kt * BK, 0, 0, 0);
}

template <int MODE, int S>
__device__ __forceinline__ v8i read_a(const Ctx<MODE>& x, int mb) {
    const char* st = stage_ptr<S>();
    v4i lo = *(const v4i*)(st + x.rd0 + mb * 128);
    v4i hi = *(const v4i*)(st + x.rd1 + mb * 128);
    return (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// ------------------------------------------------------------- compute
template <int MODE, int T, int mb>
__device__ __forceinline__ void mfma_row(Ctx<MODE>& x, const v8i& a) {
    if constexpr (MODE == MODE_PTPC) {
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
            x.acc[mb][nb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(x.bq[T][nb], a, x.acc[mb][nb], 0, 0, 0, 0, 0, 0);
    } else if constexpr (MODE == MODE_MXFP8) {
        // src1 (A) scale: byte mb % 4 of word mb / 4 of the realigned bytes
        const int sa_word = x.sxa[T][mb / 4];
        static_for<0, 4>([&](auto NBc) {
            constexpr int nb = decltype(NBc)::value;
            x.acc[mb][nb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                x.bq[T][nb], a, x.acc[mb][nb], 0, 0, 0, x.sxb[T][nb], mb % 4, sa_word);
        });
    } else {
        const float s = x.sfa[T][mb / 4][mb % 4] * x.sfb[T];
        const v4f zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            v4f p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(x.bq[T][nb], a, zero, 0, 0, 0, 0, 0, 0);
            x.acc[mb][nb] += p * s;
        }
    }
}

// Realign the 20 loaded E8M0 bytes so word q holds the bytes of rows 4q..4q+3.
template <int MODE, int T>
__device__ __forceinline__ void realign_mx(Ctx<MODE>& x, int kt) {
    if constexpr (MODE == MODE_MXFP8) {
        const int off = (4 * kt + x.g) * x.M + x.m0 + 16 * x.i;
        const int sh = off & 3;
        if (sh) {
            v4i w = x.sxa[T];
            int t = x.sxa_tail[T];
            // alignbyte(hi, lo, s) = bytes s..s+3 of the 64-bit hi:lo
            x.sxa[T] = (v4i){(int)__builtin_amdgcn_alignbyte(w[1], w[0], sh), (int)__builtin_amdgcn_alignbyte(w[2], w[1], sh),
                              (int)__builtin_amdgcn_alignbyte(w[3], w[2], sh), (int)__builtin_amdgcn_alignbyte(t, w[3], sh)};
        }
    }
    (void)x;
    (void)kt;
}

template <int MODE>
__device__ __forceinline__ void wait_mid(int k) {
    using C = Cfg<MODE>;
    if (k == 0) wait_vm_lgkm0<sched::mid_wait(0, C::NA, C::NB)>();
    else wait_vm_lgkm0<sched::mid_wait(1, C::NA, C::NB)>();
}

// One K tile.  S = k % 4 selects the LDS stage, T = k % 2 the B registers.
template <int MODE, int S>
__device__ __forceinline__ void kstep(Ctx<MODE>& x, int k) {
    using C = Cfg<MODE>;
    constexpr int T = S & 1;
    constexpr int SR = (S + 3) & 3;  // stage refilled by this step (tile k-1's)
    constexpr int SN = (S + 1) & 3;  // stage of tile k+1
    issue_b<MODE, T ^ 1>(x, k + 1, sched::b_valid(k, x.KI));
    realign_mx<MODE, T>(x, k);
    // first half of the row blocks; the first two A fragments were read at
    // the end of the previous step
    static_for<0, C::MB / 2>([&](auto MBc) {
        constexpr int mb = decltype(MBc)::value;
        v8i a;
        if constexpr (mb < 2) a = x.pre[mb];
        else a = read_a<MODE, S>(x, mb);
        mfma_row<MODE, T, mb>(x, a);
    });
    // RAW: K tile k+1 has landed in every wave's share of LDS.
    // WAR: every wave's reads of stage SR (K tile k-1) have retired.
    wait_mid<MODE>(k);
    __builtin_amdgcn_s_barrier();
    {
        const __amdgpu_buffer_rsrc_t ra = make_rsrc(x.pa, sched::a_valid(k, x.KI) ? x.na : 0u);
        char* dst = stage_ptr<SR>() + x.dma_lds;
#pragma unroll
        for (int j = 0; j < C::NA; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(dst + j * 1024), 16, x.voff_a[j] + (k + 3) * BK,
                                                     0, 0, 0);
    }
    static_for<C::MB / 2, C::MB>([&](auto MBc) {
        constexpr int mb = decltype(MBc)::value;
        v8i a = read_a<MODE, S>(x, mb);
        mfma_row<MODE, T, mb>(x, a);
    });
    // prefetch the next tile's first fragments (covered by the barrier
    // above; after the last tile the values are unused)
    x.pre[0] = read_a<MODE, SN>(x, 0);
    x.pre[1] = read_a<MODE, SN>(x, 1);
}

// ------------------------------------------------------------ epilogue
template <int MODE>
__device__ __forceinline__ void store_tile(Ctx<MODE>& x, const GemmArgs& p) {
    using C = Cfg<MODE>;
    // result lane l, register v of block (mb, nb):
    //   row    m0 + MB * (l % 16) + mb
    //   column n0 + 64 w + 16 nb + 4 (l / 16) + v
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(p.c, (uint32_t)p.m * (uint32_t)p.n * 2u);
    v4f as[C::MB / 4];
    v4f bs[4];
    if constexpr (MODE == MODE_PTPC) {
        const __amdgpu_buffer_rsrc_t rsa = make_rsrc(p.sa, (uint32_t)p.m * 4u);
        const __amdgpu_buffer_rsrc_t rsb = make_rsrc(p.sb, (uint32_t)p.n * 4u);
#pragma unroll
        for (int r = 0; r < C::MB; ++r) {
            const int row = x.m0 + C::MB * x.i + r;
            as[r / 4][r % 4] = __builtin_bit_cast(
                float, __builtin_amdgcn_raw_buffer_load_b32(rsa, (row < x.M ? row : x.M - 1) * 4, 0, 0));
        }
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
            bs[nb] = __builtin_bit_cast(
                v4f, __builtin_amdgcn_raw_buffer_load_b128(rsb, (x.n0 + 64 * x.w + 16 * nb + 4 * x.g) * 4, 0, 0));
    }
    const int row0 = x.m0 + C::MB * x.i;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
        const int col = x.n0 + 64 * x.w + 16 * nb;
        if (col >= x.N) continue;  // wave-uniform: the 16-column block is past N
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb) {
            v4f v = x.acc[mb][nb];
            if constexpr (MODE == MODE_PTPC) v = v * as[mb / 4][mb % 4] * bs[nb];
            v2i packed = {pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
            // rows at or past M fall outside the buffer and are dropped
            __builtin_amdgcn_raw_buffer_store_b64(packed, rc, ((row0 + mb) * x.N + col + 4 * x.g) * 2, 0, 0);
        }
    }
}

// -------------------------------------------------------------- kernel
template <int MODE>
__global__ void __launch_bounds__(NTHREADS, 1) gemm_a8w8_kernel(GemmArgs p) {
    using C = Cfg<MODE>;
    Ctx<MODE> x;
    int tm, tn;
    tile_of(blockIdx.x, p.tiles_m, p.tiles_n, tm, tn);
    x.M = p.m;
    x.N = p.n;
    x.K = p.k;
    x.KI = p.k / BK;
    x.m0 = tm * C::BM;
    x.n0 = tn * BN;
    x.w = wave_id();
    x.lane = lane_id();
    x.i = x.lane & 15;
    x.g = x.lane >> 4;
    x.pa = p.a;
    x.na = (uint32_t)p.m * (uint32_t)p.k;
    x.pb = p.b;
    x.nb = (uint32_t)p.n * (uint32_t)p.k;
    x.psa = p.sa;
    x.psb = p.sb;
    x.nsa = x.nsb = 0;

    // DMA: instruction j of wave w fills LDS rows 8 (NA w + j) .. +7, lane l
    // writing bytes 16 (l % 8) of row 8 (NA w + j) + l / 8; it fetches the
    // 16-byte chunk whose swizzled position that is.
    x.dma_lds = x.w * C::NA * 1024;
#pragma unroll
    for (int j = 0; j < C::NA; ++j) {
        const int r = 8 * (C::NA * x.w + j) + (x.lane >> 3);
        const int chunk = (x.lane & 7) ^ ((r / C::MB) & 7);
        x.voff_a[j] = (x.m0 + r) * x.K + chunk * 16;
    }
    // A fragment of row block mb: lane (i, g) reads row MB i + mb, K chunks
    // g (bytes 0-15) and 4 + g (bytes 16-31), each at its swizzled position.
    x.rd0 = C::MB * x.i * 128 + ((x.g ^ (x.i & 7)) * 16);
    x.rd1 = C::MB * x.i * 128 + (((4 + x.g) ^ (x.i & 7)) * 16);
    // B fragments: 16-column block (n0 + 64 w) / 16 + nb, K tile kt at
    // ((block * KI) + kt) * 2048; lane l reads 16 B at 16 l of each half.
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) x.voff_b[nb] = (((x.n0 + 64 * x.w) / 16 + nb) * x.KI) * 2048 + 16 * x.lane;
    if constexpr (MODE == MODE_MXFP8) {
        x.nsa = (uint32_t)(x.K / 32) * (uint32_t)p.m;
        x.nsb = (uint32_t)(x.K / 32) * (uint32_t)p.n;
        x.voff_sb = x.g * x.N + x.n0 + 64 * x.w + x.i;
    } else if constexpr (MODE == MODE_BLOCKSCALE) {
        x.nsa = (uint32_t)x.KI * (uint32_t)p.m * 4u;
        x.nsb = (uint32_t)((p.n + 127) / 128) * (uint32_t)x.KI * 4u;
#pragma unroll
        for (int r = 0; r < C::MB; ++r) {
            const int row = x.m0 + C::MB * x.i + r;
            x.voff_sa[r] = (row < x.M ? row : x.M - 1) * 4;
        }
        x.voff_sb = ((x.n0 + 64 * x.w) / 128) * x.KI * 4;
    }
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) x.acc[mb][nb] = (v4f){0.f, 0.f, 0.f, 0.f};

    // prologue: Bev(0), A(0), A(1), A(2)
    issue_b<MODE, 0>(x, 0, true);
    dma_a_tile<MODE>(x, stage_ptr<0>(), 0, true);
    dma_a_tile<MODE>(x, stage_ptr<1>(), 1, 1 < x.KI);
    dma_a_tile<MODE>(x, stage_ptr<2>(), 2, 2 < x.KI);
    wait_vm_lgkm0<sched::prologue_wait(C::NA)>();
    __builtin_amdgcn_s_barrier();
    x.pre[0] = read_a<MODE, 0>(x, 0);
    x.pre[1] = read_a<MODE, 0>(x, 1);

    // K loop, unrolled by the 4 LDS stages: whole groups of four steps,
    // then up to three guarded steps whose stages are again static.  Every
    // step issues its loads unconditionally, so the compiler's own vmcnt
    // tracking stays exact across the guards.
    int k = 0;
    for (; k + 4 <= x.KI; k += 4) {
        kstep<MODE, 0>(x, k);
        kstep<MODE, 1>(x, k + 1);
        kstep<MODE, 2>(x, k + 2);
        kstep<MODE, 3>(x, k + 3);
    }
    if (k < x.KI) kstep<MODE, 0>(x, k);
    if (k + 1 < x.KI) kstep<MODE, 1>(x, k + 1);
    if (k + 2 < x.KI) kstep<MODE, 2>(x, k + 2);
    store_tile<MODE>(x, p);
}

// -------------------------------------------------------------- launch
template <int MODE>
static hipError_t launch_gemm(const GemmArgs& base, hipStream_t stream) {
    GemmArgs p = base;
    p.tiles_m = (p.m + Cfg<MODE>::BM - 1) / Cfg<MODE>::BM;
    p.tiles_n = (p.n + BN - 1) / BN;
    const int tiles = p.tiles_m * p.tiles_n;
    hipLaunchKernelGGL(gemm_a8w8_kernel<MODE>, dim3(tiles), dim3(NTHREADS), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_gemm_a8w8(int mode, const uint8_t* a, const uint8_t* b, const void* sa, const void* sb,
                            uint16_t* c, int m, int n, int k, hipStream_t stream) {
    GemmArgs p{a, b, sa, sb, c, m, n, k, 0, 0};
    if (mode == MODE_PTPC) return launch_gemm<MODE_PTPC>(p, stream);
    if (mode == MODE_MXFP8) return launch_gemm<MODE_MXFP8>(p, stream);
    return launch_gemm<MODE_BLOCKSCALE>(p, stream);
}

}  // namespace dmm
