// gemm_bf16.hip -- bf16 x bf16 -> bf16 GEMM with fp32 accumulation for
// gfx950: C[m, n] = bf16(sum_k A[m, k] B[n, k]).  The shape of interest is
// DeepGEMM PR 453 ("Fix SM120 BF16 GEMM shared-memory reuse ordering",
// Reproduction and validation): [4096, 1024] x [1024, 896].
//
// BM x BN output tile per 256-thread workgroup, 2 x 2 waves of BM/2 x BN/2.
// Both operands stream global -> LDS by direct-to-LDS buffer loads into an
// NS-stage ring of separate arrays (K tile 64 = 128 B per row, 16-byte chunks
// placed by lds::bf16_chunk_pos, conflict-free for the fragment reads);
// v_mfma_f32_16x16x32_bf16 with src0 = B rows (output columns) and src1 =
// A rows (output rows), so each lane ends with 4 consecutive output columns
// of one row.
//
// K step kt (stage S = kt % NS) splits at its middle: the fragments of its
// first 32-wide k-half are already in registers (read during the previous
// step), its second k-half's are read while the first half's matrix ops
// run; then one wait (vmcnt: this wave's DMAs of K tile kt+1 have landed;
// lgkmcnt(0): its reads of stage S have retired) and a barrier (every wave
// has done both); then stage S itself is refilled with K tile kt + NS, and
// the next stage's first k-half is read while the second half's matrix ops
// run.  So each K tile is loaded NS steps ahead, no wave ever waits on an LDS
// read right after the barrier, and NS - 2 K tiles stay in flight behind the
// one each wait covers.
//
// Two tile sizes: 128 x 128 with 4 stages (one workgroup per CU, 128 KiB of
// LDS) in general, and 64 x 64 with 3 stages (48 KiB, three workgroups per
// CU) for grids too small to occupy half the CUs with 128 x 128 tiles.
//
// One workgroup per tile, placed XCD-aware (tile_order.h): workgroup b runs
// on XCD b % 8, and the tiles of one XCD are a contiguous run of the order
// in which groups of four row tiles sweep the column tiles, so an XCD's L2
// holds only its own rows of A (and B) instead of every XCD fetching nearly
// all of A.
#include "common.h"
#include "kpipe.h"
#include "lds_layout.h"
#include "tile_order.h"

#include <type_traits>

namespace dmm {

typedef __bf16 bf8 __attribute__((ext_vector_type(8)));

namespace bf16k {
constexpr int BK = 64, NT = 256;

template <int BM, int BN>
struct Cfg {
    static constexpr int NS = BM == 128 ? 4 : 3;              // LDS stages
    static constexpr int SA = BM * BK * 2, SB = BN * BK * 2;  // bytes per stage
    static constexpr int NLA = SA / 1024 / 4, NLB = SB / 1024 / 4;  // 1 KiB DMAs per wave per stage
    static constexpr int MBW = BM / 32, NBW = BN / 32;  // 16 x 16 blocks per wave
    static_assert(NLA >= 1 && NLB >= 1, "at least one DMA per wave per operand");
};

// The LDS ring: the kernel declares the arrays (one object per stage, so the
// compiler's LDS-DMA dependency tracking tells them apart) and carries their
// addresses here; after inlining they are constants again.
struct Ring {
    lds_char* a[4];
    lds_char* b[4];
};

template <int BM, int BN>
struct Ctx {
    using C = Cfg<BM, BN>;
    Ring lds;
    const void *pa, *pb;
    uint32_t na, nb;
    int KT, wm, wn, lane, i, g;
    int voff_a[C::NLA], voff_b[C::NLB];
    int rd[2];  // LDS byte offset of this lane's 16-byte chunk for MFMA k-half 0 / 1
    v4f acc[C::MBW][C::NBW];
};

// Tile kt into stage S.  Tiles past the end go through zero-length
// descriptors: no data moves, the instructions still count in vmcnt, so every
// wait below is a constant.
template <int BM, int BN, int S>
__device__ __forceinline__ void issue(Ctx<BM, BN>& x, int kt) {
    using C = Cfg<BM, BN>;
    const bool valid = kt < x.KT;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(x.pa, valid ? x.na : 0u);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(x.pb, valid ? x.nb : 0u);
    const int w = wave_id();
#pragma unroll
    for (int j = 0; j < C::NLA; ++j)
        lds_dma16(ra, x.lds.a[S] + (C::NLA * w + j) * 1024, x.voff_a[j] + kt * BK * 2);
#pragma unroll
    for (int j = 0; j < C::NLB; ++j)
        lds_dma16(rb, x.lds.b[S] + (C::NLB * w + j) * 1024, x.voff_b[j] + kt * BK * 2);
}

template <int BM, int BN, int S, int KK>
__device__ __forceinline__ void read_frags(const Ctx<BM, BN>& x, bf8 (&af)[Cfg<BM, BN>::MBW],
                                           bf8 (&bfr)[Cfg<BM, BN>::NBW]) {
    using C = Cfg<BM, BN>;
    typedef __attribute__((address_space(3))) const bf8 lds_bf8;
#pragma unroll
    for (int q = 0; q < C::MBW; ++q) af[q] = *(lds_bf8*)(x.lds.a[S] + ((BM / 2) * x.wm + 16 * q) * 128 + x.rd[KK]);
#pragma unroll
    for (int q = 0; q < C::NBW; ++q) bfr[q] = *(lds_bf8*)(x.lds.b[S] + ((BN / 2) * x.wn + 16 * q) * 128 + x.rd[KK]);
}

template <int BM, int BN>
struct Frags {
    bf8 a[Cfg<BM, BN>::MBW], b[Cfg<BM, BN>::NBW];
};

template <int BM, int BN>
__device__ __forceinline__ void mfmas(Ctx<BM, BN>& x, const Frags<BM, BN>& f) {
    using C = Cfg<BM, BN>;
#pragma unroll
    for (int mb = 0; mb < C::MBW; ++mb)
#pragma unroll
        for (int nb = 0; nb < C::NBW; ++nb)
            x.acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.b[nb], f.a[mb], x.acc[mb][nb], 0, 0, 0);
}

// Step kt (stage S); h0 holds its first k-half's fragments on entry and the
// next step's on exit.
template <int BM, int BN, int S>
__device__ __forceinline__ void step(Ctx<BM, BN>& x, int kt, Frags<BM, BN>& h0) {
    using C = Cfg<BM, BN>;
    constexpr int NS = C::NS;
    Frags<BM, BN> h1;
    read_frags<BM, BN, S, 1>(x, h1.a, h1.b);
    mfmas<BM, BN>(x, h0);
    // K tile kt+1 was followed by the DMAs of K tiles kt+2 .. kt+NS-1
    wait_vm_lgkm0<sched::bf16_mid_wait(NS, C::NLA + C::NLB)>();
    __builtin_amdgcn_s_barrier();
    issue<BM, BN, S>(x, kt + NS);
    read_frags<BM, BN, (S + 1) % NS, 0>(x, h0.a, h0.b);
    mfmas<BM, BN>(x, h1);
}
}  // namespace bf16k

template <int BM, int BN>
__global__ void __launch_bounds__(bf16k::NT) gemm_bf16_kernel(const uint16_t* a, const uint16_t* b, uint16_t* c, int m,
                                                              int n, int k, int tiles_m, int tiles_n) {
    using namespace bf16k;
    using C = Cfg<BM, BN>;
    constexpr int NS = C::NS;
    __shared__ __attribute__((aligned(1024))) char a0[C::SA], a1[C::SA], a2[C::SA], a3[NS == 4 ? C::SA : 16];
    __shared__ __attribute__((aligned(1024))) char b0[C::SB], b1[C::SB], b2[C::SB], b3[NS == 4 ? C::SB : 16];
    Ctx<BM, BN> x;
    x.lds = Ring{{(lds_char*)a0, (lds_char*)a1, (lds_char*)a2, (lds_char*)a3},
                 {(lds_char*)b0, (lds_char*)b1, (lds_char*)b2, (lds_char*)b3}};
    // the grid has one workgroup per tile: each list holds one position
    int tm, tn;
    order::coords(order::xcd_list(blockIdx.x, gridDim.x, tiles_m * tiles_n).first, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int w = wave_id();
    x.lane = lane_id();
    x.i = x.lane & 15;
    x.g = x.lane >> 4;
    x.wm = w >> 1;
    x.wn = w & 1;
    x.KT = k / BK;
    x.pa = a;
    x.na = (uint32_t)m * (uint32_t)k * 2u;
    x.pb = b;
    x.nb = (uint32_t)n * (uint32_t)k * 2u;
    // DMA j of wave w moves rows 8 (NL w + j) .. + 7 (128 bytes each); lane l
    // fetches row 8 (NL w + j) + l / 8, the chunk that belongs at byte 16 l
#pragma unroll
    for (int j = 0; j < C::NLA; ++j) {
        const int r = 8 * (C::NLA * w + j) + (x.lane >> 3);
        x.voff_a[j] = ((m0 + r) * k) * 2 + lds::bf16_chunk_pos(r, x.lane & 7) * 16;
    }
#pragma unroll
    for (int j = 0; j < C::NLB; ++j) {
        const int r = 8 * (C::NLB * w + j) + (x.lane >> 3);
        x.voff_b[j] = ((n0 + r) * k) * 2 + lds::bf16_chunk_pos(r, x.lane & 7) * 16;
    }
    // MFMA k-half kk: lane (i, g) reads row 16 q + i, 16-byte chunk 4 kk + g
    // (the position depends on (row >> 1) & 7, the same for every q)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) x.rd[kk] = x.i * 128 + lds::bf16_chunk_pos(x.i, 4 * kk + x.g) * 16;
#pragma unroll
    for (int mb = 0; mb < C::MBW; ++mb)
#pragma unroll
        for (int nb = 0; nb < C::NBW; ++nb) x.acc[mb][nb] = (v4f){0.f, 0.f, 0.f, 0.f};

    // prologue: K tiles 0 .. NS-1 into stages 0 .. NS-1; wait for tile 0
    // (followed by NS - 1 tiles' DMAs); the first k-half of tile 0
    issue<BM, BN, 0>(x, 0);
    issue<BM, BN, 1>(x, 1);
    issue<BM, BN, 2>(x, 2);
    if constexpr (NS == 4) issue<BM, BN, 3>(x, 3);
    wait_vm_lgkm0<sched::bf16_prologue_wait(NS, C::NLA + C::NLB)>();
    __builtin_amdgcn_s_barrier();
    Frags<BM, BN> h0;
    read_frags<BM, BN, 0, 0>(x, h0.a, h0.b);
    for (int kt = 0; kt < x.KT; kt += NS) {
        step<BM, BN, 0>(x, kt, h0);
        if (kt + 1 < x.KT) step<BM, BN, 1>(x, kt + 1, h0);
        if (kt + 2 < x.KT) step<BM, BN, 2>(x, kt + 2, h0);
        if constexpr (NS == 4)
            if (kt + 3 < x.KT) step<BM, BN, 3>(x, kt + 3, h0);
    }

    // lane (i, g), block (mb, nb): row m0 + BM/2 wm + 16 mb + i, columns
    // n0 + BN/2 wn + 16 nb + 4 g + [0, 4); rows past M fall outside the
    // descriptor, column blocks past N are skipped
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(c, (uint32_t)m * (uint32_t)n * 2u);
#pragma unroll
    for (int nb = 0; nb < C::NBW; ++nb) {
        const int col = n0 + (BN / 2) * x.wn + 16 * nb;
        if (col >= n) continue;
#pragma unroll
        for (int mb = 0; mb < C::MBW; ++mb) {
            const int row = m0 + (BM / 2) * x.wm + 16 * mb + x.i;
            const v4f v = x.acc[mb][nb];
            v2i packed = {pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
            __builtin_amdgcn_raw_buffer_store_b64(packed, rc, (row * n + col + 4 * x.g) * 2, 0, 0);
        }
    }
}

template <int BM, int BN>
static hipError_t launch_bf16(const uint16_t* a, const uint16_t* b, uint16_t* c, int m, int n, int k, hipStream_t st) {
    const int tiles_m = (m + BM - 1) / BM, tiles_n = (n + BN - 1) / BN;
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN>), dim3(tiles_m * tiles_n), dim3(bf16k::NT), 0, st, a, b, c, m, n, k,
                       tiles_m, tiles_n);
    return hipGetLastError();
}

static int bf16_device_cus() {
    static int cus[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cus[dev] == 0) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
        cus[dev] = v;
    }
    return cus[dev];
}

// tile 0: the library's choice (64 x 64 when the 128 x 128 grid would leave
// at least half the CUs idle), 1: 128 x 128, 2: 64 x 64.
hipError_t launch_gemm_bf16(const uint16_t* a, const uint16_t* b, uint16_t* c, int m, int n, int k, int tile,
                            hipStream_t st) {
    if (tile == 0) {
        const long big = (long)((m + 127) / 128) * ((n + 127) / 128);
        tile = 2 * big <= bf16_device_cus() ? 2 : 1;
    }
    if (tile == 2) return launch_bf16<64, 64>(a, b, c, m, n, k, st);
    return launch_bf16<128, 128>(a, b, c, m, n, k, st);
}

}  // namespace dmm
