// gemm_bf16.hip -- bf16 x bf16 -> bf16 GEMM with fp32 accumulation for
// gfx950: C[m, n] = bf16(sum_k A[m, k] B[n, k]).  The shape of interest is
// DeepGEMM PR 453 ("Fix SM120 BF16 GEMM shared-memory reuse ordering",
// Reproduction and validation): [4096, 1024] x [1024, 896].
//
// 128 x 128 output tile per 256-thread workgroup, 2 x 2 waves of 64 x 64.
// Both operands stream global -> LDS by direct-to-LDS buffer loads into a
// 3-stage ring of separate arrays (K tile 64 = 128 B per row, 16-byte chunks
// XOR-swizzled by row & 7); v_mfma_f32_16x16x32_bf16 with src0 = B rows
// (output columns) and src1 = A rows (output rows), so each lane ends with 4
// consecutive output columns of one row.  The stage written by a refill was
// last read one step earlier; the barrier that ends that step (after
// lgkmcnt(0)) orders the reads before the refill, and the wait before it
// (vmcnt) makes the next stage complete in every wave before anyone reads it.
#include "common.h"

#include <type_traits>

namespace dmm {

typedef __bf16 bf8 __attribute__((ext_vector_type(8)));

namespace bf16k {
constexpr int BM = 128, BN = 128, BK = 64, NT = 256, STAGE = BM * BK * 2;  // 16 KiB per operand per stage
constexpr int NL = STAGE / 1024 / 4;  // DMA instructions per wave per operand per stage (4)

__shared__ __attribute__((aligned(1024))) char g_a0[STAGE];
__shared__ __attribute__((aligned(1024))) char g_a1[STAGE];
__shared__ __attribute__((aligned(1024))) char g_a2[STAGE];
__shared__ __attribute__((aligned(1024))) char g_b0[STAGE];
__shared__ __attribute__((aligned(1024))) char g_b1[STAGE];
__shared__ __attribute__((aligned(1024))) char g_b2[STAGE];

template <int S>
__device__ __forceinline__ char* sa() {
    if constexpr (S == 0) return g_a0;
    else if constexpr (S == 1) return g_a1;
    else return g_a2;
}
template <int S>
__device__ __forceinline__ char* sb() {
    if constexpr (S == 0) return g_b0;
    else if constexpr (S == 1) return g_b1;
    else return g_b2;
}

struct Ctx {
    const void *pa, *pb;
    uint32_t na, nb;
    int KT, wm, wn, lane, i, g;
    int dma_lds;
    int voff_a[NL], voff_b[NL];
    int rd[2];  // LDS byte offset of this lane's 16-byte chunk for MFMA k-half 0 / 1
    v4f acc[4][4];
};

// Tile kt into stage S.  Tiles past the end go through zero-length
// descriptors: no data moves, the instructions still count in vmcnt, so every
// wait below is a constant.
template <int S>
__device__ __forceinline__ void issue(Ctx& x, int kt) {
    const bool valid = kt < x.KT;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(x.pa, valid ? x.na : 0u);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(x.pb, valid ? x.nb : 0u);
#pragma unroll
    for (int j = 0; j < NL; ++j) {
        lds_dma16(ra, (lds_char*)(sa<S>() + x.dma_lds + j * 1024), x.voff_a[j] + kt * BK * 2);
        lds_dma16(rb, (lds_char*)(sb<S>() + x.dma_lds + j * 1024), x.voff_b[j] + kt * BK * 2);
    }
}

template <int S>
__device__ __forceinline__ void compute(Ctx& x) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        bf8 af[4], bfr[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            af[q] = *(const bf8*)(sa<S>() + (64 * x.wm + 16 * q) * 128 + x.rd[kk]);
            bfr[q] = *(const bf8*)(sb<S>() + (64 * x.wn + 16 * q) * 128 + x.rd[kk]);
        }
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
                x.acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[nb], af[mb], x.acc[mb][nb], 0, 0, 0);
    }
}

// Step kt computes stage S = kt % 3 and refills stage (kt + 2) % 3.
template <int S>
__device__ __forceinline__ void step(Ctx& x, int kt) {
    issue<(S + 2) % 3>(x, kt + 2);
    compute<S>(x);
    // tile kt+1 was issued one step (2 NL instructions) before tile kt+2
    wait_vm_lgkm0<2 * NL>();
    __builtin_amdgcn_s_barrier();
}
}  // namespace bf16k

__global__ void __launch_bounds__(bf16k::NT, 1) gemm_bf16_kernel(const uint16_t* a, const uint16_t* b, uint16_t* c, int m,
                                                                 int n, int k, int tiles_n) {
    using namespace bf16k;
    Ctx x;
    const int tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
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
    x.dma_lds = w * NL * 1024;
#pragma unroll
    for (int j = 0; j < NL; ++j) {
        const int r = 8 * (NL * w + j) + (x.lane >> 3);
        const int chunk = (x.lane & 7) ^ (r & 7);
        x.voff_a[j] = ((m0 + r) * k) * 2 + chunk * 16;
        x.voff_b[j] = ((n0 + r) * k) * 2 + chunk * 16;
    }
    // MFMA k-half kk: lane (i, g) reads row 16 q + i, 16-byte chunk 4 kk + g
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) x.rd[kk] = x.i * 128 + (((4 * kk + x.g) ^ (x.i & 7)) * 16);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) x.acc[mb][nb] = (v4f){0.f, 0.f, 0.f, 0.f};

    issue<0>(x, 0);
    issue<1>(x, 1);
    wait_vm_lgkm0<2 * NL>();
    __builtin_amdgcn_s_barrier();
    for (int kt = 0; kt < x.KT; kt += 3) {
        step<0>(x, kt);
        if (kt + 1 < x.KT) step<1>(x, kt + 1);
        if (kt + 2 < x.KT) step<2>(x, kt + 2);
    }

    // lane (i, g), block (mb, nb): row m0 + 64 wm + 16 mb + i, columns
    // n0 + 64 wn + 16 nb + 4 g + [0, 4)
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(c, (uint32_t)m * (uint32_t)n * 2u);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
        const int col = n0 + 64 * x.wn + 16 * nb;
        if (col >= n) continue;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            const int row = m0 + 64 * x.wm + 16 * mb + x.i;
            const v4f v = x.acc[mb][nb];
            v2i packed = {pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
            __builtin_amdgcn_raw_buffer_store_b64(packed, rc, (row * n + col + 4 * x.g) * 2, 0, 0);
        }
    }
}

hipError_t launch_gemm_bf16(const uint16_t* a, const uint16_t* b, uint16_t* c, int m, int n, int k, hipStream_t st) {
    const int tiles_m = (m + bf16k::BM - 1) / bf16k::BM, tiles_n = (n + bf16k::BN - 1) / bf16k::BN;
    hipLaunchKernelGGL(gemm_bf16_kernel, dim3(tiles_m * tiles_n), dim3(bf16k::NT), 0, st, a, b, c, m, n, k, tiles_n);
    return hipGetLastError();
}

}  // namespace dmm
