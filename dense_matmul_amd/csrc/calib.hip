// calib.hip -- how fast gfx950 issues the GEMM's matrix instruction when
// nothing else is in the way: every wave runs a long stream of back-to-back,
// independent v_mfma_f32_16x16x128_f8f6f4 on e4m3 operands it loaded once,
// with one or two waves per SIMD.  The benchmark reports this next to the
// published dense fp8 peak, so that the GEMM's own figure can be read
// against what one wave per SIMD can reach on the part it runs on (clock
// under load included).  Not part of the GEMM path.
#include "common.h"

namespace dmm {

constexpr int kCalibFrags = 65536;  // 32-byte operand fragments read from the caller's buffer (2 MiB)

// Sixteen independent accumulators, four A and four B fragments per lane:
// each op depends only on the op sixteen places earlier, far past the
// result latency, so the matrix pipe never waits on a dependency.
template <int WPS>
__global__ void __launch_bounds__(256 * WPS, 1) mfma_ceiling_kernel(const v8i* __restrict__ frag, float* out,
                                                                   int out_len, int iters) {
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    v8i a[4], b[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        a[j] = frag[(t * 8 + j) & (kCalibFrags - 1)];
        b[j] = frag[(t * 8 + 4 + j) & (kCalibFrags - 1)];
    }
    v4f acc[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] = (v4f){0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 16; ++j)
            asm volatile("v_mfma_f32_16x16x128_f8f6f4 %0, %1, %2, %0" : "+a"(acc[j]) : "v"(b[j / 4]), "v"(a[j % 4]));
    }
    // the asm ops are invisible to the compiler's hazard tracking: wait out
    // the longest result latency before the accumulators are read
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        asm volatile("" : "+a"(acc[j]));
        s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
    }
    if (t < out_len) out[t] = s;
}

// One workgroup of 4 * wps waves per CU; returns the grid size through *grid.
hipError_t launch_mfma_ceiling(const uint8_t* frag, float* out, int out_len, int iters, int wps, int* grid,
                               hipStream_t st) {
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    *grid = cus;
    const v8i* f = reinterpret_cast<const v8i*>(frag);
    if (wps == 1) hipLaunchKernelGGL(mfma_ceiling_kernel<1>, dim3(cus), dim3(256), 0, st, f, out, out_len, iters);
    else hipLaunchKernelGGL(mfma_ceiling_kernel<2>, dim3(cus), dim3(512), 0, st, f, out, out_len, iters);
    return hipGetLastError();
}

}  // namespace dmm
