// calib.hip -- how fast gfx950 issues the GEMM's matrix instruction when
// nothing else is in the way, and what each kind of instruction the GEMM
// interleaves with it costs: every wave runs a long stream of back-to-back,
// independent v_mfma_f32_16x16x128_f8f6f4 on e4m3 operands it loaded once,
// with one or two waves per SIMD, optionally with one kind of extra
// instruction after each op.  The benchmark reports these next to the
// published dense fp8 peak, so that the GEMM's own figure can be read
// against what the part reaches under load (clock included).  Not part of
// the GEMM path.
#include "common.h"

namespace dmm {

constexpr int kCalibFrags = 65536;  // 32-byte operand fragments read from the caller's buffer (2 MiB)

// Variants (the `variant` argument of dmm_mfma_ceiling_fp8):
enum {
    CAL_PLAIN = 0,      // the ptpc / blockscale instruction alone
    CAL_SCALED = 1,     // the mxfp8 form, E8M0 scales 127 (x1) on both operands
    CAL_LDS_READ = 2,   // + one ds_read_b128 per op (an A fragment half)
    CAL_VALU2 = 3,      // + two v_mul_f32 per op (epilogue scaling)
    CAL_ACC_READ = 4,   // + one v_accvgpr_read_b32 per op (an epilogue's accumulator read-out)
    CAL_ACC_READ16 = 5, // + sixteen v_accvgpr_read_b32 after every sixteenth op
    CAL_VMEM = 6,       // + one 16-byte-per-lane buffer load into VGPRs per four ops (B fragment halves)
    CAL_DMA = 7         // + one 16-byte-per-lane buffer load into LDS per four ops (A tile DMAs)
    // (the GEMM issues both at half that rate each: eight of each per 64 ops)
    // (the reads take sixteen accumulation registers of their own, which no op
    // writes: naming single accumulator elements of the ops in asm operands
    // makes the compiler copy whole accumulator tuples through VGPRs).  The
    // load variants move 1 KiB per instruction (the buffer ones from the
    // operand buffer, 2 MiB, L2-resident after the first pass) and consume
    // each result sixteen ops after its load.
};

// LDS the read and DMA variants use: 16 KiB per wave of the workgroup.
__shared__ __attribute__((aligned(1024))) v4i g_cal_lds[8 * 1024];

// Sixteen independent accumulators, four A and four B fragments per lane:
// each op depends only on the op sixteen places earlier, far past the
// result latency, so the matrix pipe never waits on a dependency.  The
// extra instructions touch registers no op uses in that iteration.
template <int WPS, int VAR>
__global__ void __launch_bounds__(256 * WPS, 1) mfma_ceiling_kernel(const v8i* __restrict__ frag, float* out,
                                                                   int out_len, int iters) {
    typedef __attribute__((address_space(3))) const v4i lds_v4i;
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    const int lane = threadIdx.x & 63;
    v8i a[4], b[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        a[j] = frag[(t * 8 + j) & (kCalibFrags - 1)];
        b[j] = frag[(t * 8 + 4 + j) & (kCalibFrags - 1)];
    }
    v4f acc[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] = (v4f){0.f, 0.f, 0.f, 0.f};
    float f[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) f[j] = 1.0f + 0.125f * (float)j;
    v4i r[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) r[j] = (v4i){0, 0, 0, 0};
    float d[16];  // accumulation registers the read variants read
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        d[j] = (float)j;
        if constexpr (VAR == CAL_ACC_READ || VAR == CAL_ACC_READ16) asm volatile("" : "+a"(d[j]));
    }
    // this wave's 16 KiB of LDS (a wave-uniform address)
    lds_char* const wave_lds = (lds_char*)g_cal_lds + 16384 * __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if constexpr (VAR == CAL_LDS_READ) {
        for (int j = threadIdx.x; j < 8 * 1024; j += blockDim.x) g_cal_lds[j] = (v4i){j, 1, 2, 3};
        __syncthreads();
    }
    const __amdgpu_buffer_rsrc_t rf = make_rsrc(frag, kCalibFrags * 32);
    // every operand fragment has landed before the timed stream starts
    wait_vm_lgkm0<0>();
    const int one = 127;  // E8M0 2^0
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            if constexpr (VAR == CAL_SCALED)
                asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %3 op_sel:[0,0,0] op_sel_hi:[0,0,0]"
                             : "+a"(acc[j])
                             : "v"(b[j / 4]), "v"(a[j % 4]), "v"(one));
            else
                asm volatile("v_mfma_f32_16x16x128_f8f6f4 %0, %1, %2, %0" : "+a"(acc[j]) : "v"(b[j / 4]), "v"(a[j % 4]));
            // 1 KiB per load instruction at an address that moves with the
            // iteration (16 KiB of LDS per wave, 2 MiB of the operand buffer);
            // a load's result is consumed when its register is reloaded,
            // sixteen ops later, so the stream never waits on a fresh load
            const int lo = (((it * 16 + j) * 1024) & 16383) + 16 * lane;
            const int vo = (((it * 16 + j) * 1024) & (kCalibFrags * 32 - 1)) + 16 * lane;
            if constexpr (VAR == CAL_LDS_READ) {
                asm volatile("" ::"v"(r[j]));  // a use of the whole previous result, no instruction
                r[j] = *(lds_v4i*)(wave_lds + lo);
            }
            if constexpr (VAR == CAL_VMEM) {
                if (j % 4 == 0) {  // resolved at compile time: the loop is unrolled
                    asm volatile("" ::"v"(r[j]));
                    r[j] = __builtin_amdgcn_raw_buffer_load_b128(rf, vo, 0, 0);
                }
            }
            if constexpr (VAR == CAL_DMA) {
                if (j % 4 == 0) lds_dma16(rf, wave_lds + 1024 * j, vo);
            }
            if constexpr (VAR == CAL_VALU2) {
                asm volatile("v_mul_f32 %0, %0, %1" : "+v"(f[(2 * j) & 7]) : "v"(f[(2 * j + 1) & 7]));
                asm volatile("v_mul_f32 %0, %0, %1" : "+v"(f[(2 * j + 1) & 7]) : "v"(f[(2 * j + 2) & 7]));
            }
            if constexpr (VAR == CAL_ACC_READ)
                asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(f[j & 7]) : "a"(d[j]));
            if constexpr (VAR == CAL_ACC_READ16) {
                if (j == 15) {  // resolved at compile time: the loop is unrolled
#pragma unroll
                    for (int q = 0; q < 16; ++q)
                        asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(f[q & 7]) : "a"(d[q]));
                }
            }
            // keep each op's companion instruction next to it
            __builtin_amdgcn_sched_barrier(0);
        }
        // the DMAs of the previous sixteen ops have landed (they write the
        // same LDS every iteration)
        if constexpr (VAR == CAL_DMA) wait_vm<4>();
    }
    wait_vm_lgkm0<0>();
    // the asm ops are invisible to the compiler's hazard tracking: wait out
    // the longest result latency before the accumulators are read
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        asm volatile("" : "+a"(acc[j]));
        s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
    }
    float x = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) x += f[j];
#pragma unroll
    for (int j = 0; j < 16; ++j) asm volatile("" ::"v"(r[j]));
    if (t < out_len) out[t] = s;
    // the multiplies' results stay live: a store the compiler cannot rule out
    // (no caller passes this length; out[0] exists whenever it runs)
    if (out_len == 0x7fffffff && t == 0) out[0] = x;
}

template <int WPS>
static void launch_var(int var, int grid, const v8i* f, float* out, int out_len, int iters, hipStream_t st) {
    const dim3 g(grid), b(256 * WPS);
    switch (var) {
        case CAL_SCALED: hipLaunchKernelGGL((mfma_ceiling_kernel<WPS, CAL_SCALED>), g, b, 0, st, f, out, out_len, iters); break;
        case CAL_LDS_READ: hipLaunchKernelGGL((mfma_ceiling_kernel<WPS, CAL_LDS_READ>), g, b, 0, st, f, out, out_len, iters); break;
        case CAL_VALU2: hipLaunchKernelGGL((mfma_ceiling_kernel<WPS, CAL_VALU2>), g, b, 0, st, f, out, out_len, iters); break;
        case CAL_ACC_READ: hipLaunchKernelGGL((mfma_ceiling_kernel<WPS, CAL_ACC_READ>), g, b, 0, st, f, out, out_len, iters); break;
        case CAL_ACC_READ16: hipLaunchKernelGGL((mfma_ceiling_kernel<WPS, CAL_ACC_READ16>), g, b, 0, st, f, out, out_len, iters); break;
        case CAL_VMEM: hipLaunchKernelGGL((mfma_ceiling_kernel<WPS, CAL_VMEM>), g, b, 0, st, f, out, out_len, iters); break;
        case CAL_DMA: hipLaunchKernelGGL((mfma_ceiling_kernel<WPS, CAL_DMA>), g, b, 0, st, f, out, out_len, iters); break;
        default: hipLaunchKernelGGL((mfma_ceiling_kernel<WPS, CAL_PLAIN>), g, b, 0, st, f, out, out_len, iters); break;
    }
}

// One workgroup of 4 * wps waves per CU; returns the grid size through *grid.
hipError_t launch_mfma_ceiling(const uint8_t* frag, float* out, int out_len, int iters, int wps, int variant,
                               int* grid, hipStream_t st) {
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    *grid = cus;
    const v8i* f = reinterpret_cast<const v8i*>(frag);
    if (wps == 1) launch_var<1>(variant, cus, f, out, out_len, iters, st);
    else launch_var<2>(variant, cus, f, out, out_len, iters, st);
    return hipGetLastError();
}

}  // namespace dmm
