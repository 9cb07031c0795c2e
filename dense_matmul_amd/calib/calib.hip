// calib.hip -- how fast gfx950 issues the fp8 GEMM's matrix instruction when
// nothing else is in the way, and what each kind of instruction the GEMM
// interleaves with it costs: every wave runs a long stream of back-to-back,
// independent fp8 matrix ops on e4m3 operands it loaded once, with one or two
// waves per SIMD, optionally with one kind of extra instruction after each
// op.  The benchmark reports these next to the published dense fp8 peak, so
// that the GEMM's own figure can be read against what the part reaches under
// load (clock included).
//
// A second kernel measures the per-CU rates of vector-memory loads and
// stores (calib_memory_rate).
//
// This is measurement tooling for the benchmark, built into its own library
// (libdmm_calib.so) with its own C entry point; it is not part of libdmm and
// not a step of the GEMM.
#include "common.h"

#include <stdint.h>

namespace dmm {

constexpr int kCalibFrags = 65536;  // 32-byte operand fragments read from the caller's buffer (2 MiB)

// Variants (the `variant` argument of calib_mfma_ceiling_fp8).  Every
// variant does the same FLOPs per loop iteration: sixteen 16x16x128 ops, or
// eight 32x32x64 ops (each twice the work), so the extra instructions below
// come at the same rate per FLOP in both shapes.
enum {
    CAL_PLAIN = 0,      // v_mfma_f32_16x16x128_f8f6f4 alone (the ptpc / blockscale instruction)
    CAL_SCALED = 1,     // the mxfp8 form, E8M0 scales 127 (x1) on both operands
    CAL_LDS_READ = 2,   // + one ds_read_b128 per op (an A fragment half)
    CAL_VALU2 = 3,      // + two v_mul_f32 per op (epilogue scaling)
    CAL_ACC_READ = 4,   // + one v_accvgpr_read_b32 per op (an epilogue's accumulator read-out)
    CAL_ACC_READ16 = 5, // + sixteen v_accvgpr_read_b32 after every sixteenth op
    CAL_VMEM = 6,       // + one 16-byte-per-lane buffer load into VGPRs per four ops (B fragment halves)
    CAL_DMA = 7,        // + one 16-byte-per-lane buffer load into LDS per four ops (A tile DMAs)
    CAL_W32 = 8,        // v_mfma_f32_32x32x64_f8f6f4 alone
    CAL_W32_LDS = 9,    // 32x32x64 + two ds_read_b128 per op
    CAL_W32_VMEM = 10,  // 32x32x64 + one buffer load into VGPRs per two ops
    CAL_W32_DMA = 11,   // 32x32x64 + one buffer load into LDS per two ops
    CAL_NVARIANTS = 12
    // (the fp8 GEMM issues the two load kinds at half the CAL_VMEM / CAL_DMA
    // rate each: eight of each per 64 ops).  The accumulator reads take
    // sixteen accumulation registers of their own, which no op writes
    // (naming single accumulator elements of the ops in asm operands makes
    // the compiler copy whole accumulator tuples through VGPRs).  The load
    // variants move 1 KiB per instruction (the buffer ones from the operand
    // buffer, 2 MiB, L2-resident after the first pass) and consume each
    // result when its register is reloaded, one iteration later.
};

template <int VAR>
constexpr bool kW32 = VAR >= CAL_W32;

// LDS the read and DMA variants use: 16 KiB per wave of the workgroup.
__shared__ __attribute__((aligned(1024))) v4i g_cal_lds[8 * 1024];

typedef float v16f __attribute__((ext_vector_type(16)));

// Sixteen independent 16x16 accumulators (or eight 32x32 ones), four A and
// four B fragments per lane: each op depends only on the op one iteration
// earlier, far past the result latency, so the matrix pipe never waits on a
// dependency.  The extra instructions touch registers no op uses in that
// iteration.
template <int WPS, int VAR>
__global__ void __launch_bounds__(256 * WPS, 1) mfma_ceiling_kernel(const v8i* __restrict__ frag, float* out,
                                                                   int out_len, int iters) {
    typedef __attribute__((address_space(3))) const v4i lds_v4i;
    constexpr int OPS = kW32<VAR> ? 8 : 16;  // ops per iteration
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    const int lane = threadIdx.x & 63;
    v8i a[4], b[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        a[j] = frag[(t * 8 + j) & (kCalibFrags - 1)];
        b[j] = frag[(t * 8 + 4 + j) & (kCalibFrags - 1)];
    }
    v4f acc[16];
    v16f acc32[8];
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc32[j][e] = 0.f;
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
    if constexpr (VAR == CAL_LDS_READ || VAR == CAL_W32_LDS) {
        for (int j = threadIdx.x; j < 8 * 1024; j += blockDim.x) g_cal_lds[j] = (v4i){j, 1, 2, 3};
        __syncthreads();
    }
    const __amdgpu_buffer_rsrc_t rf = make_rsrc(frag, kCalibFrags * 32);
    // every operand fragment has landed before the timed stream starts
    wait_vm_lgkm0<0>();
    const int one = 127;  // E8M0 2^0
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < OPS; ++j) {
            if constexpr (kW32<VAR>)
                asm volatile("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0" : "+a"(acc32[j]) : "v"(b[j / 2]), "v"(a[j % 4]));
            else if constexpr (VAR == CAL_SCALED)
                asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %3 op_sel:[0,0,0] op_sel_hi:[0,0,0]"
                             : "+a"(acc[j])
                             : "v"(b[j / 4]), "v"(a[j % 4]), "v"(one));
            else
                asm volatile("v_mfma_f32_16x16x128_f8f6f4 %0, %1, %2, %0" : "+a"(acc[j]) : "v"(b[j / 4]), "v"(a[j % 4]));
            // 1 KiB per load instruction at an address that moves with the
            // iteration (16 KiB of LDS per wave, 2 MiB of the operand buffer);
            // a load's result is consumed when its register is reloaded, one
            // iteration later, so the stream never waits on a fresh load
            if constexpr (VAR == CAL_LDS_READ || VAR == CAL_W32_LDS) {
                constexpr int PER = VAR == CAL_W32_LDS ? 2 : 1;
#pragma unroll
                for (int q = 0; q < PER; ++q) {
                    const int slot = PER * j + q;
                    const int lo = (((it * 16 + slot) * 1024) & 16383) + 16 * lane;
                    asm volatile("" ::"v"(r[slot]));  // a use of the whole previous result, no instruction
                    r[slot] = *(lds_v4i*)(wave_lds + lo);
                }
            }
            // the buffer loads: one per four 16x16 ops or per two 32x32 ops
            constexpr int EVERY = kW32<VAR> ? 2 : 4;
            if constexpr (VAR == CAL_VMEM || VAR == CAL_W32_VMEM || VAR == CAL_DMA || VAR == CAL_W32_DMA) {
                if (j % EVERY == 0) {  // resolved at compile time: the loop is unrolled
                    const int slot = 4 * j / EVERY;
                    const int vo = (((it * 16 + slot) * 1024) & (kCalibFrags * 32 - 1)) + 16 * lane;
                    if constexpr (VAR == CAL_VMEM || VAR == CAL_W32_VMEM) {
                        asm volatile("" ::"v"(r[slot]));
                        r[slot] = __builtin_amdgcn_raw_buffer_load_b128(rf, vo, 0, 0);
                    } else {
                        lds_dma16(rf, wave_lds + 1024 * slot, vo);
                    }
                }
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
        // the DMAs of the previous iteration have landed (they write the
        // same LDS every iteration)
        if constexpr (VAR == CAL_DMA || VAR == CAL_W32_DMA) wait_vm<4>();
    }
    wait_vm_lgkm0<0>();
    // the asm ops are invisible to the compiler's hazard tracking: wait out
    // the longest result latency before the accumulators are read
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    float s = 0.f;
    if constexpr (kW32<VAR>) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            asm volatile("" : "+a"(acc32[j]));
#pragma unroll
            for (int e = 0; e < 16; ++e) s += acc32[j][e];
        }
    } else {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            asm volatile("" : "+a"(acc[j]));
            s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
        }
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

template <int WPS, int VAR = 0>
static void launch_var(int var, int grid, const v8i* f, float* out, int out_len, int iters, hipStream_t st) {
    if constexpr (VAR < CAL_NVARIANTS) {
        if (var == VAR)
            hipLaunchKernelGGL((mfma_ceiling_kernel<WPS, VAR>), dim3(grid), dim3(256 * WPS), 0, st, f, out, out_len,
                               iters);
        else
            launch_var<WPS, VAR + 1>(var, grid, f, out, out_len, iters, st);
    }
}


// ------------------------------------------------------------------ memory
// Per-CU vector-memory rates, the other resource the GEMMs run into: one
// workgroup of four waves per CU streams 1 KiB buffer instructions (16 bytes
// per lane) through its own region of the caller's buffer, sixteen in flight
// per wave.  Loads go into VGPRs or through the direct-to-LDS path; stores
// write their region in whole 128-byte lines or in the pattern of the fp8
// GEMM's 256-wide epilogue (each instruction 64 bytes of each of 16 rows,
// rows 14336 bytes apart: N = 7168 bf16).  Wave 0 records s_memtime (shader
// cycles) at its start and end.
enum { MEM_LOAD_VGPR = 0, MEM_LOAD_LDS = 1, MEM_STORE_LINES = 2, MEM_STORE_EPILOGUE = 3, MEM_NKINDS = 4 };
constexpr uint32_t kEpiRowBytes = 14336;
constexpr uint32_t kEpiBlocks = 17;  // 16-row blocks the epilogue pattern cycles through (< 4 MiB)

// 96 KiB: more than half the CU's LDS, so no CU holds two workgroups
__shared__ __attribute__((aligned(1024))) v4i g_mem_lds[6 * 1024];

template <int KIND, int AUX>
__global__ void __launch_bounds__(256, 1) memory_rate_kernel(uint8_t* buf, uint32_t region, int iters, uint64_t* cyc) {
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(buf + (size_t)blockIdx.x * region, region);
    lds_char* wl = (lds_char*)g_mem_lds + w * 16384;
    const v4i val = (v4i){lane, w, (int)blockIdx.x, 7};
    v4i r[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) r[j] = (v4i){0, 0, 0, 0};
    if (threadIdx.x == 0) g_mem_lds[0] = val;  // every kind holds the LDS block
    __syncthreads();
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    uint32_t k = (uint32_t)w * 16u;  // instruction index: the four waves interleave in the region
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const uint32_t kk = k + (uint32_t)j;
            if constexpr (KIND == MEM_STORE_EPILOGUE) {
                const int vo = (int)((kk % (kEpiRowBytes / 64u)) * 64u + ((kk / (kEpiRowBytes / 64u)) % kEpiBlocks) * 16u *
                               kEpiRowBytes) + (lane >> 2) * (int)kEpiRowBytes + (lane & 3) * 16;
                __builtin_amdgcn_raw_buffer_store_b128(val, rs, vo, 0, AUX);
            } else {
                const int vo = (int)((kk * 1024u) & (region - 1u)) + 16 * lane;
                if constexpr (KIND == MEM_STORE_LINES) {
                    __builtin_amdgcn_raw_buffer_store_b128(val, rs, vo, 0, AUX);
                } else if constexpr (KIND == MEM_LOAD_VGPR) {
                    asm volatile("" ::"v"(r[j]));  // the previous result is used: sixteen loads in flight
                    r[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, vo, 0, 0);
                } else {
                    lds_dma16(rs, wl + 1024 * j, vo);
                }
            }
        }
        k += 64u;
    }
    wait_vm_lgkm0<0>();
    __syncthreads();
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
#pragma unroll
    for (int j = 0; j < 16; ++j) asm volatile("" ::"v"(r[j]));
    if (threadIdx.x == 0) {
        cyc[2 * blockIdx.x] = t0;
        cyc[2 * blockIdx.x + 1] = t1;
    }
}

template <int KIND = 0>
static void launch_mem(int kind, bool nt_sc1, int grid, uint8_t* buf, uint32_t region, int iters, uint64_t* cyc,
                       hipStream_t st) {
    if constexpr (KIND < MEM_NKINDS) {
        if (kind != KIND) {
            launch_mem<KIND + 1>(kind, nt_sc1, grid, buf, region, iters, cyc, st);
        } else if (nt_sc1) {
            hipLaunchKernelGGL((memory_rate_kernel<KIND, 18>), dim3(grid), dim3(256), 0, st, buf, region, iters, cyc);
        } else {
            hipLaunchKernelGGL((memory_rate_kernel<KIND, 0>), dim3(grid), dim3(256), 0, st, buf, region, iters, cyc);
        }
    }
}

}  // namespace dmm

namespace {
thread_local char g_calib_err[256];
}

extern "C" {

// What went wrong in the last call that returned non-zero ("" if none).
const char* calib_last_error(void) { return g_calib_err; }

// One launch of the issue-ceiling kernel: one workgroup per compute unit,
// with waves_per_simd (1 or 2) waves on each of its four SIMDs; every wave
// loads four A and four B fragments (32 bytes per lane each) from frag and
// runs iters iterations of the variant's ops (see the enum above), then
// writes the sum of its accumulators to out[thread] for threads below
// out_len.  One launch does
//     2 * 16 * 16 * 128 * 16 * iters * (*workgroups) * 4 * waves_per_simd
// FLOPs whatever the variant.  *workgroups (host, may be NULL) receives the
// grid size.  frag: device, at least 2 MiB of e4m3 codes (the operand bytes
// change the power the part draws, so pass real codes); out: device fp32
// [out_len].  Returns 0, 1 for a rule broken (1 <= iters <= 2^20;
// waves_per_simd 1 or 2; 0 <= variant < 12; frag_bytes >= 2 MiB;
// 1 <= out_len < 2^31; frag and out non-null and 16-byte aligned) before
// any HIP call, or 3 when the HIP runtime reports an error.
int calib_mfma_ceiling_fp8(const uint8_t* frag, int64_t frag_bytes, float* out, int64_t out_len, int iters,
                           int waves_per_simd, int variant, int* workgroups, void* stream) {
    auto fail = [](int code, const char* msg) {
        snprintf(g_calib_err, sizeof g_calib_err, "%s", msg);
        return code;
    };
    if (frag == nullptr || ((uintptr_t)frag & 15u)) return fail(1, "frag: pointer is null or not 16-byte aligned");
    if (out == nullptr || ((uintptr_t)out & 15u)) return fail(1, "out: pointer is null or not 16-byte aligned");
    if (frag_bytes < (int64_t)dmm::kCalibFrags * 32) return fail(1, "frag must hold at least 2 MiB");
    if (out_len < 1 || out_len >= ((int64_t)1 << 31)) return fail(1, "out_len must be in [1, 2^31)");
    if (iters < 1 || iters > (1 << 20)) return fail(1, "iters must be in [1, 2^20]");
    if (waves_per_simd != 1 && waves_per_simd != 2) return fail(1, "waves_per_simd must be 1 or 2");
    if (variant < 0 || variant >= dmm::CAL_NVARIANTS) return fail(1, "variant must be in [0, 11]");
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return fail(3, "no HIP device");
    const dmm::v8i* f = reinterpret_cast<const dmm::v8i*>(frag);
    if (waves_per_simd == 1) dmm::launch_var<1>(variant, cus, f, out, (int)out_len, iters, (hipStream_t)stream);
    else dmm::launch_var<2>(variant, cus, f, out, (int)out_len, iters, (hipStream_t)stream);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(3, hipGetErrorString(e));
    if (workgroups) *workgroups = cus;
    g_calib_err[0] = 0;
    return 0;
}

// One launch of the memory-rate kernel: `grid` workgroups (1 .. the CU
// count), workgroup g on bytes [g region, (g+1) region) of buf, each of its
// four waves issuing 16 iters 1 KiB instructions of `kind` (0 loads into
// VGPRs, 1 loads into LDS, 2 stores of whole lines, 3 stores in the GEMM
// epilogue's half-line pattern) with the default cache policy, or for
// stores with nt_sc1 the non-temporal device-scope one the GEMM uses at
// K < 4096.  cycles (device, 2 grid uint64) receives each workgroup's
// s_memtime at start and end.  region: a power of two, at least 64 KiB (4 MiB
// for kind 3) and at most 1 GiB; buf (device, 16-byte aligned) must hold
// grid * region bytes.  Returns 0, 1 for a rule broken (before any HIP
// call), 3 when the HIP runtime reports an error.
int calib_memory_rate(uint8_t* buf, int64_t buf_bytes, int64_t region, int iters, int kind, int nt_sc1, int grid,
                      uint64_t* cycles, void* stream) {
    auto fail = [](int code, const char* msg) {
        snprintf(g_calib_err, sizeof g_calib_err, "%s", msg);
        return code;
    };
    if (buf == nullptr || ((uintptr_t)buf & 15u)) return fail(1, "buf: pointer is null or not 16-byte aligned");
    if (cycles == nullptr || ((uintptr_t)cycles & 7u)) return fail(1, "cycles: pointer is null or not 8-byte aligned");
    if (kind < 0 || kind >= dmm::MEM_NKINDS) return fail(1, "kind must be in [0, 3]");
    const int64_t min_region = kind == dmm::MEM_STORE_EPILOGUE ? (int64_t)4 << 20 : (int64_t)64 << 10;
    if (region < min_region || region > ((int64_t)1 << 30) || (region & (region - 1)))
        return fail(1, "region must be a power of two in [64 KiB (4 MiB for kind 3), 1 GiB]");
    if (iters < 1 || iters > (1 << 16)) return fail(1, "iters must be in [1, 2^16]");
    int dev = 0, cus = 0;
    const hipError_t ed = hipGetDevice(&dev);
    const hipError_t ea = ed == hipSuccess ? hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) : ed;
    if (ea != hipSuccess) return fail(3, hipGetErrorString(ea));
    if (grid < 1 || grid > cus) return fail(1, "grid must be in [1, the CU count]");
    if (buf_bytes < (int64_t)grid * region) return fail(1, "buf must hold grid * region bytes");
    dmm::launch_mem(kind, nt_sc1 != 0, grid, buf, (uint32_t)region, iters, cycles, (hipStream_t)stream);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(3, hipGetErrorString(e));
    g_calib_err[0] = 0;
    return 0;
}

}  // extern "C"
