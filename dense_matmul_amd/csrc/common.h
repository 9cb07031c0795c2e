// common.h -- device helpers shared by the libdmm kernels (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dmm {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) char lds_char;

// Raw buffer resource over [base, base + bytes).  Loads past the end return
// zero and stores past the end are dropped, which is how the kernels mask
// the partial last row and column tiles.  Word 3 (0x00020000) selects the
// 32-bit untyped format used for raw buffer access on gfx9-family parts.
// Every descriptor the kernels build is wave-uniform: its base is a kernel
// argument and its extent goes through readfirstlane, so that the compiler
// knows it too (where it cannot prove it, it wraps each load in a loop over
// the distinct descriptors of the wave's lanes).  Tile-dependent positions
// belong in the per-lane offset, not in the base.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                             __builtin_amdgcn_readfirstlane((int)bytes), 0x00020000);
}

// Direct global -> LDS load of 16 bytes per lane through a buffer
// descriptor: lane l writes lds + 16 l (lds must be wave-uniform); the
// address is the descriptor's base + voffset + soffset (soffset uniform).  The host
// compilation pass cannot type-check this builtin inside device function
// templates, so the call exists in the device pass only; the host pass never
// executes device code.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, lds_char* lds, int voffset, int soffset = 0) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, voffset, soffset, 0, 0);
#else
    (void)r;
    (void)lds;
    (void)voffset;
    (void)soffset;
#endif
}

// s_waitcnt immediate for the gfx9 encoding: vmcnt in bits [3:0] and
// [15:14], expcnt [6:4], lgkmcnt [11:8]; fields set to their maximum do not
// wait.
constexpr int waitcnt_imm(int vm, int lgkm) {
    return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | ((lgkm & 15) << 8);
}

// Wait until at most VM vector-memory operations of this wave are
// outstanding and all of its LDS / scalar-memory operations have returned.
template <int VM>
__device__ __forceinline__ void wait_vm_lgkm0() {
    static_assert(VM >= 0 && VM <= 63, "vmcnt is a 6-bit field");
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(VM, 0));
}

template <int VM>
__device__ __forceinline__ void wait_vm() {
    static_assert(VM >= 0 && VM <= 63, "vmcnt is a 6-bit field");
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(VM, 15));
}

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }
__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Two floats to a packed pair of bf16 (round to nearest even).
__device__ __forceinline__ int pack_bf16(float lo, float hi) {
    v2f f = {lo, hi};
    bf2 h = __builtin_convertvector(f, bf2);
    return __builtin_bit_cast(int, h);
}

}  // namespace dmm
