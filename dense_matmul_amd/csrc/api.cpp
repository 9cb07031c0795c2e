// api.cpp -- the C ABI declared in include/dmm.h: argument rules, device
// check and dispatch to the gfx950 kernels.  Every rule is checked before
// any HIP call, so invalid arguments never reach a kernel.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "dmm.h"

namespace dmm {
hipError_t launch_gemm_a8w8(int mode, int tile, const uint8_t* a, const uint8_t* b, const void* sa, const void* sb, uint16_t* c,
                            int m, int n, int k, hipStream_t stream);
hipError_t launch_gemm_a8w8_gathered(const uint8_t* a, const uint8_t* b, const float* sa, const float* sb,
                                     uint16_t* c, int m, int n, int k, const uint32_t* flags, int src_rows,
                                     int nchunks, int own, uint32_t epoch, long long spin_limit, int* status,
                                     hipStream_t stream);
hipError_t launch_gemm_bf16(const uint16_t* a, const uint16_t* b, uint16_t* c, int m, int n, int k, int tile,
                            hipStream_t st);
hipError_t launch_quantize_rows(const float* x, uint8_t* q, float* s, int rows, int cols, hipStream_t st);
hipError_t launch_quantize_rows_bf16(const uint16_t* x, uint8_t* q, float* s, int rows, int cols, hipStream_t st);
hipError_t launch_quantize_blockscale_a(const float* x, uint8_t* q, float* s, int m, int k, hipStream_t st);
hipError_t launch_quantize_blockscale_b(const float* x, uint8_t* q, float* s, int n, int k, hipStream_t st);
hipError_t launch_quantize_mxfp8(const float* x, uint8_t* q, uint8_t* s, int rows, int k, hipStream_t st);
hipError_t launch_preshuffle_b(const uint8_t* b, uint8_t* out, int n, int k, hipStream_t st);
}  // namespace dmm

namespace {

thread_local char g_err[512];

dmm_status fail(dmm_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

constexpr int64_t kLimit = (int64_t)1 << 31;  // operands are addressed with 32-bit buffer offsets

bool bad_ptr(const void* p) { return p == nullptr || ((uintptr_t)p & 15u) != 0; }

#define REQUIRE(cond, ...)                                 \
    do {                                                   \
        if (!(cond)) return fail(DMM_EINVAL, __VA_ARGS__); \
    } while (0)

#define REQUIRE_PTR(p) REQUIRE(!bad_ptr(p), "%s: pointer is null or not 16-byte aligned", #p)

dmm_status check_device() {
    static int state[64];  // 0 unknown, 1 gfx950, 2 other
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(DMM_ENODEV, "no HIP device is available");
    if (dev < 0 || dev >= 64) return fail(DMM_ENODEV, "device index %d out of range", dev);
    if (state[dev] == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return fail(DMM_ENODEV, "hipGetDeviceProperties failed");
        state[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        if (state[dev] == 2) return fail(DMM_ENODEV, "device %d is %s, this library is built for gfx950", dev, prop.gcnArchName);
    }
    return state[dev] == 1 ? DMM_OK : fail(DMM_ENODEV, "device %d is not gfx950", dev);
}

dmm_status launched(hipError_t e) {
    if (e != hipSuccess) return fail(DMM_ELAUNCH, "launch failed: %s", hipGetErrorString(e));
    g_err[0] = 0;
    return DMM_OK;
}

dmm_status check_gemm_shape(int64_t m, int64_t n, int64_t k) {
    REQUIRE(m >= 1, "m must be >= 1 (got %lld)", (long long)m);
    REQUIRE(n >= 16 && n % 16 == 0, "n must be a positive multiple of 16 (got %lld)", (long long)n);
    REQUIRE(k >= 128 && k % 128 == 0, "k must be a positive multiple of 128 (got %lld)", (long long)k);
    REQUIRE((m + 256) * k < kLimit, "a is too large: (m + 256) * k must be < 2^31");
    REQUIRE((n + 256) * k < kLimit, "b is too large: (n + 256) * k must be < 2^31");
    REQUIRE((m + 256) * n * 2 < kLimit, "c is too large: (m + 256) * n * 2 must be < 2^31");
    return DMM_OK;
}

dmm_status gemm_common(int mode, int tile, const uint8_t* a, const uint8_t* b, const void* sa, const void* sb,
                       uint16_t* c, int64_t m, int64_t n, int64_t k, void* stream) {
    REQUIRE_PTR(a);
    REQUIRE_PTR(b);
    REQUIRE_PTR(sa);
    REQUIRE_PTR(sb);
    REQUIRE_PTR(c);
    dmm_status s = check_gemm_shape(m, n, k);
    if (s != DMM_OK) return s;
    if (mode == 1) REQUIRE((k / 128) * (m + 256) * 4 < kLimit, "a_scale is too large");
    if (mode == 2) REQUIRE((k / 32) * (m + 256) < kLimit && (k / 32) * (n + 256) < kLimit, "scales are too large");
    if ((s = check_device()) != DMM_OK) return s;
    return launched(dmm::launch_gemm_a8w8(mode, tile, a, b, sa, sb, c, (int)m, (int)n, (int)k, (hipStream_t)stream));
}

}  // namespace

extern "C" {

const char* dmm_status_str(int status) {
    switch (status) {
        case DMM_OK: return "DMM_OK";
        case DMM_EINVAL: return "DMM_EINVAL";
        case DMM_ENODEV: return "DMM_ENODEV";
        case DMM_ELAUNCH: return "DMM_ELAUNCH";
        default: return "DMM_UNKNOWN";
    }
}

const char* dmm_last_error(void) { return g_err; }

dmm_status quantize_per_token(const float* x, uint8_t* q, float* scale, int64_t rows, int64_t cols, void* stream) {
    REQUIRE_PTR(x);
    REQUIRE_PTR(q);
    REQUIRE_PTR(scale);
    REQUIRE(rows >= 1, "rows must be >= 1");
    REQUIRE(cols >= 16 && cols % 16 == 0, "cols must be a positive multiple of 16 (got %lld)", (long long)cols);
    REQUIRE(rows * cols * 4 < ((int64_t)1 << 40), "x is too large");
    REQUIRE(rows < kLimit && cols < kLimit, "rows and cols must be < 2^31");
    dmm_status s = check_device();
    if (s != DMM_OK) return s;
    return launched(dmm::launch_quantize_rows(x, q, scale, (int)rows, (int)cols, (hipStream_t)stream));
}

dmm_status quantize_per_token_bf16(const uint16_t* x, uint8_t* q, float* scale, int64_t rows, int64_t cols,
                                   void* stream) {
    REQUIRE_PTR(x);
    REQUIRE_PTR(q);
    REQUIRE_PTR(scale);
    REQUIRE(rows >= 1, "rows must be >= 1");
    REQUIRE(cols >= 16 && cols % 16 == 0, "cols must be a positive multiple of 16 (got %lld)", (long long)cols);
    REQUIRE(rows * cols * 2 < ((int64_t)1 << 40), "x is too large");
    REQUIRE(rows < kLimit && cols < kLimit, "rows and cols must be < 2^31");
    dmm_status s = check_device();
    if (s != DMM_OK) return s;
    return launched(dmm::launch_quantize_rows_bf16(x, q, scale, (int)rows, (int)cols, (hipStream_t)stream));
}

dmm_status quantize_blockscale_a(const float* x, uint8_t* q, float* scale, int64_t m, int64_t k, void* stream) {
    REQUIRE_PTR(x);
    REQUIRE_PTR(q);
    REQUIRE_PTR(scale);
    REQUIRE(m >= 1, "m must be >= 1");
    REQUIRE(k >= 128 && k % 128 == 0, "k must be a positive multiple of 128 (got %lld)", (long long)k);
    REQUIRE(m < kLimit && k < kLimit && (k / 128) * m < kLimit, "m and k must be < 2^31");
    dmm_status s = check_device();
    if (s != DMM_OK) return s;
    return launched(dmm::launch_quantize_blockscale_a(x, q, scale, (int)m, (int)k, (hipStream_t)stream));
}

dmm_status quantize_blockscale_b(const float* x, uint8_t* q, float* scale, int64_t n, int64_t k, void* stream) {
    REQUIRE_PTR(x);
    REQUIRE_PTR(q);
    REQUIRE_PTR(scale);
    REQUIRE(n >= 16 && n % 16 == 0, "n must be a positive multiple of 16 (got %lld)", (long long)n);
    REQUIRE(k >= 128 && k % 128 == 0, "k must be a positive multiple of 128 (got %lld)", (long long)k);
    REQUIRE(n < kLimit && k < kLimit && (k / 128) < 65536, "n and k are too large");
    dmm_status s = check_device();
    if (s != DMM_OK) return s;
    return launched(dmm::launch_quantize_blockscale_b(x, q, scale, (int)n, (int)k, (hipStream_t)stream));
}

dmm_status quantize_mxfp8(const float* x, uint8_t* q, uint8_t* scale, int64_t rows, int64_t k, void* stream) {
    REQUIRE_PTR(x);
    REQUIRE_PTR(q);
    REQUIRE_PTR(scale);
    REQUIRE(rows >= 1, "rows must be >= 1");
    REQUIRE(k >= 128 && k % 128 == 0, "k must be a positive multiple of 128 (got %lld)", (long long)k);
    REQUIRE(rows < kLimit && k < kLimit && (k / 32) * rows < kLimit, "rows and k are too large");
    dmm_status s = check_device();
    if (s != DMM_OK) return s;
    return launched(dmm::launch_quantize_mxfp8(x, q, scale, (int)rows, (int)k, (hipStream_t)stream));
}

dmm_status preshuffle_b(const uint8_t* b, uint8_t* b_shuf, int64_t n, int64_t k, void* stream) {
    REQUIRE_PTR(b);
    REQUIRE_PTR(b_shuf);
    REQUIRE(n >= 16 && n % 16 == 0, "n must be a positive multiple of 16 (got %lld)", (long long)n);
    REQUIRE(k >= 128 && k % 128 == 0, "k must be a positive multiple of 128 (got %lld)", (long long)k);
    REQUIRE((n + 256) * k < kLimit, "b is too large: (n + 256) * k must be < 2^31");
    const uintptr_t b0 = (uintptr_t)b, s0 = (uintptr_t)b_shuf, len = (uintptr_t)(n * k);
    REQUIRE(b0 + len <= s0 || s0 + len <= b0, "b and b_shuf overlap");
    dmm_status s = check_device();
    if (s != DMM_OK) return s;
    return launched(dmm::launch_preshuffle_b(b, b_shuf, (int)n, (int)k, (hipStream_t)stream));
}

dmm_status gemm_a8w8_ptpc(const uint8_t* a, const uint8_t* b_shuf, const float* a_scale, const float* b_scale,
                          uint16_t* c, int64_t m, int64_t n, int64_t k, void* stream) {
    return gemm_common(0, 0, a, b_shuf, a_scale, b_scale, c, m, n, k, stream);
}

dmm_status gemm_a8w8_ptpc_tile(const uint8_t* a, const uint8_t* b_shuf, const float* a_scale, const float* b_scale,
                               uint16_t* c, int64_t m, int64_t n, int64_t k, int tile, void* stream) {
    REQUIRE(tile >= 0 && tile <= 3, "tile must be 0 (auto), 1 (256x256), 2 (128x256) or 3 (128x128) (got %d)", tile);
    return gemm_common(0, tile, a, b_shuf, a_scale, b_scale, c, m, n, k, stream);
}

dmm_status gemm_a8w8_ptpc_gathered(const uint8_t* a, const uint8_t* b_shuf, const float* a_scale,
                                   const float* b_scale, uint16_t* c, int64_t m, int64_t n, int64_t k,
                                   const uint32_t* flags, int64_t src_rows, int nchunks, int own, uint32_t epoch,
                                   int64_t spin_limit, int* status, void* stream) {
    REQUIRE_PTR(a);
    REQUIRE_PTR(b_shuf);
    REQUIRE_PTR(a_scale);
    REQUIRE_PTR(b_scale);
    REQUIRE_PTR(c);
    dmm_status s = check_gemm_shape(m, n, k);
    if (s != DMM_OK) return s;
    REQUIRE(flags != nullptr && (uintptr_t)flags % 4 == 0, "flags: null or not 4-byte aligned");
    REQUIRE(status != nullptr && (uintptr_t)status % 4 == 0, "status: null or not 4-byte aligned");
    REQUIRE(nchunks >= 1, "nchunks must be >= 1 (got %d)", nchunks);
    REQUIRE(src_rows >= 256 && src_rows % (256 * (int64_t)nchunks) == 0,
            "src_rows must be a positive multiple of 256 * nchunks (got %lld)", (long long)src_rows);
    REQUIRE(m % src_rows == 0, "m must be a multiple of src_rows (got m %lld, src_rows %lld)", (long long)m,
            (long long)src_rows);
    REQUIRE((m / src_rows) * nchunks <= 64, "at most 64 bands (sources x nchunks)");
    REQUIRE(own >= 0 && own < m / src_rows, "own must name a source slab (got %d)", own);
    REQUIRE(spin_limit >= 0, "spin_limit must be >= 0");
    if ((s = check_device()) != DMM_OK) return s;
    return launched(dmm::launch_gemm_a8w8_gathered(a, b_shuf, a_scale, b_scale, c, (int)m, (int)n, (int)k, flags,
                                                   (int)src_rows, nchunks, own, epoch, (long long)spin_limit,
                                                   status, (hipStream_t)stream));
}

dmm_status gemm_a8w8_blockscale(const uint8_t* a, const uint8_t* b_shuf, const float* a_scale, const float* b_scale,
                                uint16_t* c, int64_t m, int64_t n, int64_t k, void* stream) {
    return gemm_common(1, 0, a, b_shuf, a_scale, b_scale, c, m, n, k, stream);
}

dmm_status gemm_a8w8_blockscale_tile(const uint8_t* a, const uint8_t* b_shuf, const float* a_scale,
                                     const float* b_scale, uint16_t* c, int64_t m, int64_t n, int64_t k, int tile,
                                     void* stream) {
    REQUIRE(tile >= 0 && tile <= 2, "tile must be 0 (auto), 1 (128x256) or 2 (128x128) (got %d)", tile);
    return gemm_common(1, tile, a, b_shuf, a_scale, b_scale, c, m, n, k, stream);
}

dmm_status gemm_a8w8_mxfp8(const uint8_t* a, const uint8_t* b_shuf, const uint8_t* a_scale, const uint8_t* b_scale,
                           uint16_t* c, int64_t m, int64_t n, int64_t k, void* stream) {
    return gemm_common(2, 0, a, b_shuf, a_scale, b_scale, c, m, n, k, stream);
}

dmm_status gemm_a8w8_mxfp8_tile(const uint8_t* a, const uint8_t* b_shuf, const uint8_t* a_scale,
                                const uint8_t* b_scale, uint16_t* c, int64_t m, int64_t n, int64_t k, int tile,
                                void* stream) {
    REQUIRE(tile >= 0 && tile <= 2, "tile must be 0 (auto), 1 (256x256) or 2 (256x128) (got %d)", tile);
    return gemm_common(2, tile, a, b_shuf, a_scale, b_scale, c, m, n, k, stream);
}

dmm_status gemm_bf16_tile(const uint16_t* a, const uint16_t* b, uint16_t* c, int64_t m, int64_t n, int64_t k,
                          int tile, void* stream) {
    REQUIRE_PTR(a);
    REQUIRE_PTR(b);
    REQUIRE_PTR(c);
    REQUIRE(tile >= 0 && tile <= 2, "tile must be 0 (auto), 1 (128x128) or 2 (64x64) (got %d)", tile);
    REQUIRE(m >= 1, "m must be >= 1 (got %lld)", (long long)m);
    REQUIRE(n >= 16 && n % 16 == 0, "n must be a positive multiple of 16 (got %lld)", (long long)n);
    REQUIRE(k >= 64 && k % 64 == 0, "k must be a positive multiple of 64 (got %lld)", (long long)k);
    REQUIRE((m + 256) * k * 2 < kLimit && (n + 256) * k * 2 < kLimit && (m + 256) * n * 2 < kLimit,
            "operands are too large (each must be < 2^31 bytes with a 256-row margin)");
    dmm_status s = check_device();
    if (s != DMM_OK) return s;
    return launched(dmm::launch_gemm_bf16(a, b, c, (int)m, (int)n, (int)k, tile, (hipStream_t)stream));
}

dmm_status gemm_bf16(const uint16_t* a, const uint16_t* b, uint16_t* c, int64_t m, int64_t n, int64_t k, void* stream) {
    return gemm_bf16_tile(a, b, c, m, n, k, 0, stream);
}

}  // extern "C"
