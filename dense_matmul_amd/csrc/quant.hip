// quant.hip -- E4M3 quantisers and the B preshuffle for gfx950.
//
// Per-token quantisation with scale amax / 448 is the activation path of
// mori PR 809 ("mori.ops.ag_gemm", section Using it); blockscale (1x128 for
// A, 128x128 for B) and mxfp8 (E8M0 per 32 K) are the other two modes of
// mori PR 785 (section Cost).  All kernels are HBM-bound streams: fully
// coalesced 16-byte loads, wave-level max reductions through lane shuffles,
// and the quantised bytes written 4 per lane.
#include "b_layout.h"
#include "common.h"

namespace dmm {

// fp32 -> OCP E4M3 code, round to nearest even, saturating at +-448; NaN
// maps to 0x7F.  Bit arithmetic: below 2^-6 the grid is uniform (2^-9), so
// rint(|v| * 512) is the code; above it, rounding the fp32 significand to 3
// fraction bits (adding 0x7FFFF plus the kept LSB at bit 20) carries into the
// exponent exactly like the format does.
__device__ __forceinline__ uint32_t e4m3_code(float v) {
    const uint32_t u = __builtin_bit_cast(uint32_t, v);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t au = u & 0x7FFFFFFFu;
    if (au > 0x7F800000u) return 0x7Fu;                       // NaN
    if (au >= 0x43E00000u) return sign | 0x7Eu;               // |v| >= 448 (incl. inf)
    if (au < 0x3C800000u) {                                   // |v| < 2^-6
        const float a = __builtin_bit_cast(float, au);
        return sign | (uint32_t)__builtin_rintf(a * 512.0f); // exact scaling, RNE
    }
    const uint32_t r = au + 0x7FFFFu + ((au >> 20) & 1u);
    const uint32_t e = (r >> 23) - 127u + 7u;                 // 1 .. 15
    return sign | (e << 3) | ((r >> 20) & 7u);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

__device__ __forceinline__ float group_max(float v, int width) {
    for (int o = width / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

__device__ __forceinline__ float amax_to_scale(float amax) { return amax == 0.0f ? 1.0f : amax / 448.0f; }

__device__ __forceinline__ uint32_t pack4(v4f v, float s) {
    return e4m3_code(v[0] / s) | (e4m3_code(v[1] / s) << 8) | (e4m3_code(v[2] / s) << 16) | (e4m3_code(v[3] / s) << 24);
}

// The hardware conversion v_cvt_pk_fp8_f32 (OCP E4M3, round to nearest even)
// returns e4m3_code's byte for every fp32 input of magnitude below 464 (the
// two were compared over all 2^32 bit patterns on gfx950); at 464 and above,
// for infinities and for NaN they differ, so those inputs never reach it.
__device__ __forceinline__ uint32_t cvt4(float a, float b, float c, float d) {
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// Quantisation by a scale s: the code of each value v is e4m3_code of the
// quotient v / s rounded to fp32.  A correctly rounded fp32 division costs
// about ten instructions per value; instead y = v * r, with r = 1 / s
// rounded once, is within 3 fp32 ulps of the rounded quotient (two
// roundings of relative size at most 2^-24 in y, one more in the quotient).
// Two values that close round to the same E4M3 code unless an E4M3 rounding
// midpoint lies between them, and a midpoint has its fp32 fraction bits 19..0
// equal to 0x80000 wherever |y| >= 2^-6 (three fraction bits survive), so y
// is encoded directly when it is zero, or when 2^-6 <= |y| < 464 and those
// bits are more than 5 ulps from 0x80000.  Every other value -- tiny, near a
// midpoint, non-finite, or under a scale whose reciprocal is not normal (r
// is NaN then, and so is y) -- takes the division.
struct DivQuant {
    float s, r;
    __device__ __forceinline__ explicit DivQuant(float scale)
        : s(scale), r(scale >= 0x1p-126f && scale <= 0x1p126f ? 1.0f / scale : __builtin_nanf("")) {}
    // 1 if y may be encoded directly (bitwise operators throughout: one
    // flag per lane, no branch per value)
    __device__ __forceinline__ static uint32_t direct(float y) {
        const uint32_t au = __builtin_bit_cast(uint32_t, y) & 0x7FFFFFFFu;
        const uint32_t in_range = au - 0x3C800000u < 0x43E80000u - 0x3C800000u;  // 2^-6 <= |y| < 464
        const uint32_t far_mid = (au & 0xFFFFFu) - 0x7FFFBu > 10u;                // > 5 ulps from a midpoint
        return (uint32_t)(au == 0) | (in_range & far_mid);
    }
    __device__ __forceinline__ uint32_t pack(v4f v) const {
        const float y0 = v[0] * r, y1 = v[1] * r, y2 = v[2] * r, y3 = v[3] * r;
        uint32_t w = cvt4(y0, y1, y2, y3);
        if (!(direct(y0) & direct(y1) & direct(y2) & direct(y3))) w = pack4(v, s);
        return w;
    }
};

// ------------------------------------------------------------- per token
// One, two or four waves per row (launch_rows below); cols % 16 == 0.
// Four consecutive values of a row as fp32: fp32 rows load 16 bytes, bf16
// rows 8 bytes, widened exactly (a bf16 value is the high half of an fp32).
__device__ __forceinline__ v4f load4(const float* xr, int c) { return ((const v4f*)xr)[c]; }
__device__ __forceinline__ v4f load4(const uint16_t* xr, int c) {
    typedef uint32_t v2u __attribute__((ext_vector_type(2)));
    const v2u w = ((const v2u*)xr)[c];
    return (v4f){__builtin_bit_cast(float, w[0] << 16), __builtin_bit_cast(float, w[0] & 0xFFFF0000u),
                 __builtin_bit_cast(float, w[1] << 16), __builtin_bit_cast(float, w[1] & 0xFFFF0000u)};
}

// One wave per row: rows of up to 256 NC columns stay in registers (NC
// 16-byte chunks per lane), so each value is read from HBM once and every
// load of the row is in flight before the first wait.
template <typename In, int NC>
__global__ void __launch_bounds__(256) quantize_rows_reg_kernel(const In* __restrict__ x, uint8_t* __restrict__ q,
                                                                float* __restrict__ scale, int rows, int cols) {
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= rows) return;
    const In* xr = x + (size_t)row * cols;
    uint32_t* qr = (uint32_t*)(q + (size_t)row * cols);
    const int n4 = cols / 4;
    v4f v[NC];
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < NC; ++j) {
        const int c = lane + 64 * j;
        v[j] = c < n4 ? load4(xr, c) : (v4f){0.f, 0.f, 0.f, 0.f};
        amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[j][0]), fabsf(v[j][1])), fmaxf(fabsf(v[j][2]), fabsf(v[j][3]))));
    }
    const float s = amax_to_scale(wave_max(amax));
    const DivQuant dq(s);
#pragma unroll
    for (int j = 0; j < NC; ++j) {
        const int c = lane + 64 * j;
        if (c < n4) qr[c] = dq.pack(v[j]);
    }
    if (lane == 0) scale[row] = s;
}

// Rows of 513 .. 7168 columns: W (2 or 4) waves per row, wave h holding
// the 64-chunk slices h, h + W, h + 2W, ... of it (NC chunks per lane), their
// maxima combined through LDS; 1/W of the registers of one wave per row, so
// W times the rows in flight.
template <typename In, int NC, int W>
__global__ void __launch_bounds__(256) quantize_rows_split_kernel(const In* __restrict__ x, uint8_t* __restrict__ q,
                                                                  float* __restrict__ scale, int rows, int cols) {
    static_assert(W == 2 || W == 4, "two or four waves per row");
    __shared__ float red[4];
    const int w = threadIdx.x >> 6, h = w % W, first = w - h;
    const int row = blockIdx.x * (4 / W) + w / W;
    const int lane = threadIdx.x & 63;
    const bool live = row < rows;  // the W waves of a row agree; every wave reaches the barrier
    const In* xr = x + (size_t)(live ? row : 0) * cols;
    uint32_t* qr = (uint32_t*)(q + (size_t)(live ? row : 0) * cols);
    const int n4 = cols / 4;
    v4f v[NC];
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < NC; ++j) {
        const int c = lane + 64 * (W * j + h);
        v[j] = live && c < n4 ? load4(xr, c) : (v4f){0.f, 0.f, 0.f, 0.f};
        amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[j][0]), fabsf(v[j][1])), fmaxf(fabsf(v[j][2]), fabsf(v[j][3]))));
    }
    amax = wave_max(amax);
    if (lane == 0) red[w] = amax;
    __syncthreads();
    float m = red[first];
#pragma unroll
    for (int o = 1; o < W; ++o) m = fmaxf(m, red[first + o]);
    const float s = amax_to_scale(m);
    if (!live) return;
    const DivQuant dq(s);
#pragma unroll
    for (int j = 0; j < NC; ++j) {
        const int c = lane + 64 * (W * j + h);
        if (c < n4) qr[c] = dq.pack(v[j]);
    }
    if (lane == 0 && h == 0) scale[row] = s;
}

// Rows beyond 7168 columns: one wave per row in two passes, the second
// re-reading the row (from L2) to quantise it.
template <typename In>
__global__ void __launch_bounds__(256) quantize_rows_kernel(const In* __restrict__ x, uint8_t* __restrict__ q,
                                                            float* __restrict__ scale, int rows, int cols) {
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= rows) return;
    const In* xr = x + (size_t)row * cols;
    uint32_t* qr = (uint32_t*)(q + (size_t)row * cols);
    const int n4 = cols / 4;
    float amax = 0.0f;
    for (int c = lane; c < n4; c += 64) {
        const v4f v = load4(xr, c);
        amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))));
    }
    const float s = amax_to_scale(wave_max(amax));
    const DivQuant dq(s);
    for (int c = lane; c < n4; c += 64) qr[c] = dq.pack(load4(xr, c));
    if (lane == 0) scale[row] = s;
}

// ------------------------------------------------------- blockscale A
// One wave per row; each pass covers 256 columns, lanes 0-31 one 128-wide
// block and lanes 32-63 the next.  k % 128 == 0.
__global__ void __launch_bounds__(256) quantize_blockscale_a_kernel(const float* __restrict__ x, uint8_t* __restrict__ q,
                                                                    float* __restrict__ scale, int m, int k) {
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= m) return;
    const v4f* xr = (const v4f*)(x + (size_t)row * k);
    uint32_t* qr = (uint32_t*)(q + (size_t)row * k);
    const int n4 = k / 4;
    for (int base = 0; base < n4; base += 64) {
        const int c = base + lane;
        const bool valid = c < n4;  // false only for lanes 32-63 of a last half pass
        v4f v = valid ? xr[c] : (v4f){0.f, 0.f, 0.f, 0.f};
        // the maximum starts from 0 like the row and block maxima: fmax
        // ignores NaN, so a group of NaN has maximum 0 (scale 1 / exponent 0)
        float a = fmaxf(fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))), 0.0f);
        const float s = amax_to_scale(group_max(a, 32));
        if (valid) {
            qr[c] = DivQuant(s).pack(v);
            if ((lane & 31) == 0) scale[(size_t)(c / 32) * m + row] = s;
        }
    }
}

// ------------------------------------------------------- blockscale B
// One workgroup of sixteen waves per 128 x 128 block (rows past n are
// skipped).  The block stays in registers, four rows of 16 bytes per
// thread: it is read from HBM once, with all of a thread's loads in flight
// before the first wait.  Many small threads keep the time from a block's
// last load to its stores short (measured against four and eight waves per
// block: sixteen is 7-31 % faster than four on every shape tried).
__global__ void __launch_bounds__(1024) quantize_blockscale_b_kernel(const float* __restrict__ x, uint8_t* __restrict__ q,
                                                                     float* __restrict__ scale, int n, int k) {
    __shared__ float red[16];
    const int kb = blockIdx.x, nb = blockIdx.y, kblocks = k / 128;
    const int t = threadIdx.x;
    const int col4 = t & 31;  // float4 column within the block
    const int r0 = t >> 5;    // 32 row lanes: thread rows r0, r0 + 32, r0 + 64, r0 + 96
    const int rows = min(128, n - nb * 128);
    v4f v[4];
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = r0 + 32 * j;
        v[j] = r < rows ? *(const v4f*)(x + (size_t)(nb * 128 + r) * k + kb * 128 + col4 * 4)
                        : (v4f){0.f, 0.f, 0.f, 0.f};
        amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[j][0]), fabsf(v[j][1])), fmaxf(fabsf(v[j][2]), fabsf(v[j][3]))));
    }
    amax = wave_max(amax);
    if ((t & 63) == 0) red[t >> 6] = amax;
    __syncthreads();
    float m = red[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) m = fmaxf(m, red[i]);
    const float s = amax_to_scale(m);
    const DivQuant dq(s);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = r0 + 32 * j;
        if (r < rows) *(uint32_t*)(q + (size_t)(nb * 128 + r) * k + kb * 128 + col4 * 4) = dq.pack(v[j]);
    }
    if (t == 0) scale[(size_t)nb * kblocks + kb] = s;
}

// ------------------------------------------------------------- mxfp8
// Exponent e = ceil(log2(amax / 448)) read off the fp32 bits of r = amax/448:
// a power of two keeps its exponent, anything else rounds up by one.
__device__ __forceinline__ int mx_exp(float amax) {
    if (amax == 0.0f) return 0;
    float r = amax / 448.0f;
    int bias = 0;
    uint32_t u = __builtin_bit_cast(uint32_t, r);
    if ((u >> 23) == 0) {  // subnormal: scale up exactly by 2^24 first
        r = r * 16777216.0f;
        u = __builtin_bit_cast(uint32_t, r);
        bias = 24;
    }
    int e = (int)(u >> 23) - 127 - bias + ((u & 0x7FFFFFu) ? 1 : 0);
    return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// One wave per row; each pass covers 256 columns = 8 groups of 32 (8 lanes
// per group).  k % 128 == 0 so a pass is never split inside a group.
__global__ void __launch_bounds__(256) quantize_mxfp8_kernel(const float* __restrict__ x, uint8_t* __restrict__ q,
                                                             uint8_t* __restrict__ scale, int rows, int k) {
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= rows) return;
    const v4f* xr = (const v4f*)(x + (size_t)row * k);
    uint32_t* qr = (uint32_t*)(q + (size_t)row * k);
    const int n4 = k / 4;
    for (int base = 0; base < n4; base += 64) {
        const int c = base + lane;
        const bool valid = c < n4;
        v4f v = valid ? xr[c] : (v4f){0.f, 0.f, 0.f, 0.f};
        // the maximum starts from 0 like the row and block maxima: fmax
        // ignores NaN, so a group of NaN has maximum 0 (scale 1 / exponent 0)
        float a = fmaxf(fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))), 0.0f);
        const int e = mx_exp(group_max(a, 8));
        if (valid) {
            // scaling by 2^-e is exact (or one rounding into the subnormals)
            // and leaves |q| <= 448 for finite v; NaN and infinities (the bit
            // test below is false for both) take the bit-arithmetic encoder
            const float q0 = __builtin_ldexpf(v[0], -e), q1 = __builtin_ldexpf(v[1], -e);
            const float q2 = __builtin_ldexpf(v[2], -e), q3 = __builtin_ldexpf(v[3], -e);
            auto small = [](float f) { return (__builtin_bit_cast(uint32_t, f) & 0x7FFFFFFFu) < 0x43E80000u; };
            qr[c] = small(q0) && small(q1) && small(q2) && small(q3)
                        ? cvt4(q0, q1, q2, q3)
                        : e4m3_code(q0) | (e4m3_code(q1) << 8) | (e4m3_code(q2) << 16) | (e4m3_code(q3) << 24);
            if ((lane & 7) == 0) scale[(size_t)(c / 8) * rows + row] = (uint8_t)(e + 127);
        }
    }
}

// ----------------------------------------------------------- preshuffle
// Output chunk (block j of 16 fragment rows, K tile kt) = 2 KiB at
// (j * KI + kt) * 2048.  Byte 16 l + t of half h (t < 16) holds
// B[src(j, l % 16)][128 kt + 64 h + 16 (l / 16) + t]: exactly the 32 bytes
// matrix-core lane l consumes for a 16 x 128 fp8 operand, so each half is
// one coalesced 1 KiB load.  Fragment row r of block j is B row
// src(j, r) = 64 G + bl::frag_col(j % 4, r, p) of its group G = j / 4 of p
// blocks (b_layout.h): the order in which the GEMM's lanes hold contiguous
// output columns.
__global__ void __launch_bounds__(256) preshuffle_b_kernel(const uint8_t* __restrict__ b, uint8_t* __restrict__ out,
                                                           int n, int k) {
    const size_t t = (size_t)blockIdx.x * 256 + threadIdx.x;  // one 16-byte piece per thread
    const int KI = k / 128;
    const size_t total = (size_t)n * k / 16;
    if (t >= total) return;
    const int l = (int)(t & 63);
    const int h = (int)((t >> 6) & 1);
    const size_t chunk = t >> 7;
    const int kt = (int)(chunk % KI);
    const int j = (int)(chunk / KI);
    const int G = j >> 2;
    const int row = 64 * G + bl::frag_col(j & 3, l & 15, bl::group_blocks(G, n / 16));
    const size_t src = (size_t)row * k + 128 * kt + 64 * h + 16 * (l >> 4);
    *(v4i*)(out + t * 16) = *(const v4i*)(b + src);
}

// -------------------------------------------------------------- launch
// Per-token quantisation, rows held in registers up to 7168 columns: one
// wave per row up to 512 columns, two up to 2048 (4 chunks per lane each)
// and up to 4096 (8 each), four up to 7168 (7 each); the two-pass kernel
// beyond.  (Two waves per row against one, same-box A/B: 32768 x 1792
// 44.2 -> 43.2 us, 65536 x 1024 59.2 -> 56.5 us, but 16384 x 512 9.7 ->
// 11.6 us.)
template <typename In>
static hipError_t launch_rows(const In* x, uint8_t* q, float* s, int rows, int cols, hipStream_t st) {
    const dim3 g4((rows + 3) / 4), g2((rows + 1) / 2), g1(rows), b(256);
    const int chunks = (cols / 4 + 63) / 64;  // 64-lane slices of 16-byte chunks in a row
    if (chunks <= 2) hipLaunchKernelGGL((quantize_rows_reg_kernel<In, 2>), g4, b, 0, st, x, q, s, rows, cols);
    else if (chunks <= 8) hipLaunchKernelGGL((quantize_rows_split_kernel<In, 4, 2>), g2, b, 0, st, x, q, s, rows, cols);
    else if (chunks <= 16) hipLaunchKernelGGL((quantize_rows_split_kernel<In, 8, 2>), g2, b, 0, st, x, q, s, rows, cols);
    else if (chunks <= 28) hipLaunchKernelGGL((quantize_rows_split_kernel<In, 7, 4>), g1, b, 0, st, x, q, s, rows, cols);
    else hipLaunchKernelGGL(quantize_rows_kernel<In>, g4, b, 0, st, x, q, s, rows, cols);
    return hipGetLastError();
}

hipError_t launch_quantize_rows(const float* x, uint8_t* q, float* s, int rows, int cols, hipStream_t st) {
    return launch_rows<float>(x, q, s, rows, cols, st);
}

hipError_t launch_quantize_rows_bf16(const uint16_t* x, uint8_t* q, float* s, int rows, int cols, hipStream_t st) {
    return launch_rows<uint16_t>(x, q, s, rows, cols, st);
}

hipError_t launch_quantize_blockscale_a(const float* x, uint8_t* q, float* s, int m, int k, hipStream_t st) {
    hipLaunchKernelGGL(quantize_blockscale_a_kernel, dim3((m + 3) / 4), dim3(256), 0, st, x, q, s, m, k);
    return hipGetLastError();
}

hipError_t launch_quantize_blockscale_b(const float* x, uint8_t* q, float* s, int n, int k, hipStream_t st) {
    hipLaunchKernelGGL(quantize_blockscale_b_kernel, dim3(k / 128, (n + 127) / 128), dim3(1024), 0, st, x, q, s, n, k);
    return hipGetLastError();
}

hipError_t launch_quantize_mxfp8(const float* x, uint8_t* q, uint8_t* s, int rows, int k, hipStream_t st) {
    hipLaunchKernelGGL(quantize_mxfp8_kernel, dim3((rows + 3) / 4), dim3(256), 0, st, x, q, s, rows, k);
    return hipGetLastError();
}

hipError_t launch_preshuffle_b(const uint8_t* b, uint8_t* out, int n, int k, hipStream_t st) {
    const size_t pieces = (size_t)n * k / 16;
    hipLaunchKernelGGL(preshuffle_b_kernel, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0, st, b, out, n, k);
    return hipGetLastError();
}

}  // namespace dmm
