/*
 * dmm.h -- C ABI of libdmm, an fp8 a8w8 GEMM library for AMD Instinct MI355X
 * (gfx950).
 *
 * The user sequence follows mori PR 809 ("mori.ops.ag_gemm"), section Using
 * it: quantise the activations per token, preshuffle the fp8 weight once,
 * then call the GEMM with both operands and their scales; the result is a
 * contiguous bf16 [M, N] tensor.  The GEMM computes
 *
 *     C[m, n] = bf16( sum_k (A[m, k] * sa(m, k)) * (B[n, k] * sb(n, k)) )
 *
 * with fp32 accumulation, where A [M, K] and B [N, K] hold OCP FP8 E4M3 codes
 * and sa / sb depend on the scaling mode (ptpc, blockscale, mxfp8) named in
 * mori PR 785 ("fix(gemm-ar): drain the peeled tail's producers instead of
 * tightening the loop"), section Cost.
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers owned by the caller.  The library
 *     allocates nothing and keeps no state beyond a per-device arch check.
 *   - Every call is asynchronous on `stream` (a hipStream_t passed as void*;
 *     NULL is the default stream).  Nothing synchronises the host.
 *   - Layouts are row-major and contiguous.  e4m3 codes are uint8_t (OCP
 *     FP8 E4M3, max 448, NaN = S.1111.111); bf16 values are uint16_t bit
 *     patterns; E8M0 scales are uint8_t (2^(b-127)).
 *   - Argument errors return DMM_EINVAL before any HIP call is made;
 *     dmm_last_error() then describes the first violated rule.  A device that
 *     is not gfx950 returns DMM_ENODEV.  A failed launch returns DMM_ELAUNCH.
 *   - Every pointer must be 16-byte aligned, and every operand (A, B, C,
 *     scales) must be smaller than 2^31 bytes: the kernels address operands
 *     through 32-bit buffer offsets.
 *   - Calls on one stream are ordered; calls on different streams that write
 *     the same buffer race, as with any kernel.
 */
#ifndef DMM_H
#define DMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DMM_OK = 0,
    DMM_EINVAL = 1,  /* an argument breaks a documented rule */
    DMM_ENODEV = 2,  /* the current device is not gfx950 */
    DMM_ELAUNCH = 3  /* the HIP runtime reported an error */
} dmm_status;

/* Name of a status code ("DMM_OK", ...). */
const char* dmm_status_str(int status);

/* Detail for the last non-OK return on the calling thread ("" if none). */
const char* dmm_last_error(void);

/* ---------------------------------------------------------------- quantise */

/* Per-row E4M3 quantisation (mori PR 809, Using it: quantize_per_token; the
 * workloads use scale = amax / 448).  For each row r of x [rows, cols] fp32:
 *   scale[r] = amax_r / 448 (IEEE fp32 division; 1.0 when the row is zero),
 *   q[r, c]  = E4M3(x[r, c] / scale[r]), round to nearest even, saturating
 *              to +-448.
 * Used per token for A and per output channel for B [N, K].
 * Rules: rows >= 1, cols >= 16, cols % 16 == 0.  q [rows, cols] u8, scale
 * [rows] fp32, both written. */
dmm_status quantize_per_token(const float* x, uint8_t* q, float* scale, int64_t rows, int64_t cols,
                              void* stream);

/* The same for bf16 activations: x [rows, cols] bf16 (uint16_t bit
 * patterns), each value widened exactly to fp32, then the rule above.
 * Same rules and outputs. */
dmm_status quantize_per_token_bf16(const uint16_t* x, uint8_t* q, float* scale, int64_t rows, int64_t cols,
                                   void* stream);

/* Blockscale A: one fp32 scale per row per 128-wide K block (mori PR 785,
 * Cost: blockscale; the A scale is K-block major, mori PR 809, Not done yet).
 *   scale[kb * m + r] = amax(x[r, 128kb .. 128kb+127]) / 448 (1.0 if zero),
 *   q[r, c] = E4M3(x[r, c] / scale[c/128 * m + r]).
 * Rules: m >= 1, k >= 128, k % 128 == 0. */
dmm_status quantize_blockscale_a(const float* x, uint8_t* q, float* scale, int64_t m, int64_t k, void* stream);

/* Blockscale B [n, k]: one fp32 scale per 128 x 128 block, stored
 * scale[nb * (k/128) + kb]; a partial last row block uses only the rows it
 * has.  Rules: n >= 16, n % 16 == 0, k >= 128, k % 128 == 0. */
dmm_status quantize_blockscale_b(const float* x, uint8_t* q, float* scale, int64_t n, int64_t k, void* stream);

/* mxfp8: one E8M0 scale per 32 consecutive K values of a row (mori PR 785,
 * Cost: mxfp8).  e = ceil(log2(amax / 448)) clamped to [-127, 127] (0 for a
 * zero group), stored scale[(c/32) * rows + r] = e + 127;
 * q[r, c] = E4M3(x[r, c] * 2^-e).  Used for both A [M, K] and B [N, K].
 * Rules: rows >= 1, k >= 128, k % 128 == 0. */
dmm_status quantize_mxfp8(const float* x, uint8_t* q, uint8_t* scale, int64_t rows, int64_t k, void* stream);

/* ------------------------------------------------------------- preshuffle */

/* Reorders B [n, k] E4M3 codes (one row per output channel) into the byte
 * order the GEMM's matrix-core operands use (aiter PR 6539 names the kernels
 * "bpreshuffle"; mori PR 809, Using it, calls preshuffle_b once per weight).
 * The layout is library-defined: b_shuf has the same size as b (n * k
 * bytes) and is only meant to be passed to the gemm_a8w8_* calls.  (For
 * reference: 2 KiB chunk (j, kt) at (j * k/128 + kt) * 2048 holds block j of
 * 16 fragment rows for K tile kt; byte 16 l + t of its half h is
 * B[src(j, l % 16)][128 kt + 64 h + 16 (l / 16) + t].  Blocks come in groups
 * of four, 64 output columns; in group G = j / 4 of p blocks, fragment row r
 * of block nb = j % 4 is B row 64 G + 32 (nb / 2) + 8 (r / 4) + 4 (nb % 2) +
 * r % 4, except that the last block of a group with an odd p keeps row
 * order, 64 G + 16 nb + r.)
 * b and b_shuf must not overlap.  Rules: n >= 16, n % 16 == 0, k >= 128,
 * k % 128 == 0. */
dmm_status preshuffle_b(const uint8_t* b, uint8_t* b_shuf, int64_t n, int64_t k, void* stream);

/* --------------------------------------------------------------- the GEMM */

/* Rules shared by the three fp8 GEMMs:
 *   m >= 1; n >= 16 and n % 16 == 0 (the last 256-column tile may be
 *   partial; mori PR 809, Using it); k >= 128 and k % 128 == 0 (k = 256
 *   runs the peeled tail only; mori PR 785, Why the existing A+B-1 did not
 *   fix it).  a [m, k] u8 codes; b_shuf from preshuffle_b; c [m, n] bf16 is
 *   fully overwritten and nothing outside it is written. */

/* ptpc: a_scale [m] fp32 per token, b_scale [n] fp32 per output channel.
 *   C[m, n] = bf16(a_scale[m] * b_scale[n] * sum_k A[m, k] B[n, k]). */
dmm_status gemm_a8w8_ptpc(const uint8_t* a, const uint8_t* b_shuf, const float* a_scale, const float* b_scale,
                          uint16_t* c, int64_t m, int64_t n, int64_t k, void* stream);

/* ptpc with an explicit output-tile shape, the same result as
 * gemm_a8w8_ptpc: tile 1 = 256 x 256 (four waves), 2 = 128 x 256 (eight
 * waves), 3 = 128 x 128 (four waves), 0 = the choice gemm_a8w8_ptpc makes:
 * the tile whose waves over the compute units cost least, a 128 x 256 tile
 * costing 0.625 and a 128 x 128 tile 0.34 of a wide tile's time (so the
 * smaller tiles win only where the wide grid would leave many compute units
 * idle).  The pages size the
 * tile to the problem in the same spirit (mori PR 785, Cost: the table's
 * shapes; aiter PR 6539, Motivation and its review thread: the tuned rows,
 * one kernel configuration per shape).  Other values of tile return
 * DMM_EINVAL. */
dmm_status gemm_a8w8_ptpc_tile(const uint8_t* a, const uint8_t* b_shuf, const float* a_scale,
                               const float* b_scale, uint16_t* c, int64_t m, int64_t n, int64_t k, int tile,
                               void* stream);

/* ptpc over a gathered A: the GEMM half of an all-gather + GEMM (mori PR
 * 809, How it works: the tile order and the wait), on one GPU.  A [m, k] and
 * a_scale [m] are m / src_rows source slabs of src_rows rows; slab `own` is
 * resident when the call starts, and every other slab arrives in nchunks
 * row bands of src_rows / nchunks rows: band s * nchunks + c (rows
 * s * src_rows + c * src_rows / nchunks ...) may be read once
 * flags[s * nchunks + c] has reached epoch, compared wrap-safe as
 * (int32_t)(flags[band] - epoch) >= 0, so a caller advances epoch per call
 * and never resets the flags.  Tiles of the own slab run first, never
 * waiting; then, for each chunk c, the sources own+1, own+2, ... (mod the
 * source count).  A workgroup polls a band's flag with system-scope loads
 * before any load of its rows and fences (acquire) after seeing it; flags
 * may live in device memory or in pinned host memory that a host thread
 * writes.  After spin_limit polls (each about 0.3 us) for one band the wait
 * gives up: *status (device int, zeroed by the caller) becomes the largest
 * 1 + band that timed out and the result is undefined; the kernel still
 * finishes.  The result is otherwise bitwise that of gemm_a8w8_ptpc.
 * Rules beyond gemm_a8w8_ptpc's: src_rows a positive multiple of
 * 256 * nchunks; m a multiple of src_rows; at most 64 bands; 0 <= own <
 * m / src_rows; spin_limit >= 0; flags and status non-null, 4-byte aligned. */
dmm_status gemm_a8w8_ptpc_gathered(const uint8_t* a, const uint8_t* b_shuf, const float* a_scale,
                                   const float* b_scale, uint16_t* c, int64_t m, int64_t n, int64_t k,
                                   const uint32_t* flags, int64_t src_rows, int nchunks, int own, uint32_t epoch,
                                   int64_t spin_limit, int* status, void* stream);

/* blockscale: a_scale [k/128][m] fp32 (1x128 blocks, K-block major),
 * b_scale [ceil(n/128)][k/128] fp32 (128x128 blocks).
 *   C[m, n] = bf16(sum_kb a_scale[kb][m] b_scale[n/128][kb] sum_{k in kb} A B). */
dmm_status gemm_a8w8_blockscale(const uint8_t* a, const uint8_t* b_shuf, const float* a_scale,
                                const float* b_scale, uint16_t* c, int64_t m, int64_t n, int64_t k,
                                void* stream);

/* blockscale with an explicit output-tile shape, the same result as
 * gemm_a8w8_blockscale: tile 1 = 128 x 256 (eight waves, two per SIMD),
 * 2 = 128 x 128 (four waves), 0 = the choice gemm_a8w8_blockscale makes
 * (128 x 128 when its waves over the compute units cost less than the
 * 128 x 256 tile's, by the rule gemm_a8w8_mxfp8_tile describes; the pages
 * tune one configuration per shape: aiter PR 6539, Motivation and the tuned
 * rows of its review thread).  Other values of tile return DMM_EINVAL. */
dmm_status gemm_a8w8_blockscale_tile(const uint8_t* a, const uint8_t* b_shuf, const float* a_scale,
                                     const float* b_scale, uint16_t* c, int64_t m, int64_t n, int64_t k, int tile,
                                     void* stream);

/* mxfp8: a_scale [k/32][m] and b_scale [k/32][n] E8M0 bytes, one per 32
 * consecutive K values.
 *   C[m, n] = bf16(sum_g 2^(a_scale[g][m]-127) 2^(b_scale[g][n]-127) sum_{k in g} A B).
 * Scale byte 255 (NaN) is outside the contract. */
dmm_status gemm_a8w8_mxfp8(const uint8_t* a, const uint8_t* b_shuf, const uint8_t* a_scale,
                           const uint8_t* b_scale, uint16_t* c, int64_t m, int64_t n, int64_t k, void* stream);

/* mxfp8 with an explicit output-tile shape, the same result as
 * gemm_a8w8_mxfp8: tile 1 = 256 x 256, 2 = 256 x 128 (four waves, each
 * owning all 256 rows and 32 columns: the A tile that goes through LDS is
 * twice the B tile -- the narrow mxfp8 shape whose A side outgrows its B
 * side, mori PR 785, review thread), 0 = the choice gemm_a8w8_mxfp8 makes (256 x 128 when its
 * waves over the compute units cost less than the 256 x 256 tile's, e.g.
 * when the wide grid leaves most CUs idle).  The same choice rule picks
 * between gemm_a8w8_ptpc's two tiles.  Other values of tile return
 * DMM_EINVAL. */
dmm_status gemm_a8w8_mxfp8_tile(const uint8_t* a, const uint8_t* b_shuf, const uint8_t* a_scale,
                                const uint8_t* b_scale, uint16_t* c, int64_t m, int64_t n, int64_t k, int tile,
                                void* stream);

/* bf16 GEMM with fp32 accumulation (DeepGEMM PR 453, "Fix SM120 BF16 GEMM
 * shared-memory reuse ordering", Reproduction and validation: [4096, 1024]
 * x [1024, 896]).  a [m, k] bf16, b [n, k] bf16 (the weight given one row
 * per output column), c [m, n] bf16 = bf16(sum_k a[m, k] b[n, k]).
 * Rules: m >= 1; n >= 16, n % 16 == 0; k >= 64, k % 64 == 0. */
dmm_status gemm_bf16(const uint16_t* a, const uint16_t* b, uint16_t* c, int64_t m, int64_t n, int64_t k,
                     void* stream);

/* gemm_bf16 with an explicit output-tile shape, the same result: tile 1 =
 * 128 x 128, 2 = 64 x 64, 0 = gemm_bf16's choice (64 x 64 when the problem
 * has at most one 128 x 128 tile per two compute units).  Other values
 * return DMM_EINVAL. */
dmm_status gemm_bf16_tile(const uint16_t* a, const uint16_t* b, uint16_t* c, int64_t m, int64_t n, int64_t k,
                          int tile, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DMM_H */
