/*
 * oracle.c -- TEST INFRASTRUCTURE ONLY.  A plain, slow, obviously correct CPU
 * statement of what the fp8 a8w8 GEMM computes.  Only tests/, the smoke check
 * and the benchmark's CPU-baseline leg may load this library; the product
 * path never does, and this file shares no code, header, table or constant
 * with the HIP library.
 *
 * What the GEMM computes (the reference the pages check their kernels
 * against):
 *   - mori PR 785 ("fix(gemm-ar): drain the peeled tail's producers instead
 *     of tightening the loop"), section Test: the output is compared with a
 *     bf16-rounded fp32 reference built from the quantised operands.
 *   - aiter PR 6539 ("[FlyDSL] Fix cross-wave LDS race on the last K tile in
 *     8-wave GEMM and gather_kv_b_proj"), Test Plan and review thread: an fp32
 *     reference (run_torch / ref_gemm) over the quantised operands xq, wq and
 *     their scales, cast to bf16.
 *   - mori PR 809 ("mori.ops.ag_gemm"), section Using it: the per-token
 *     quantiser and the ptpc operands a_fp8, a_scale, b_fp8, b_scale; section
 *     Not done yet: blockscale and mxfp8 keep their A scale K-block major.
 *
 * Definition implemented here, for every mode:
 *   a'(m,k) = fl32(dec_e4m3(qa[m,k]) * sa(m,k))
 *   b'(n,k) = fl32(dec_e4m3(qb[n,k]) * sb(n,k))
 *   acc     = 0; for k ascending: acc = fl32(acc + fl32(a'(m,k) * b'(n,k)))
 *   C[m,n]  = bf16_rne(acc)
 * with sa / sb chosen by the scaling mode (ptpc, 1x128 / 128x128 blockscale,
 * e8m0 per 32 K).  This file must be compiled without FMA contraction
 * (-ffp-contract=off) and without fast-math so that every product and every
 * sum is a separately rounded fp32 operation.
 *
 * Readings of points the pages leave open (each is listed with its reason in
 * the design notes):
 *   - e4m3 is the OCP FP8 E4M3 ("fn") format: bias 7, max 448, no infinity,
 *     NaN = S.1111.111.  The workloads quantise with scale = amax / 448.
 *   - Quantisation rounds to nearest even and saturates to +-448.
 *   - A zero row (amax == 0) gets scale 1.0 and all-zero codes.
 *   - mxfp8 exponent: e = ceil(log2(amax / 448)), clamped to [-127, 127],
 *     stored as e + 127 (E8M0); a zero group stores 127.
 *   - Scale layouts: blockscale A [K/128][M], B [ceil(N/128)][K/128];
 *     mxfp8 A [K/32][M], B [K/32][N].
 *
 * Parity of every function here is pinned by tests/test_oracle_pins.py
 * against library routines, closed forms, exact-arithmetic cases and a
 * float64 brute force; no function is left "parity unpinned".
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define ORC_MODE_PTPC 0
#define ORC_MODE_BLOCKSCALE 1
#define ORC_MODE_MXFP8 2

/* ---------------------------------------------------------------- codecs */

/* OCP FP8 E4M3: sign s, exponent e (4 bits, bias 7), fraction f (3 bits).
 * e == 0 is subnormal: f * 2^-9.  S.1111.111 is NaN; there is no infinity. */
float orc_dec_e4m3(uint8_t q) {
    int s = q >> 7, e = (q >> 3) & 15, f = q & 7;
    float mag;
    if (e == 15 && f == 7) return NAN;
    if (e == 0)
        mag = ldexpf((float)f, -9);
    else
        mag = ldexpf(1.0f + (float)f / 8.0f, e - 7);
    return s ? -mag : mag;
}

/* Round-to-nearest-even onto the E4M3 grid, saturating to +-448. */
uint8_t orc_enc_e4m3(float v) {
    uint8_t sign;
    float a;
    if (isnan(v)) return 0x7F;
    sign = signbit(v) ? 0x80 : 0x00;
    a = fabsf(v);
    if (a >= 448.0f) return sign | 0x7E;
    if (a < ldexpf(1.0f, -6)) {
        /* subnormal range: multiples of 2^-9; 8 * 2^-9 is the smallest normal,
         * whose code (exponent 1, fraction 0) is 8 as well */
        float t = nearbyintf(ldexpf(a, 9)); /* exact scaling, RNE */
        return sign | (uint8_t)t;
    } else {
        int ex;
        float fr = frexpf(a, &ex); /* a = fr * 2^ex, fr in [0.5, 1) */
        int e = ex - 1;            /* a = (2 fr) * 2^e, 2 fr in [1, 2) */
        float frac8 = nearbyintf((2.0f * fr - 1.0f) * 8.0f); /* exact, RNE */
        int f = (int)frac8;
        if (f == 8) { f = 0; e += 1; }
        if (e + 7 > 15 || (e + 7 == 15 && f == 7)) return sign | 0x7E;
        return sign | (uint8_t)(((e + 7) << 3) | f);
    }
}

/* OCP MX E8M0 scale: 2^(b - 127); 255 is NaN. */
float orc_dec_e8m0(uint8_t b) {
    if (b == 255) return NAN;
    return ldexpf(1.0f, (int)b - 127);
}

/* fp32 -> bf16 with round-to-nearest-even; any NaN becomes the quiet NaN 0x7FC0. */
uint16_t orc_bf16_rne(float x) {
    uint32_t u;
    memcpy(&u, &x, 4);
    if (isnan(x)) return 0x7FC0;
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

float orc_bf16_to_f32(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float x;
    memcpy(&x, &u, 4);
    return x;
}

/* ----------------------------------------------------------- quantisers */

/* One group of values sharing an fp32 scale amax / 448 (IEEE division). */
static float amax_scale(float amax) { return amax == 0.0f ? 1.0f : amax / 448.0f; }

/* Per-row quantisation: per token for A, per output channel for B[N,K]
 * (mori PR 809, Using it: quantize_per_token). */
void orc_quantize_rows(const float* x, int64_t rows, int64_t cols, uint8_t* q, float* scale) {
    for (int64_t r = 0; r < rows; ++r) {
        const float* xr = x + r * cols;
        float amax = 0.0f, s;
        for (int64_t c = 0; c < cols; ++c) amax = fmaxf(amax, fabsf(xr[c]));
        s = amax_scale(amax);
        scale[r] = s;
        for (int64_t c = 0; c < cols; ++c) q[r * cols + c] = orc_enc_e4m3(xr[c] / s);
    }
}

/* Blockscale A: one fp32 scale per row per 128-wide K block, stored K-block
 * major as scale[kb * M + m]. */
void orc_quantize_blockscale_a(const float* x, int64_t m, int64_t k, uint8_t* q, float* scale) {
    int64_t kblocks = k / 128;
    for (int64_t r = 0; r < m; ++r)
        for (int64_t kb = 0; kb < kblocks; ++kb) {
            const float* xb = x + r * k + kb * 128;
            float amax = 0.0f, s;
            for (int c = 0; c < 128; ++c) amax = fmaxf(amax, fabsf(xb[c]));
            s = amax_scale(amax);
            scale[kb * m + r] = s;
            for (int c = 0; c < 128; ++c) q[r * k + kb * 128 + c] = orc_enc_e4m3(xb[c] / s);
        }
}

/* Blockscale B[N,K]: one fp32 scale per 128 x 128 block, scale[nb * (K/128) + kb];
 * a partial last N block uses only the rows it has. */
void orc_quantize_blockscale_b(const float* x, int64_t n, int64_t k, uint8_t* q, float* scale) {
    int64_t kblocks = k / 128, nblocks = (n + 127) / 128;
    for (int64_t nb = 0; nb < nblocks; ++nb)
        for (int64_t kb = 0; kb < kblocks; ++kb) {
            int64_t r0 = nb * 128, r1 = r0 + 128 < n ? r0 + 128 : n;
            float amax = 0.0f, s;
            for (int64_t r = r0; r < r1; ++r)
                for (int c = 0; c < 128; ++c) amax = fmaxf(amax, fabsf(x[r * k + kb * 128 + c]));
            s = amax_scale(amax);
            scale[nb * kblocks + kb] = s;
            for (int64_t r = r0; r < r1; ++r)
                for (int c = 0; c < 128; ++c)
                    q[r * k + kb * 128 + c] = orc_enc_e4m3(x[r * k + kb * 128 + c] / s);
        }
}

/* Smallest power-of-two exponent e with amax / 2^e <= 448, i.e.
 * e = ceil(log2(amax / 448)), taken exactly from frexpf.  An infinite
 * maximum has no such e: ceil(log2(inf)) is +inf, clamped like every other
 * exponent to the format's largest, 127 (frexpf's exponent is unspecified
 * for an infinite argument, so it is not consulted). */
static int mx_exponent(float amax) {
    int ex, e;
    float r, fr;
    if (amax == 0.0f) return 0;
    if (isinf(amax)) return 127;
    r = amax / 448.0f;
    fr = frexpf(r, &ex); /* r = fr * 2^ex, fr in [0.5, 1) */
    e = (fr == 0.5f) ? ex - 1 : ex;
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return e;
}

/* mxfp8: one E8M0 scale per 32 consecutive K values of a row, stored
 * e[(k / 32) * rows + r]; codes q = enc_e4m3(x * 2^-e). */
void orc_quantize_mxfp8(const float* x, int64_t rows, int64_t k, uint8_t* q, uint8_t* e8) {
    int64_t groups = k / 32;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t g = 0; g < groups; ++g) {
            const float* xg = x + r * k + g * 32;
            float amax = 0.0f;
            int e;
            for (int c = 0; c < 32; ++c) amax = fmaxf(amax, fabsf(xg[c]));
            e = mx_exponent(amax);
            e8[g * rows + r] = (uint8_t)(e + 127);
            for (int c = 0; c < 32; ++c) q[r * k + g * 32 + c] = orc_enc_e4m3(ldexpf(xg[c], -e));
        }
}

/* ------------------------------------------------------------------ GEMM */

/* Scale that multiplies A element (m, k) in each mode. */
static float scale_a(int mode, const void* sa, int64_t M, int64_t m, int64_t k) {
    if (mode == ORC_MODE_PTPC) return ((const float*)sa)[m];
    if (mode == ORC_MODE_BLOCKSCALE) return ((const float*)sa)[(k / 128) * M + m];
    return orc_dec_e8m0(((const uint8_t*)sa)[(k / 32) * M + m]);
}

/* Scale that multiplies B element (n, k) in each mode. */
static float scale_b(int mode, const void* sb, int64_t N, int64_t K, int64_t n, int64_t k) {
    if (mode == ORC_MODE_PTPC) return ((const float*)sb)[n];
    if (mode == ORC_MODE_BLOCKSCALE) return ((const float*)sb)[(n / 128) * (K / 128) + k / 128];
    return orc_dec_e8m0(((const uint8_t*)sb)[(k / 32) * N + n]);
}

typedef struct {
    int mode; /* -1: bf16 operands */
    const uint8_t* qa;
    const void* sa;
    const uint16_t* abf;
    const float* bt; /* b'(n,k) stored at bt[k * N + n] */
    int64_t M, N, K;
    const int64_t* rows;
    int64_t nrows;
    uint16_t* c;    /* [nrows][N] bf16, may be NULL */
    float* c32;     /* [nrows][N] unrounded fp32, may be NULL */
    int64_t i0, i1; /* this worker's slice of rows[] */
} job_t;

static void* gemm_rows(void* p) {
    job_t* j = (job_t*)p;
    float* arow = (float*)malloc(sizeof(float) * (size_t)j->K);
    float* acc = (float*)malloc(sizeof(float) * (size_t)j->N);
    for (int64_t i = j->i0; i < j->i1; ++i) {
        int64_t m = j->rows ? j->rows[i] : i;
        for (int64_t k = 0; k < j->K; ++k)
            arow[k] = j->mode < 0 ? orc_bf16_to_f32(j->abf[m * j->K + k])
                                  : orc_dec_e4m3(j->qa[m * j->K + k]) * scale_a(j->mode, j->sa, j->M, m, k);
        for (int64_t n = 0; n < j->N; ++n) acc[n] = 0.0f;
        /* every acc[n] is its own fp32 dot product, summed in ascending k */
        for (int64_t k = 0; k < j->K; ++k) {
            const float a = arow[k];
            const float* b = j->bt + k * j->N;
            for (int64_t n = 0; n < j->N; ++n) acc[n] = acc[n] + a * b[n];
        }
        for (int64_t n = 0; n < j->N; ++n) {
            if (j->c) j->c[i * j->N + n] = orc_bf16_rne(acc[n]);
            if (j->c32) j->c32[i * j->N + n] = acc[n];
        }
    }
    free(arow);
    free(acc);
    return NULL;
}

static int run_rows(job_t* base, int threads) {
    pthread_t tid[512];
    job_t jobs[512];
    int64_t per;
    if (threads <= 0) threads = (int)sysconf(_SC_NPROCESSORS_ONLN);
    if (threads < 1) threads = 1;
    if (threads > 512) threads = 512;
    if (threads > base->nrows) threads = (int)(base->nrows > 0 ? base->nrows : 1);
    per = (base->nrows + threads - 1) / threads;
    for (int t = 0; t < threads; ++t) {
        jobs[t] = *base;
        jobs[t].i0 = t * per < base->nrows ? t * per : base->nrows;
        jobs[t].i1 = (t + 1) * per < base->nrows ? (t + 1) * per : base->nrows;
        if (pthread_create(&tid[t], NULL, gemm_rows, &jobs[t]) != 0) return -1;
    }
    for (int t = 0; t < threads; ++t) pthread_join(tid[t], NULL);
    return threads;
}

/* C rows listed in rows[0..nrows) (all M rows in order when rows == NULL):
 * c[i][n] = bf16(sum_k a'(rows[i],k) b'(n,k)).  c32, when non-NULL, receives
 * the unrounded fp32 sums.  Returns the number of threads used, or -1. */
int orc_gemm_a8w8(int mode, const uint8_t* qa, const uint8_t* qb, const void* sa, const void* sb,
                  int64_t M, int64_t N, int64_t K, const int64_t* rows, int64_t nrows, uint16_t* c,
                  float* c32, int threads) {
    job_t job;
    int used;
    float* bt = (float*)malloc(sizeof(float) * (size_t)N * (size_t)K);
    if (!bt) return -1;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            bt[k * N + n] = orc_dec_e4m3(qb[n * K + k]) * scale_b(mode, sb, N, K, n, k);
    memset(&job, 0, sizeof job);
    job.mode = mode;
    job.qa = qa;
    job.sa = sa;
    job.bt = bt;
    job.M = M;
    job.N = N;
    job.K = K;
    job.rows = rows;
    job.nrows = rows ? nrows : M;
    job.c = c;
    job.c32 = c32;
    used = run_rows(&job, threads);
    free(bt);
    return used;
}

/* bf16 GEMM: a [M,K] and b [N,K] bf16, fp32 accumulation in ascending k,
 * bf16 result (DeepGEMM PR 453, "Fix SM120 BF16 GEMM shared-memory reuse
 * ordering", Reproduction and validation: the [4096,1024] x [1024,896] shape). */
int orc_gemm_bf16(const uint16_t* a, const uint16_t* b, int64_t M, int64_t N, int64_t K,
                  const int64_t* rows, int64_t nrows, uint16_t* c, float* c32, int threads) {
    job_t job;
    int used;
    float* bt = (float*)malloc(sizeof(float) * (size_t)N * (size_t)K);
    if (!bt) return -1;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) bt[k * N + n] = orc_bf16_to_f32(b[n * K + k]);
    memset(&job, 0, sizeof job);
    job.mode = -1;
    job.abf = a;
    job.bt = bt;
    job.M = M;
    job.N = N;
    job.K = K;
    job.rows = rows;
    job.nrows = rows ? nrows : M;
    job.c = c;
    job.c32 = c32;
    used = run_rows(&job, threads);
    free(bt);
    return used;
}

/* ------------------------------------------------ array forms for ctypes */

void orc_dec_e4m3_n(const uint8_t* q, float* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_dec_e4m3(q[i]);
}
void orc_enc_e4m3_n(const float* x, uint8_t* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_enc_e4m3(x[i]);
}
void orc_dec_e8m0_n(const uint8_t* b, float* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_dec_e8m0(b[i]);
}
void orc_bf16_rne_n(const float* x, uint16_t* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_rne(x[i]);
}
void orc_bf16_to_f32_n(const uint16_t* h, float* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_to_f32(h[i]);
}
