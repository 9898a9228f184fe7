/*
 * Plain CPU oracle for GGML Q4_0 / Q8_0 block quantization and the
 * Q4_0 x f32 and Q8_0 x f32 matrix products.
 *
 * TEST INFRASTRUCTURE. This file is the reference the GPU library is checked
 * against; it is not part of the product. Only the test suite, the smoke check
 * and the CPU-baseline leg of the benchmark may load it. It shares no code,
 * header, table or constant with the GPU library, and it never calls it.
 *
 * Every function is written straight from its definition, in loops, with no
 * blocking, vector intrinsics or reordering. Build with
 *   gcc -O2 -fno-fast-math -ffp-contract=off -fopenmp -shared -fPIC
 * so that every floating-point operation below is one correctly rounded IEEE
 * operation in the precision written (x86-64 SSE evaluates float in float).
 *
 * Sources (all on the docs.rs page "fuel-vulkan-kernels — quantized (GGML)
 * kernel contracts", fuel-dispatch 0.20.71, kernel-contracts/vulkan/quantized.fkc.md):
 *   - Q4_0 block and decode rule: section "dequant_q4_0".
 *   - Q8_0 block and decode rule: section "dequant_q8_0".
 *   - Q8_0 quantize rule: section "quantize_q8_0".
 *   - Q4_0 x f32 product: sections "qmatvec_q4_0" and "matmul_q4_0_tiled".
 *   - Q8_0 x f32 product: the same product over Q8_0 weights; the page's
 *     quantized-matmul binding picks Q4_0 or Q8_0 blocks by quant type
 *     (section "qmatvec_q4_0", as-built note), and a Q8_0 weight is the
 *     value of section "dequant_q8_0".
 *   - Q4_0 quantize rule: not on the pages; it is GGML's reference rule as
 *     stated with the benchmark workloads (d = signed max-abs / -8,
 *     q = min(15, int(x/d + 8.5))). It only generates test weights.
 */
#include <math.h>
#include <omp.h>
#include <stdlib.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#define ORC_Q4_0_BLOCK_BYTES 18
#define ORC_Q8_0_BLOCK_BYTES 34
#define ORC_QK 32

/* ------------------------------------------------------------------------ */
/* IEEE 754 binary16 codec. The pages widen the stored f16 scale d to f32
 * ("dequant_q4_0": d widened to f32) and narrow the Q8_0 scale to f16
 * ("quantize_q8_0": the f16-narrowed d). Byte order of the stored d is not
 * stated on the pages; this oracle reads it little-endian (GGML's order). */

/* bfloat16 -> binary32. A bfloat16 value is the binary32 value whose upper
 * 16 bits are its bits and whose lower 16 bits are zero (the format is the
 * top half of binary32), so the widening is exact. Activations given as
 * bfloat16 enter the products through this. */
float orc_bf16_to_f32(uint16_t h)
{
    uint32_t bits = (uint32_t)h << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return f;
}

void orc_bf16_to_f32_array(const uint16_t *h, size_t n, float *out)
{
    for (size_t i = 0; i < n; ++i)
        out[i] = orc_bf16_to_f32(h[i]);
}

/* binary16 -> binary32. Exact: every binary16 value is a binary32 value. */
float orc_f16_to_f32(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1F;
    int frac = h & 0x3FF;
    double v;
    if (expo == 0)
        v = ldexp((double)frac, -24);               /* zero and subnormals */
    else if (expo == 31)
        v = frac ? (double)NAN : (double)INFINITY;  /* inf and NaN */
    else
        v = ldexp((double)(1024 + frac), expo - 25); /* (1 + frac/1024) * 2^(expo-15) */
    return (float)(sign ? -v : v);
}

/* binary32 -> binary16, round to nearest, ties to even (the IEEE default;
 * the pages do not name a rounding mode), with gradual underflow and overflow
 * to infinity. */
uint16_t orc_f32_to_f16(float f)
{
    uint16_t sign = signbit(f) ? 0x8000 : 0;
    if (isnan(f))
        return (uint16_t)(sign | 0x7E00);
    if (isinf(f))
        return (uint16_t)(sign | 0x7C00);
    double a = fabs((double)f);
    if (a == 0.0)
        return sign;
    int e2;
    frexp(a, &e2);            /* a in [2^(e2-1), 2^e2) */
    int binade = e2 - 1;
    if (binade < -14)
        binade = -14;         /* subnormal spacing is 2^-24 */
    double ulp = ldexp(1.0, binade - 10);
    double r = rint(a / ulp); /* a/ulp is exact; rint rounds half to even */
    double v = r * ulp;       /* the rounded magnitude (exact) */
    if (v > 65504.0)
        return (uint16_t)(sign | 0x7C00);
    if (v < ldexp(1.0, -14))  /* subnormal (or rounded up to 2^-14 below) */
        return (uint16_t)(sign | (uint16_t)(v / ldexp(1.0, -24)));
    frexp(v, &e2);
    int ve = e2 - 1;          /* v in [2^ve, 2^(ve+1)) */
    int mant = (int)(v / ldexp(1.0, ve - 10)) - 1024;
    return (uint16_t)(sign | (uint16_t)((ve + 15) << 10) | (uint16_t)mant);
}

/* ------------------------------------------------------------------------ */
/* Q4_0 dequant ("dequant_q4_0"): each 18-byte block holds a 2-byte f16 scale d
 * and 16 bytes of nibbles; byte j's low nibble is element j and its high nibble
 * is element j+16; each element is (nibble - 8) * d with d widened to f32. */
void orc_q4_0_dequant(const uint8_t *blob, size_t n_blocks, float *out)
{
    for (size_t b = 0; b < n_blocks; ++b) {
        const uint8_t *blk = blob + b * ORC_Q4_0_BLOCK_BYTES;
        float d = orc_f16_to_f32((uint16_t)(blk[0] | (blk[1] << 8)));
        for (int j = 0; j < 16; ++j) {
            int lo = blk[2 + j] & 0x0F;
            int hi = blk[2 + j] >> 4;
            out[b * ORC_QK + j] = (float)(lo - 8) * d;
            out[b * ORC_QK + 16 + j] = (float)(hi - 8) * d;
        }
    }
}

/* Q4_0 quantize (test-weight generation only; GGML's reference rule as stated
 * with the workloads). Per 32-element block:
 *   max = the element of largest |x| (the first one on ties, scanning up);
 *   d   = max / -8 in f32;
 *   q_j = min(15, (int)(x_j / d + 8.5)) with two separately rounded f32 ops,
 *         or 8 for every element when d == 0 (an all-zero block);
 *   store f16(d) little-endian, then byte j = q_j | q_{j+16} << 4.
 * (int) truncates toward zero. x_j/d lies in [-8, 8] for a normal d, so the
 * sum lies in [0.5, 16.5]; the lower clamp below only matters for a subnormal
 * d and keeps every code a valid nibble. */
void orc_q4_0_quantize(const float *x, size_t n, uint8_t *out)
{
    size_t n_blocks = n / ORC_QK;
    for (size_t b = 0; b < n_blocks; ++b) {
        const float *xb = x + b * ORC_QK;
        float amax = 0.0f, max = 0.0f;
        for (int j = 0; j < ORC_QK; ++j) {
            if (fabsf(xb[j]) > amax) {
                amax = fabsf(xb[j]);
                max = xb[j];
            }
        }
        float d = max / -8.0f;
        uint16_t dh = orc_f32_to_f16(d);
        uint8_t *blk = out + b * ORC_Q4_0_BLOCK_BYTES;
        blk[0] = (uint8_t)(dh & 0xFF);
        blk[1] = (uint8_t)(dh >> 8);
        int q[ORC_QK];
        for (int j = 0; j < ORC_QK; ++j) {
            if (d == 0.0f) {
                q[j] = 8;
            } else {
                float t = xb[j] / d;
                t = t + 8.5f;
                int c = (int)t;
                if (c > 15) c = 15;
                if (c < 0) c = 0;
                q[j] = c;
            }
        }
        for (int j = 0; j < 16; ++j)
            blk[2 + j] = (uint8_t)(q[j] | (q[j + 16] << 4));
    }
}

/* ------------------------------------------------------------------------ */
/* Q8_0 quantize ("quantize_q8_0"): per 32-element block, d = max|x| / 127,
 * store the f16-narrowed d, then 32 signed bytes q = round(x / d).
 * Readings where the page is silent: the division uses the f32 d (narrowing is
 * the storage step), round() is C roundf (half away from zero), and a block
 * with max|x| == 0 stores d = +0 and q = 0. */
void orc_q8_0_quantize(const float *x, size_t n, uint8_t *out)
{
    size_t n_blocks = n / ORC_QK;
    for (size_t b = 0; b < n_blocks; ++b) {
        const float *xb = x + b * ORC_QK;
        float amax = 0.0f;
        for (int j = 0; j < ORC_QK; ++j)
            if (fabsf(xb[j]) > amax)
                amax = fabsf(xb[j]);
        float d = amax / 127.0f;
        uint16_t dh = orc_f32_to_f16(d);
        uint8_t *blk = out + b * ORC_Q8_0_BLOCK_BYTES;
        blk[0] = (uint8_t)(dh & 0xFF);
        blk[1] = (uint8_t)(dh >> 8);
        for (int j = 0; j < ORC_QK; ++j) {
            int q = 0;
            if (d != 0.0f)
                q = (int)roundf(xb[j] / d);
            blk[2 + j] = (uint8_t)(int8_t)q;
        }
    }
}

/* Q8_0 dequant ("dequant_q8_0"): x = qs * d, qs a signed byte, d widened. */
void orc_q8_0_dequant(const uint8_t *blob, size_t n_blocks, float *out)
{
    for (size_t b = 0; b < n_blocks; ++b) {
        const uint8_t *blk = blob + b * ORC_Q8_0_BLOCK_BYTES;
        float d = orc_f16_to_f32((uint16_t)(blk[0] | (blk[1] << 8)));
        for (int j = 0; j < ORC_QK; ++j)
            out[b * ORC_QK + j] = (float)(int8_t)blk[2 + j] * d;
    }
}

/* ------------------------------------------------------------------------ */
/* Block-quantized x f32 product ("qmatvec_q4_0", "matmul_q4_0_tiled"):
 *   y[m, n] = sum_k a[m, k] * dequant(W)[n, k],
 * with a row-major [M, K] f32, W the row-major [N, K/32] block stream (Q4_0 or
 * Q8_0) and y row-major [M, N]. The weight is the dequantized value (the pages
 * multiply by dequant(W)). The sum runs over k in ascending order in f64; each
 * product of an f32 activation and a dequantized weight (24 x at most 18
 * significant bits) is exact in f64. bound[m, n] = sum_k |a[m, k] * w[n, k]| is
 * the scale of the parity tolerance. */
static void orc_dot_row(const float *arow, const float *wrow, int K,
                        double *y, double *bound)
{
    double s = 0.0, b = 0.0;
    for (int k = 0; k < K; ++k) {
        double p = (double)arow[k] * (double)wrow[k];
        s += p;
        b += fabs(p);
    }
    *y = s;
    *bound = b;
}

/* Weight row n of the stream, dequantized into wrow[K]. */
typedef void (*orc_dequant_fn)(const uint8_t *blob, size_t n_blocks, float *out);

/* Full product. threads <= 0 means the OpenMP default; the parallel loop is
 * over independent output columns and changes no result. Returns 0, or 1 for
 * a shape that breaks K % 32 == 0, or 2 when scratch memory is unavailable. */
static int orc_matmul(const float *a, const uint8_t *w, int M, int N, int K,
                      size_t block_bytes, orc_dequant_fn dequant,
                      double *y, double *bound, int threads)
{
    if (M < 0 || N < 0 || K < 0 || K % ORC_QK != 0)
        return 1;
    size_t row_bytes = (size_t)(K / ORC_QK) * block_bytes;
    int failed = 0;
    if (threads > 0)
        omp_set_num_threads(threads);
#pragma omp parallel
    {
        float *wrow = (float *)malloc((size_t)(K > 0 ? K : 1) * sizeof(float));
        if (!wrow) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(static)
        for (int n = 0; n < N; ++n) {
            if (!wrow)
                continue;
            dequant(w + (size_t)n * row_bytes, (size_t)(K / ORC_QK), wrow);
            for (int m = 0; m < M; ++m)
                orc_dot_row(a + (size_t)m * K, wrow, K,
                            y + (size_t)m * N + n, bound + (size_t)m * N + n);
        }
        free(wrow);
    }
    return failed ? 2 : 0;
}

/* The same product at a list of sampled outputs (m_idx[i], n_idx[i]), for
 * shapes too large to compute whole. */
static int orc_matmul_sampled(const float *a, const uint8_t *w, int M, int N, int K,
                              size_t block_bytes, orc_dequant_fn dequant,
                              const int64_t *m_idx, const int64_t *n_idx,
                              int64_t count, double *y, double *bound, int threads)
{
    if (M < 0 || N < 0 || K < 0 || K % ORC_QK != 0)
        return 1;
    for (int64_t i = 0; i < count; ++i)
        if (m_idx[i] < 0 || m_idx[i] >= M || n_idx[i] < 0 || n_idx[i] >= N)
            return 1;
    size_t row_bytes = (size_t)(K / ORC_QK) * block_bytes;
    int failed = 0;
    if (threads > 0)
        omp_set_num_threads(threads);
#pragma omp parallel
    {
        float *wrow = (float *)malloc((size_t)(K > 0 ? K : 1) * sizeof(float));
        if (!wrow) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(static)
        for (int64_t i = 0; i < count; ++i) {
            if (!wrow)
                continue;
            dequant(w + (size_t)n_idx[i] * row_bytes, (size_t)(K / ORC_QK), wrow);
            orc_dot_row(a + (size_t)m_idx[i] * K, wrow, K, y + i, bound + i);
        }
        free(wrow);
    }
    return failed ? 2 : 0;
}

int orc_q4_0_matmul(const float *a, const uint8_t *w, int M, int N, int K,
                    double *y, double *bound, int threads)
{
    return orc_matmul(a, w, M, N, K, ORC_Q4_0_BLOCK_BYTES, orc_q4_0_dequant, y, bound, threads);
}

int orc_q4_0_matmul_sampled(const float *a, const uint8_t *w, int M, int N, int K,
                            const int64_t *m_idx, const int64_t *n_idx,
                            int64_t count, double *y, double *bound, int threads)
{
    return orc_matmul_sampled(a, w, M, N, K, ORC_Q4_0_BLOCK_BYTES, orc_q4_0_dequant,
                              m_idx, n_idx, count, y, bound, threads);
}

int orc_q8_0_matmul(const float *a, const uint8_t *w, int M, int N, int K,
                    double *y, double *bound, int threads)
{
    return orc_matmul(a, w, M, N, K, ORC_Q8_0_BLOCK_BYTES, orc_q8_0_dequant, y, bound, threads);
}

int orc_q8_0_matmul_sampled(const float *a, const uint8_t *w, int M, int N, int K,
                            const int64_t *m_idx, const int64_t *n_idx,
                            int64_t count, double *y, double *bound, int threads)
{
    return orc_matmul_sampled(a, w, M, N, K, ORC_Q8_0_BLOCK_BYTES, orc_q8_0_dequant,
                              m_idx, n_idx, count, y, bound, threads);
}

/* Threads OpenMP will use for the next parallel region (for reporting). */
int orc_max_threads(void)
{
    return omp_get_max_threads();
}
