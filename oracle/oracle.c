/*
 * oracle.c -- plain, slow, fp64 reference for the fp8 (OCP e4m3) block-scaled GEMM.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or call this
 * file: only the tests, the smoke check and the bench's CPU-baseline leg use it.
 * It shares no code, header, table or helper with the HIP library.
 *
 * What it computes is the definition of the operation, written out:
 *
 *   route BS (page "Flydsl Fp8 Blockscale Gemm", Mechanism A and Procedure step 1:
 *   fp32 dequant -> matmul -> bf16, with fp32 per-1x128 activation scales and fp32
 *   per-[128,128] weight scales):
 *       C[m,n] = bf16( sum_kb a_s[m,kb] * b_s[n/128,kb] * sum_{k in block kb} A[m,k]*B[n,k] )
 *
 *   route MX (page "aiter PR #6370", "Why it is faster" and "Correctness": 1x32 ue8m0
 *   scales are exact powers of two applied per 32-wide K group):
 *       C[m,n] = bf16( sum_g 2^(ea[m,g]-127) * 2^(eb[n,g]-127) * sum_{k in group g} A[m,k]*B[n,k] )
 *
 *   route PT (the promote-free twin, see oracle_pt_gemm): one fp32 scale per row of A and
 *   one per row of B:
 *       C[m,n] = bf16( a_s[m] * b_s[n] * sum_k A[m,k]*B[n,k] )
 *
 * Precision: every e4m3 value is an integer times 2^-9, so every product is an integer
 * times 2^-18 below 2^36 and a 128-term block sum stays below 2^43: the block sums are
 * exact in fp64. The scale product a_s*b_s (24+24 significant bits) is exact in fp64.
 * Only the scaling of a block sum and the sum over blocks round, at 2^-53 relative.
 * The result is rounded ONCE, from fp64 straight to bf16, round-to-nearest-even.
 *
 * Readings where the pages are silent (each listed in the design notes): bf16 rounding is
 * round-to-nearest-even; e4m3 NaN codes (0x7F, 0xFF) decode to NaN and propagate; ue8m0
 * byte 255 (NaN) propagates NaN.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* OCP FP8 E4M3 ("fn" flavour): 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits,
 * no infinities, NaN only for S.1111.111, largest finite magnitude 448, smallest
 * subnormal 2^-9. */
static double e4m3_decode(uint8_t c)
{
    int s = c >> 7;
    int e = (c >> 3) & 15;
    int f = c & 7;
    double v;
    if (e == 15 && f == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)f, -9);            /* subnormal: f/8 * 2^(1-7) */
    else
        v = ldexp((double)(8 + f), e - 10);  /* normal: (1 + f/8) * 2^(e-7) */
    return s ? -v : v;
}

/* ue8m0: an unsigned biased exponent, value 2^(byte-127); 255 is NaN. */
static double e8m0_decode(uint8_t b)
{
    if (b == 255)
        return NAN;
    return ldexp(1.0, (int)b - 127);
}

/* Round a double to the nearest bfloat16 (8 significant bits, exponent range of fp32),
 * ties to even, and return its 16-bit pattern. Rounding happens exactly once. */
static uint16_t bf16_round_from_f64(double x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double v = fabs(x);
    if (isnan(x))
        return 0x7FC0;
    /* Largest finite bf16 is (2 - 2^-7) * 2^127. The midpoint between it and 2^128 is
     * (2 - 2^-8) * 2^127; at or above it the value rounds to infinity (at exactly the
     * midpoint the even neighbour is 2^128, whose mantissa is zero). */
    if (v >= ldexp(2.0 - ldexp(1.0, -8), 127))
        return sign | 0x7F80;
    if (v == 0.0)
        return sign;
    int ex;
    frexp(v, &ex);                 /* v = f * 2^ex, f in [0.5, 1): floor(log2 v) = ex - 1 */
    int e = ex - 1;
    if (e < -126)
        e = -126;                  /* subnormal range: fixed quantum 2^-133 */
    double quantum = ldexp(1.0, e - 7);
    double q = v / quantum;        /* exact: scaling by a power of two */
    double r = nearbyint(q);       /* default rounding mode is to-nearest-even */
    double rounded = r * quantum;  /* exactly representable in bf16 (may step to the next binade) */
    float f32 = (float)rounded;    /* exact: bf16 values are fp32 values */
    uint32_t bits;
    memcpy(&bits, &f32, 4);
    return sign | (uint16_t)(bits >> 16);
}

/* Route BS.
 *   A       [M, K] e4m3 codes, row-major
 *   a_scale [M, K/128] fp32, row-major (a_s[m, kb])
 *   B       [N, K] e4m3 codes, row-major
 *   b_scale [ceil(N/128), K/128] fp32, row-major (b_s[nb, kb])
 * Computes C at the grid rows[0..nr) x cols[0..nc): out_acc[i*nc + j] is the fp64 sum
 * for (rows[i], cols[j]) and out_bf16[i*nc + j] its bf16 bit pattern. Either output may
 * be NULL. K must be a multiple of 128. */
void oracle_bs_gemm(const uint8_t *A, const float *a_scale, const uint8_t *B,
                    const float *b_scale, int M, int N, int K, const int *rows, int nr,
                    const int *cols, int nc, double *out_acc, uint16_t *out_bf16)
{
    const int KB = K / 128;
    double table[256];
    (void)M;
    (void)N;
    for (int c = 0; c < 256; c++)
        table[c] = e4m3_decode((uint8_t)c);
#pragma omp parallel for schedule(dynamic, 1)
    for (int i = 0; i < nr; i++) {
        const int m = rows[i];
        double *arow = (double *)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
        for (int k = 0; k < K; k++)
            arow[k] = table[A[(size_t)m * K + k]];
        for (int j = 0; j < nc; j++) {
            const int n = cols[j];
            const uint8_t *brow = B + (size_t)n * K;
            double acc = 0.0;
            for (int kb = 0; kb < KB; kb++) {
                double p = 0.0;
                for (int k = kb * 128; k < kb * 128 + 128; k++)
                    p += arow[k] * table[brow[k]];
                double s = (double)a_scale[(size_t)m * KB + kb] *
                           (double)b_scale[(size_t)(n / 128) * KB + kb];
                acc += p * s;
            }
            if (out_acc)
                out_acc[(size_t)i * nc + j] = acc;
            if (out_bf16)
                out_bf16[(size_t)i * nc + j] = bf16_round_from_f64(acc);
        }
        free(arow);
    }
}

/* Route MX.
 *   A      [M, K] e4m3 codes, row-major;   a_e8m0 [M, K/32] ue8m0 bytes, row-major
 *   B      [N, K] e4m3 codes, row-major;   b_e8m0 [N, K/32] ue8m0 bytes, row-major
 * Same output convention as oracle_bs_gemm. K must be a multiple of 32. */
void oracle_mx_gemm(const uint8_t *A, const uint8_t *a_e8m0, const uint8_t *B,
                    const uint8_t *b_e8m0, int M, int N, int K, const int *rows, int nr,
                    const int *cols, int nc, double *out_acc, uint16_t *out_bf16)
{
    const int G = K / 32;
    double table[256];
    (void)M;
    (void)N;
    for (int c = 0; c < 256; c++)
        table[c] = e4m3_decode((uint8_t)c);
#pragma omp parallel for schedule(dynamic, 1)
    for (int i = 0; i < nr; i++) {
        const int m = rows[i];
        double *arow = (double *)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
        for (int k = 0; k < K; k++)
            arow[k] = table[A[(size_t)m * K + k]];
        for (int j = 0; j < nc; j++) {
            const int n = cols[j];
            const uint8_t *brow = B + (size_t)n * K;
            double acc = 0.0;
            for (int g = 0; g < G; g++) {
                double p = 0.0;
                for (int k = g * 32; k < g * 32 + 32; k++)
                    p += arow[k] * table[brow[k]];
                acc += p * e8m0_decode(a_e8m0[(size_t)m * G + g]) *
                       e8m0_decode(b_e8m0[(size_t)n * G + g]);
            }
            if (out_acc)
                out_acc[(size_t)i * nc + j] = acc;
            if (out_bf16)
                out_bf16[(size_t)i * nc + j] = bf16_round_from_f64(acc);
        }
        free(arow);
    }
}

/* Route PT, the promote-free twin of route BS (page "Flydsl Fp8 Blockscale Gemm",
 * Bottleneck diagnosis, item 2: the same matrix work with a cheap row-by-column scale in
 * place of the per-block promote; page "aiter PR #6370" calls the per-token / per-channel
 * kernel "ptpc"):
 *   A [M, K] e4m3 codes, a_scale [M] fp32 (one per row of A, per token)
 *   B [N, K] e4m3 codes, b_scale [N] fp32 (one per row of B, per output channel)
 *       C[m,n] = bf16( a_s[m] * b_s[n] * sum_k A[m,k]*B[n,k] )
 * The dot product is exact in fp64 while K <= 2^17 (each product is an integer times 2^-18
 * below 2^36), a_s*b_s is exact, and their product rounds once before the bf16 rounding.
 * Same output convention as oracle_bs_gemm. */
void oracle_pt_gemm(const uint8_t *A, const float *a_scale, const uint8_t *B,
                    const float *b_scale, int M, int N, int K, const int *rows, int nr,
                    const int *cols, int nc, double *out_acc, uint16_t *out_bf16)
{
    double table[256];
    (void)M;
    (void)N;
    for (int c = 0; c < 256; c++)
        table[c] = e4m3_decode((uint8_t)c);
#pragma omp parallel for schedule(dynamic, 1)
    for (int i = 0; i < nr; i++) {
        const int m = rows[i];
        double *arow = (double *)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
        for (int k = 0; k < K; k++)
            arow[k] = table[A[(size_t)m * K + k]];
        for (int j = 0; j < nc; j++) {
            const int n = cols[j];
            const uint8_t *brow = B + (size_t)n * K;
            double dot = 0.0;
            for (int k = 0; k < K; k++)
                dot += arow[k] * table[brow[k]];
            const double acc = dot * ((double)a_scale[m] * (double)b_scale[n]);
            if (out_acc)
                out_acc[(size_t)i * nc + j] = acc;
            if (out_bf16)
                out_bf16[(size_t)i * nc + j] = bf16_round_from_f64(acc);
        }
        free(arow);
    }
}

/* ---- activation quantisers (the step before the GEMM) ---------------------------------
 * Route BS (page "Flydsl Fp8 Blockscale Gemm", Procedure step 6, and the 1x128 activation
 * groups of Mechanism A): per 1x128 group of a row, scale = amax / 448 in fp32 (1 for an
 * all-zero group), codes = e4m3(x / scale), the division in fp32.
 * Route MX (page "aiter PR #6370", "Why it is faster"): per 1x32 group, the smallest integer
 * e with amax <= 448 * 2^e (clamped to [-127, 127]; 0 for an all-zero group) is stored as the
 * ue8m0 byte e + 127, codes = e4m3(x * 2^-e) (exact scaling).
 * The e4m3 encoding is the nearest finite code, ties to the code with an even mantissa, and
 * saturates at +-448 (plainest reading: the pages quantise with scale amax/448, so in-range
 * values never exceed 448 by more than a rounding step). A NaN element encodes as NaN and is
 * left out of its group's amax (the pages say nothing about NaN inputs). */

/* Nearest finite e4m3 code to x (|x| handled by search over all 127 finite magnitudes). */
static uint8_t e4m3_encode_nearest(float x)
{
    if (isnan(x))
        return signbit(x) ? 0xFF : 0x7F;
    const double a = fabs((double)x);
    int best = 0;
    double best_d = INFINITY;
    for (int c = 0; c <= 0x7E; c++) {
        const double d = fabs(e4m3_decode((uint8_t)c) - a);
        /* strictly closer, or equally close and even (ties to even mantissa) */
        if (d < best_d || (d == best_d && (c & 1) == 0)) {
            best = c;
            best_d = d;
        }
    }
    return (uint8_t)(signbit(x) ? (best | 0x80) : best);
}

/* x [M, K] fp32 row-major -> codes [M, K], scale [M, K/128] fp32 (row-major, a_s[m, kb]). */
void oracle_quantize_bs(const float *x, int M, int K, uint8_t *codes, float *scale)
{
    const int KB = K / 128;
#pragma omp parallel for schedule(static)
    for (int m = 0; m < M; m++) {
        for (int kb = 0; kb < KB; kb++) {
            const float *g = x + (size_t)m * K + (size_t)kb * 128;
            float amax = 0.0f;
            for (int k = 0; k < 128; k++)
                if (fabsf(g[k]) > amax)  /* false for NaN: NaN is left out */
                    amax = fabsf(g[k]);
            float s = amax / 448.0f;
            if (amax == 0.0f)
                s = 1.0f;
            scale[(size_t)m * KB + kb] = s;
            for (int k = 0; k < 128; k++) {
                const float q = isnan(g[k]) ? g[k] : g[k] / s;  /* NaN keeps its own sign */
                codes[(size_t)m * K + (size_t)kb * 128 + k] = e4m3_encode_nearest(q);
            }
        }
    }
}

/* x [M, K] fp32 row-major -> codes [M, K], e8m0 [M, K/32] bytes (row-major). */
void oracle_quantize_mx(const float *x, int M, int K, uint8_t *codes, uint8_t *e8m0)
{
    const int G = K / 32;
#pragma omp parallel for schedule(static)
    for (int m = 0; m < M; m++) {
        for (int gi = 0; gi < G; gi++) {
            const float *g = x + (size_t)m * K + (size_t)gi * 32;
            double amax = 0.0;
            for (int k = 0; k < 32; k++)
                if (fabs((double)g[k]) > amax)
                    amax = fabs((double)g[k]);
            int e = 0;
            if (amax > 0.0) {
                /* the smallest e with amax <= 448 * 2^e, by direct search */
                e = -140;
                while (amax > ldexp(448.0, e))
                    e++;
                if (e < -127)
                    e = -127;
                if (e > 127)
                    e = 127;
            }
            e8m0[(size_t)m * G + gi] = (uint8_t)(e + 127);
            for (int k = 0; k < 32; k++) {
                const float q = isnan(g[k]) ? g[k] : (float)ldexp((double)g[k], -e);
                codes[(size_t)m * K + (size_t)gi * 32 + k] = e4m3_encode_nearest(q);
            }
        }
    }
}

/* Exposed so the tests can pin the codecs on their own. */
double oracle_e4m3_decode(uint8_t c) { return e4m3_decode(c); }
double oracle_e8m0_decode(uint8_t b) { return e8m0_decode(b); }
uint8_t oracle_e4m3_encode(float x) { return e4m3_encode_nearest(x); }
uint16_t oracle_bf16_round(double x) { return bf16_round_from_f64(x); }

/* Number of OpenMP threads a parallel region would use (0 when built without OpenMP). */
#ifdef _OPENMP
#include <omp.h>
int oracle_num_threads(void) { return omp_get_max_threads(); }
#else
int oracle_num_threads(void) { return 0; }
#endif
