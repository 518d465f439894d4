/*
 * gemm_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow CPU reference for the dense product C[M,N] = A[M,K] x B[K,N].
 * Only the test suite, the package smoke check and the CPU-baseline leg of the
 * benchmark may load this file's library.  It shares no code, header, table or
 * helper with the GPU path and includes nothing from it.
 *
 * What it computes (the definition, written out):
 *   C[i][j] = sum over k = 0 .. K-1 of A[i][k] * B[k][j]
 * as stated in "CUDA tile" (2.1, the block-tiling walk-through, where the
 * element formula of the product is written out) and in "Tiling 策略与内存层次
 * 优化" (the roofline section's GEMM example C[M,N] = A[M,K] x B[K,N]).
 * Tiling only reorders data movement; the partial sums over K slabs add up to
 * the same total (qian.cx tiling note, the K-split paragraph), and zero padding
 * of edge tiles contributes nothing because 0 is the identity of the sum
 * ("CUDA tile", 4, boundary checks).  So the oracle is the untiled sum.
 *
 * Arithmetic: every element is decoded exactly to binary64; every product of two
 * fp16, bf16 or fp32 values is exact in binary64 (at most 48 significant bits);
 * each output element is one running binary64 sum with k ascending.  Build with
 * -ffp-contract=off so no fused multiply-add changes a rounding.
 *
 * Storage addressing (row-major C with leading dimension N in the output):
 *   A(i,k) = A[i*lda + k]  (A row-major)     A(i,k) = A[k*lda + i]  (A column-major)
 *   B(k,j) = B[k*ldb + j]  (B row-major)     B(k,j) = B[j*ldb + k]  (B column-major)
 *
 * Element codes: 0 = fp32, 1 = fp16 (IEEE binary16), 2 = bf16 (upper half of binary32).
 * The fp16 and bf16 decoders and the binary64 -> fp16/bf16 round-to-nearest-even
 * encoders below are written from the IEEE 754 field definitions (sign, biased
 * exponent, trailing significand), not from any other code in this repository.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_F32 0
#define OR_F16 1
#define OR_BF16 2

/* ---- element decoders (exact) ------------------------------------------------ */

/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 trailing significand bits. */
double oracle_decode_f16(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1f;
    int frac = h & 0x3ff;
    double mag;
    if (expo == 0)
        mag = ldexp((double)frac, -24);            /* subnormal: frac * 2^(1-15-10) */
    else if (expo == 0x1f)
        mag = frac ? NAN : INFINITY;
    else
        mag = ldexp((double)(frac + 1024), expo - 25); /* (1.frac) * 2^(expo-15) */
    return sign ? -mag : mag;
}

/* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 trailing significand bits. */
double oracle_decode_bf16(uint16_t b)
{
    int sign = (b >> 15) & 1;
    int expo = (b >> 7) & 0xff;
    int frac = b & 0x7f;
    double mag;
    if (expo == 0)
        mag = ldexp((double)frac, -133);           /* subnormal: frac * 2^(1-127-7) */
    else if (expo == 0xff)
        mag = frac ? NAN : INFINITY;
    else
        mag = ldexp((double)(frac + 128), expo - 134); /* (1.frac) * 2^(expo-127) */
    return sign ? -mag : mag;
}

static double decode_at(const void *base, int64_t idx, int code)
{
    if (code == OR_F32) {
        float f;
        memcpy(&f, (const char *)base + idx * 4, 4);
        return (double)f;
    }
    uint16_t u;
    memcpy(&u, (const char *)base + idx * 2, 2);
    return code == OR_F16 ? oracle_decode_f16(u) : oracle_decode_bf16(u);
}

/* ---- round-to-nearest-even encoders (binary64 -> 16-bit formats) ----------------
 * Generic rule for a binary format with p-1 trailing significand bits, minimum
 * normal exponent emin and maximum finite value vmax: the representable values
 * around |x| are spaced by the quantum 2^(max(e, emin) - (p-1)), where 2^e <= |x| <
 * 2^(e+1).  Divide by the quantum (exact: power of two), round the quotient to
 * the nearest integer with ties to even (rint in the default rounding mode), and
 * multiply back; a result above vmax overflows to infinity. */
static double round_to_format(double a, int mant_bits, int emin)
{
    int e;
    frexp(a, &e);                 /* a = f * 2^e with f in [0.5, 1): 2^(e-1) <= a < 2^e */
    int unb = e - 1;
    if (unb < emin)
        unb = emin;               /* subnormal range shares the quantum of the smallest binade */
    double q = ldexp(1.0, unb - mant_bits);
    return rint(a / q) * q;
}

uint16_t oracle_encode_f16(double x)
{
    if (isnan(x))
        return 0x7e00;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (a == 0.0)
        return sign;
    double v = isinf(a) ? INFINITY : round_to_format(a, 10, -14);
    if (v > 65504.0)
        return sign | 0x7c00;
    if (v == 0.0)
        return sign;
    if (v < ldexp(1.0, -14))
        return sign | (uint16_t)(v / ldexp(1.0, -24));          /* subnormal count */
    int e;
    frexp(v, &e);
    int unb = e - 1;
    uint16_t frac = (uint16_t)(v / ldexp(1.0, unb - 10) - 1024.0);
    return sign | (uint16_t)((unb + 15) << 10) | frac;
}

uint16_t oracle_encode_bf16(double x)
{
    if (isnan(x))
        return 0x7fc0;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (a == 0.0)
        return sign;
    double vmax = ldexp(255.0, 120);                            /* (2 - 2^-7) * 2^127 */
    double v = isinf(a) ? INFINITY : round_to_format(a, 7, -126);
    if (v > vmax)
        return sign | 0x7f80;
    if (v == 0.0)
        return sign;
    if (v < ldexp(1.0, -126))
        return sign | (uint16_t)(v / ldexp(1.0, -133));
    int e;
    frexp(v, &e);
    int unb = e - 1;
    uint16_t frac = (uint16_t)(v / ldexp(1.0, unb - 7) - 128.0);
    return sign | (uint16_t)((unb + 127) << 7) | frac;
}

void oracle_encode_array(const double *src, uint16_t *dst, int64_t n, int code)
{
    for (int64_t i = 0; i < n; ++i)
        dst[i] = code == OR_F16 ? oracle_encode_f16(src[i]) : oracle_encode_bf16(src[i]);
}

void oracle_decode_array(const void *src, double *dst, int64_t n, int code)
{
    for (int64_t i = 0; i < n; ++i)
        dst[i] = decode_at(src, i, code);
}

/* ---- the product ---------------------------------------------------------------
 * Rows [row0, row1) of C (row-major, leading dimension N) are written.  B is
 * decoded once into a dense binary64 K x N array so that the inner loop reads
 * plain doubles; each row of A is decoded into a K-vector.  The loop nest is
 * i, k, j with one running sum per output element C[i][j] (acc[j]), k ascending:
 * the same additions in the same order as the i, j, k textbook nest.
 * Returns 0, or -1 when memory for the decoded operands cannot be obtained. */
int oracle_gemm_rows(int64_t M, int64_t N, int64_t K,
                     const void *A, int64_t lda, int a_col,
                     const void *B, int64_t ldb, int b_col,
                     int code, int64_t row0, int64_t row1, double *C)
{
    (void)M;
    if (row1 <= row0 || N <= 0)
        return 0;
    double *Bd = NULL;
    if (K > 0) {
        Bd = (double *)malloc(sizeof(double) * (size_t)K * (size_t)N);
        if (!Bd)
            return -1;
#pragma omp parallel for schedule(static)
        for (int64_t k = 0; k < K; ++k)
            for (int64_t j = 0; j < N; ++j)
                Bd[k * N + j] = decode_at(B, b_col ? j * ldb + k : k * ldb + j, code);
    }
    int failed = 0;
#pragma omp parallel
    {
        double *arow = (double *)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
        if (!arow) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(static)
            for (int64_t i = row0; i < row1; ++i) {
                double *acc = C + (i - row0) * N;
                for (int64_t k = 0; k < K; ++k)
                    arow[k] = decode_at(A, a_col ? k * lda + i : i * lda + k, code);
                for (int64_t j = 0; j < N; ++j)
                    acc[j] = 0.0;
                for (int64_t k = 0; k < K; ++k) {
                    const double a = arow[k];
                    const double *brow = Bd + k * N;
                    for (int64_t j = 0; j < N; ++j)
                        acc[j] += a * brow[j];
                }
            }
            free(arow);
        }
    }
    free(Bd);
    return failed ? -1 : 0;
}

/* Individual elements C[ii[t]][jj[t]] for t in [0, n): one dot product each, in
 * the same k-ascending order, decoding operands on the fly (no workspace).  Used
 * to check sampled outputs of products too large to form whole on the CPU. */
void oracle_gemm_elements(int64_t K,
                          const void *A, int64_t lda, int a_col,
                          const void *B, int64_t ldb, int b_col,
                          int code, const int64_t *ii, const int64_t *jj, int64_t n,
                          double *out)
{
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t t = 0; t < n; ++t) {
        const int64_t i = ii[t], j = jj[t];
        double s = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double a = decode_at(A, a_col ? k * lda + i : i * lda + k, code);
            double b = decode_at(B, b_col ? j * ldb + k : k * ldb + j, code);
            s += a * b;
        }
        out[t] = s;
    }
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Thread count of the parallel loops above (timing of the oracle on a given number of
 * host cores); n < 1 is taken as 1.  The results do not depend on it. */
void oracle_set_threads(int n)
{
#ifdef _OPENMP
    extern void omp_set_num_threads(int);
    omp_set_num_threads(n < 1 ? 1 : n);
#else
    (void)n;
#endif
}
