/* Sanitizer run of the oracle (tests/test_sanitizers.py builds this with ASan and UBSan
 * and runs it on the CPU): every entry point of oracle/gemm_oracle.c over small and
 * edge-case shapes, every layout and element code, padded leading dimensions, row
 * ranges, sampled elements and every 16-bit pattern through the codecs.  Each operand
 * is allocated at exactly the size its extents need, so an access past it is reported.
 * Prints "oracle sanitizer run ok" at the end. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double oracle_decode_f16(uint16_t h);
double oracle_decode_bf16(uint16_t b);
uint16_t oracle_encode_f16(double x);
uint16_t oracle_encode_bf16(double x);
void oracle_encode_array(const double *src, uint16_t *dst, int64_t n, int code);
void oracle_decode_array(const void *src, double *dst, int64_t n, int code);
int oracle_gemm_rows(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, int a_col, const void *B,
                     int64_t ldb, int b_col, int code, int64_t row0, int64_t row1, double *C);
void oracle_gemm_elements(int64_t K, const void *A, int64_t lda, int a_col, const void *B, int64_t ldb, int b_col,
                          int code, const int64_t *ii, const int64_t *jj, int64_t n, double *out);
void oracle_set_threads(int n);

static int64_t need(int64_t rows, int64_t cols, int64_t ld) { return rows && cols ? (rows - 1) * ld + cols : 0; }

static void *operand(int64_t elems, int code, unsigned seed) {
    const size_t esz = code == 0 ? 4 : 2;
    unsigned char *p = (unsigned char *)malloc(elems ? (size_t)elems * esz : 1);
    for (int64_t i = 0; i < elems; ++i) {
        seed = seed * 1103515245u + 12345u;
        if (code == 0) {
            float f = (float)((int)(seed >> 16) % 9 - 4);
            memcpy(p + i * 4, &f, 4);
        } else {
            uint16_t h = code == 1 ? oracle_encode_f16((double)((int)(seed >> 16) % 9 - 4))
                                   : oracle_encode_bf16((double)((int)(seed >> 16) % 9 - 4));
            memcpy(p + i * 2, &h, 2);
        }
    }
    return p;
}

int main(void) {
    const int64_t ext[] = {0, 1, 2, 3, 7, 16, 33};
    int cases = 0;
    for (int threads = 1; threads <= 3; threads += 2) {
        oracle_set_threads(threads);
        for (int code = 0; code < 3; ++code)
            for (int lay = 0; lay < 4; ++lay)
                for (int im = 0; im < 7; ++im)
                    for (int in = 0; in < 7; ++in)
                        for (int ik = 0; ik < 7; ik += 2) {
                            const int64_t M = ext[im], N = ext[in], K = ext[ik];
                            const int a_col = lay & 1, b_col = (lay >> 1) & 1;
                            const int64_t lda = (a_col ? M : K) + (im & 1), ldb = (b_col ? K : N) + (in & 1);
                            const int64_t na = a_col ? need(K, M, lda) : need(M, K, lda);
                            const int64_t nb = b_col ? need(N, K, ldb) : need(K, N, ldb);
                            void *A = operand(na, code, 1u + (unsigned)cases);
                            void *B = operand(nb, code, 7u + (unsigned)cases);
                            double *C = (double *)malloc((size_t)(M * N > 0 ? M * N : 1) * sizeof(double));
                            if (oracle_gemm_rows(M, N, K, A, lda, a_col, B, ldb, b_col, code, 0, M, C) != 0) return 1;
                            if (M > 1 && oracle_gemm_rows(M, N, K, A, lda, a_col, B, ldb, b_col, code, 1, M, C) != 0)
                                return 1;
                            if (M > 0 && N > 0) {
                                int64_t ii[3] = {0, M - 1, M / 2}, jj[3] = {N - 1, 0, N / 2};
                                double e[3];
                                oracle_gemm_elements(K, A, lda, a_col, B, ldb, b_col, code, ii, jj, 3, e);
                            }
                            free(A);
                            free(B);
                            free(C);
                            ++cases;
                        }
    }
    /* codecs: every 16-bit pattern, both ways */
    uint16_t *bits = (uint16_t *)malloc(65536 * sizeof(uint16_t));
    double *vals = (double *)malloc(65536 * sizeof(double));
    uint16_t *back = (uint16_t *)malloc(65536 * sizeof(uint16_t));
    for (int i = 0; i < 65536; ++i) bits[i] = (uint16_t)i;
    for (int code = 1; code < 3; ++code) {
        oracle_decode_array(bits, vals, 65536, code);
        oracle_encode_array(vals, back, 65536, code);
    }
    float f4[5] = {0.0f, -1.5f, 3.0e38f, 1.0e-45f, -0.0f};
    double d4[5];
    oracle_decode_array(f4, d4, 5, 0);
    free(bits);
    free(vals);
    free(back);
    printf("oracle sanitizer run ok (%d products)\n", cases);
    return 0;
}
