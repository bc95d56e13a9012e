/* Oracle driver for the sanitizer build: every entry point of oracle_gemm.c
 * on small problems of every layout and input type, row subsets and thread
 * counts, bad arguments, and the rounding and decoding helpers over special
 * values, built with AddressSanitizer and UndefinedBehaviorSanitizer.  The
 * results are checked against a direct double loop written here.  Exit status
 * 0 when every check holds. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_gemm(int64_t M, int64_t N, int64_t K, char a_major, char b_major, int in_type, const void* A,
                int64_t lda, const void* B, int64_t ldb, int64_t row0, int64_t row1, double* C_out, int nthreads);
float oracle_round_f32(double x);
uint16_t oracle_round_bf16(double x);
uint16_t oracle_round_f16(double x);
double oracle_decode_f16(uint16_t h);
double oracle_decode_bf16(uint16_t h);

static int failures = 0;
#define EXPECT(c) do { if (!(c)) { fprintf(stderr, "%s:%d: expected %s\n", __FILE__, __LINE__, #c); ++failures; } } while (0)

int main(void)
{
    const int64_t M = 7, N = 5, K = 9;
    for (int am = 0; am < 2; ++am)
        for (int bm = 0; bm < 2; ++bm) {
            const int64_t lda = (am ? M : K) + 3, ldb = (bm ? N : K) + 1;
            float* A = malloc(sizeof(float) * (size_t)((am ? K : M) * lda));
            float* B = malloc(sizeof(float) * (size_t)((bm ? K : N) * ldb));
            for (int64_t i = 0; i < (am ? K : M) * lda; ++i) A[i] = (float)((i * 7) % 11) - 5.f;
            for (int64_t i = 0; i < (bm ? K : N) * ldb; ++i) B[i] = (float)((i * 5) % 11) - 5.f;
            for (int threads = 1; threads <= 4; ++threads)
                for (int64_t r0 = 0; r0 <= M; r0 += 3) {
                    const int64_t r1 = M;
                    double* C = calloc((size_t)((r1 - r0) * N + 1), sizeof(double));
                    EXPECT(oracle_gemm(M, N, K, am ? 'm' : 'k', bm ? 'n' : 'k', 0, A, lda, B, ldb, r0, r1, C,
                                       threads) == 0);
                    for (int64_t m = r0; m < r1; ++m)
                        for (int64_t n = 0; n < N; ++n) {
                            double s = 0.0;
                            for (int64_t k = 0; k < K; ++k)
                                s += (double)A[am ? m + k * lda : m * lda + k] * (double)B[bm ? n + k * ldb : n * ldb + k];
                            EXPECT(C[(m - r0) * N + n] == s);
                        }
                    free(C);
                }
            free(A);
            free(B);
        }
    /* 16-bit inputs: all-ones patterns of fp16 (0x3c00) and bf16 (0x3f80) give K */
    uint16_t* h = malloc(sizeof(uint16_t) * 64);
    double C16[16];
    for (int t = 1; t <= 2; ++t) {
        for (int i = 0; i < 64; ++i) h[i] = t == 1 ? 0x3c00 : 0x3f80;
        EXPECT(oracle_gemm(4, 4, 16, 'k', 'k', t, h, 16, h, 16, 0, 4, C16, 2) == 0);
        for (int i = 0; i < 16; ++i) EXPECT(C16[i] == 16.0);
    }
    free(h);
    /* bad arguments and empty problems */
    double dummy[1];
    EXPECT(oracle_gemm(-1, 1, 1, 'k', 'k', 0, dummy, 1, dummy, 1, 0, 0, dummy, 1) == -1);
    EXPECT(oracle_gemm(2, 1, 1, 'x', 'k', 0, dummy, 1, dummy, 1, 0, 2, dummy, 1) == -1);
    EXPECT(oracle_gemm(2, 1, 1, 'k', 'k', 7, dummy, 1, dummy, 1, 0, 2, dummy, 1) == -1);
    EXPECT(oracle_gemm(2, 1, 1, 'k', 'k', 0, dummy, 1, dummy, 1, 1, 3, dummy, 1) == -1);
    EXPECT(oracle_gemm(0, 0, 0, 'k', 'k', 0, NULL, 1, NULL, 1, 0, 0, NULL, 1) == 0);
    /* rounding and decoding over special values and every 16-bit pattern */
    const double xs[] = {0.0, -0.0, 1.0, -1.0, 65504.0, 65520.0, 1e-8, -1e-8, 5.96e-8, 3.4e38, 3.5e38, 1e300,
                         -1e300, INFINITY, -INFINITY, NAN, 0.1, 1.0 / 3.0};
    for (size_t i = 0; i < sizeof xs / sizeof xs[0]; ++i) {
        (void)oracle_round_f32(xs[i]);
        (void)oracle_round_bf16(xs[i]);
        (void)oracle_round_f16(xs[i]);
    }
    for (uint32_t v = 0; v < 65536; ++v) {
        const double a = oracle_decode_f16((uint16_t)v), b = oracle_decode_bf16((uint16_t)v);
        if (!isnan(a)) EXPECT(oracle_round_f16(a) == (uint16_t)v || a == 0.0);
        if (!isnan(b)) EXPECT(oracle_round_bf16(b) == (uint16_t)v || b == 0.0);
    }
    fprintf(stderr, "oracle driver: %d failure(s)\n", failures);
    return failures == 0 ? 0 : 1;
}
