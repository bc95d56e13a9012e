/*
 * oracle_gemm.c -- plain CPU reference for the dense GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code, header, table or helper with the
 * HIP library.
 *
 * What it computes (CuTe DSL Ampere SGEMM example, module docstring and the
 * reference check in run(); CK Tile practice GEMM README, "Host Matrix
 * Creation"): A is logically M x K, B is logically N x K, C is M x N and
 *
 *     C[m][n] = sum over k = 0 .. K-1 of A[m][k] * B[n][k]
 *
 * Each element is accumulated in IEEE double, k ascending, with the multiply
 * and the add as separate operations (this file must be built with
 * -ffp-contract=off and without fast-math).  Inputs of type fp32, fp16 and
 * bf16 convert to double exactly and every pairwise product is exact in
 * double, so the only rounding is in the K-1 additions.
 *
 * Storage ("major" = the index that is contiguous), as the SGEMM example's
 * create_and_permute_tensor() and its --a_major/--b_major/--c_major flags
 * define it:
 *   A 'k': A[m][k] at A + m*lda + k        A 'm': at A + m + k*lda
 *   B 'k': B[n][k] at B + n*ldb + k        B 'n': at B + n + k*ldb
 * The result is returned as a dense row-major M x N array of doubles; the
 * caller rounds it to the output type with the oracle_round_* functions.
 *
 * Parallelism: rows of C are split evenly over POSIX threads, and each thread
 * walks four columns of a row at a time.  Neither changes the sequence of
 * operations of any element.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { IN_F32 = 0, IN_F16 = 1, IN_BF16 = 2 };

/* ---- element decoding, from the IEEE 754 binary16 / bfloat16 formats ---- */

/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double oracle_decode_f16(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);                 /* zero or subnormal: f * 2^-24 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);     /* (1 + f/2^10) * 2^(e-15) */
    return sign ? -v : v;
}

/* bfloat16 is the upper half of an IEEE binary32. */
double oracle_decode_bf16(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double element(const void* base, int in_type, int64_t idx)
{
    switch (in_type) {
    case IN_F32: return (double)((const float*)base)[idx];
    case IN_F16: return oracle_decode_f16(((const uint16_t*)base)[idx]);
    default:     return oracle_decode_bf16(((const uint16_t*)base)[idx]);
    }
}

/* ---- the definition ---- */

typedef struct {
    int64_t N, K;
    const double* A;   /* rows [row0, row1) of logical A, each K long */
    const double* B;   /* logical B, N rows of K */
    double* C;         /* rows [row0, row1) of C, each N long */
    int64_t r_begin, r_end;  /* local row range for this thread */
} job_t;

static void* run_rows(void* arg)
{
    const job_t* j = (const job_t*)arg;
    const int64_t N = j->N, K = j->K;
    for (int64_t m = j->r_begin; m < j->r_end; ++m) {
        const double* a = j->A + m * K;
        double* c = j->C + m * N;
        int64_t n = 0;
        /* Four columns side by side: four independent sums, each still one
         * fp64 multiply and one fp64 add per k, k ascending. */
        for (; n + 4 <= N; n += 4) {
            const double* b0 = j->B + n * K;
            const double* b1 = b0 + K;
            const double* b2 = b1 + K;
            const double* b3 = b2 + K;
            double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const double x = a[k];
                s0 = s0 + x * b0[k];
                s1 = s1 + x * b1[k];
                s2 = s2 + x * b2[k];
                s3 = s3 + x * b3[k];
            }
            c[n] = s0;
            c[n + 1] = s1;
            c[n + 2] = s2;
            c[n + 3] = s3;
        }
        for (; n < N; ++n) {
            const double* b = j->B + n * K;
            double s = 0.0;
            for (int64_t k = 0; k < K; ++k)
                s = s + a[k] * b[k];
            c[n] = s;
        }
    }
    return NULL;
}

/*
 * oracle_gemm: rows [row0, row1) of C = A * B^T (storage B is N x K).
 *   in_type: 0 fp32, 1 fp16, 2 bf16 (raw 16-bit patterns for the latter two)
 *   C_out:   (row1 - row0) x N doubles, row-major, caller-allocated
 *   nthreads <= 0 means one thread.
 * Returns 0, or -1 on a bad argument, -2 when memory runs out.
 */
int oracle_gemm(int64_t M, int64_t N, int64_t K, char a_major, char b_major, int in_type,
                const void* A, int64_t lda, const void* B, int64_t ldb,
                int64_t row0, int64_t row1, double* C_out, int nthreads)
{
    if (M < 0 || N < 0 || K < 0 || row0 < 0 || row1 > M || row0 > row1) return -1;
    if (in_type < IN_F32 || in_type > IN_BF16) return -1;
    if (a_major != 'k' && a_major != 'm') return -1;
    if (b_major != 'k' && b_major != 'n') return -1;
    int64_t rows = row1 - row0;
    if (rows == 0 || N == 0) return 0;

    /* Read the logical matrices out of their storage into dense K-long rows. */
    double* a = (double*)malloc(sizeof(double) * (size_t)(rows * (K ? K : 1)));
    double* b = (double*)malloc(sizeof(double) * (size_t)(N * (K ? K : 1)));
    if (!a || !b) { free(a); free(b); return -2; }
    for (int64_t m = 0; m < rows; ++m)
        for (int64_t k = 0; k < K; ++k) {
            int64_t mm = row0 + m;
            int64_t idx = (a_major == 'k') ? mm * lda + k : mm + k * lda;
            a[m * K + k] = element(A, in_type, idx);
        }
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            int64_t idx = (b_major == 'k') ? n * ldb + k : n + k * ldb;
            b[n * K + k] = element(B, in_type, idx);
        }

    if (nthreads < 1) nthreads = 1;
    if (nthreads > rows) nthreads = (int)rows;
    pthread_t* tid = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
    job_t* jobs = (job_t*)malloc(sizeof(job_t) * (size_t)nthreads);
    if (!tid || !jobs) { free(a); free(b); free(tid); free(jobs); return -2; }
    char* joined = (char*)calloc((size_t)nthreads, 1);   /* 1 = runs on its own thread */
    if (!joined) { free(a); free(b); free(tid); free(jobs); return -2; }
    for (int t = 0; t < nthreads; ++t) {
        jobs[t].N = N; jobs[t].K = K; jobs[t].A = a; jobs[t].B = b; jobs[t].C = C_out;
        jobs[t].r_begin = rows * t / nthreads;
        jobs[t].r_end = rows * (t + 1) / nthreads;
        if (t > 0 && pthread_create(&tid[t], NULL, run_rows, &jobs[t]) == 0) joined[t] = 1;
    }
    for (int t = 0; t < nthreads; ++t)     /* row block 0, and any that failed to start */
        if (!joined[t]) run_rows(&jobs[t]);
    for (int t = 0; t < nthreads; ++t)
        if (joined[t]) pthread_join(tid[t], NULL);
    free(joined);
    free(tid); free(jobs); free(a); free(b);
    return 0;
}

/* ---- rounding of the double result to the output type ---- */

/* binary32, round to nearest even: the C conversion in the default mode. */
float oracle_round_f32(double x) { return (float)x; }

/*
 * Round x to the nearest value with `p` significand bits and minimum normal
 * exponent `emin` (IEEE binary formats), ties to even, by scaling x to an
 * integer multiple of the quantum (2^(e-p+1), or the subnormal quantum
 * 2^(emin-p+1)) and applying rint() in the default rounding mode.
 */
static double round_to_format(double x, int p, int emin)
{
    if (x == 0.0 || isnan(x) || isinf(x)) return x;
    int e2;
    frexp(fabs(x), &e2);           /* |x| = f * 2^e2, f in [0.5, 1) */
    int e = e2 - 1;                /* |x| in [2^e, 2^(e+1)) */
    if (e < emin) e = emin;
    int q = e - p + 1;
    return ldexp(rint(ldexp(x, -q)), q);
}

/* bfloat16: 8 significand bits, exponent range of binary32. */
uint16_t oracle_round_bf16(double x)
{
    if (isnan(x)) return 0x7fc0;
    double r = round_to_format(x, 8, -126);
    /* largest finite bf16 is (2 - 2^-7) * 2^127; anything rounding above it is inf */
    double maxv = ldexp(255.0, 120);
    float f;
    if (fabs(r) > maxv) f = (r > 0) ? INFINITY : -INFINITY;
    else f = (float)r;             /* exact: r has at most 8 significand bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

/* binary16: 11 significand bits, emin = -14, largest finite 65504. */
uint16_t oracle_round_f16(double x)
{
    if (isnan(x)) return 0x7e00;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double r = fabs(round_to_format(x, 11, -14));
    if (r > 65504.0) return sign | 0x7c00;
    if (r == 0.0) return sign;
    int e2;
    double f = frexp(r, &e2);      /* r = f * 2^e2 */
    int e = e2 - 1;
    if (e < -14)                   /* subnormal: r = frac * 2^-24 */
        return sign | (uint16_t)(int64_t)ldexp(r, 24);
    int64_t sig = (int64_t)ldexp(f, 11);           /* 1024 .. 2047 */
    return sign | (uint16_t)(((e + 15) << 10) | (sig - 1024));
}

/* Bulk versions over n elements, for the comparison helpers. */
void oracle_round_f32_n(const double* x, float* y, int64_t n)
{ for (int64_t i = 0; i < n; ++i) y[i] = oracle_round_f32(x[i]); }
void oracle_round_bf16_n(const double* x, uint16_t* y, int64_t n)
{ for (int64_t i = 0; i < n; ++i) y[i] = oracle_round_bf16(x[i]); }
void oracle_round_f16_n(const double* x, uint16_t* y, int64_t n)
{ for (int64_t i = 0; i < n; ++i) y[i] = oracle_round_f16(x[i]); }
void oracle_decode_f16_n(const uint16_t* x, double* y, int64_t n)
{ for (int64_t i = 0; i < n; ++i) y[i] = oracle_decode_f16(x[i]); }
void oracle_decode_bf16_n(const uint16_t* x, double* y, int64_t n)
{ for (int64_t i = 0; i < n; ++i) y[i] = oracle_decode_bf16(x[i]); }
