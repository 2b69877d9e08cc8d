/*
 * Drives every function of oracle/sgemm_ref.c over small and degenerate
 * shapes with heap buffers of exactly the size each matrix spans, so that a
 * read or write one element out of range, or undefined arithmetic, stops the
 * AddressSanitizer / UndefinedBehaviorSanitizer build.  A few results are
 * checked too (identity products, K = 0, the decoders' named values).
 * Exit status 0 on success.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

void sgemm_ref_f64(int M, int N, int K, const float *A, long long lda, const float *B,
                   long long ldb, double *C, long long ldc);
void sgemm_ref_f64_entries(int K, const float *A, long long lda, const float *B, long long ldb,
                           long long n, const long long *rows, const long long *cols, double *out);
void micro4x4_seq_fma_f32(int K, const float *A, const float *B, float *C);
void sgemm_ex_ref_f64(int M, int N, int K, const float *A, long long lda, const float *B,
                      long long ldb, const float *Cin, long long ldc, double alpha, double beta,
                      const float *bias, int act, double *out, long long ldo);
void sgemm_ex_ref_f64_entries(int K, const float *A, long long lda, const float *B, long long ldb,
                              const float *Cin, long long ldc, double alpha, double beta,
                              const float *bias, int act, long long n, const long long *rows,
                              const long long *cols, double *out);
void decode16_f32(int fmt, long long n, const uint16_t *in, float *out);
int gemm_lowp_ref_f64(int M, int N, int K, const uint16_t *A, long long lda, const uint16_t *B,
                      long long ldb, int fmt, double *C, long long ldc);

static int failures = 0;
#define CHECK(c)                                                        \
    do {                                                                \
        if (!(c)) {                                                     \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
            ++failures;                                                 \
        }                                                               \
    } while (0)

/* elements spanned by a rows x cols matrix with leading dimension ld */
static size_t span(int rows, int cols, long long ld) {
    return rows && cols ? (size_t)(rows - 1) * (size_t)ld + (size_t)cols : 0;
}
static void *xmalloc(size_t bytes) { return malloc(bytes ? bytes : 1); }

static void one_shape(int M, int N, int K, int pa, int pb, int pc) {
    const long long lda = K + pa, ldb = N + pb, ldc = N + pc;
    float *A = xmalloc(span(M, K, lda) * sizeof(float));
    float *B = xmalloc(span(K, N, ldb) * sizeof(float));
    float *Cin = xmalloc(span(M, N, ldc) * sizeof(float));
    float *bias = xmalloc((size_t)N * sizeof(float));
    double *C = xmalloc(span(M, N, ldc) * sizeof(double));
    for (size_t i = 0; i < span(M, K, lda); ++i) A[i] = (float)((int)(i % 7) - 3);
    for (size_t i = 0; i < span(K, N, ldb); ++i) B[i] = (float)((int)(i % 5) - 2);
    for (size_t i = 0; i < span(M, N, ldc); ++i) Cin[i] = (float)((int)(i % 3) - 1);
    for (int j = 0; j < N; ++j) bias[j] = (float)j;
    sgemm_ref_f64(M, N, K, A, lda, B, ldb, C, ldc);
    if (K == 0)
        for (int i = 0; i < M; ++i)
            for (int j = 0; j < N; ++j) CHECK(C[(size_t)i * ldc + j] == 0.0);
    sgemm_ex_ref_f64(M, N, K, A, lda, B, ldb, Cin, ldc, 2.0, -1.0, bias, 1, C, ldc);
    sgemm_ex_ref_f64(M, N, K, A, lda, B, ldb, NULL, ldc, 0.5, 0.0, NULL, 0, C, ldc);
    if (M && N) {
        long long rows[4] = {0, M - 1, 0, M - 1}, cols[4] = {0, N - 1, N - 1, 0};
        double e[4];
        sgemm_ref_f64_entries(K, A, lda, B, ldb, 4, rows, cols, e);
        sgemm_ex_ref_f64_entries(K, A, lda, B, ldb, Cin, ldc, 1.5, 2.0, bias, 1, 4, rows, cols, e);
        sgemm_ex_ref_f64_entries(K, A, lda, B, ldb, NULL, ldc, 1.5, 0.0, NULL, 0, 4, rows, cols, e);
    }
    uint16_t *A16 = xmalloc(span(M, K, lda) * sizeof(uint16_t));
    uint16_t *B16 = xmalloc(span(K, N, ldb) * sizeof(uint16_t));
    for (size_t i = 0; i < span(M, K, lda); ++i) A16[i] = (uint16_t)(0x3f80 + (i % 9));
    for (size_t i = 0; i < span(K, N, ldb); ++i) B16[i] = (uint16_t)(0x3c00 + (i % 11));
    CHECK(gemm_lowp_ref_f64(M, N, K, A16, lda, B16, ldb, 1, C, ldc) == 0);
    CHECK(gemm_lowp_ref_f64(M, N, K, A16, lda, B16, ldb, 2, C, ldc) == 0);
    free(A); free(B); free(Cin); free(bias); free(C); free(A16); free(B16);
}

int main(void) {
    const int dims[] = {0, 1, 2, 3, 5, 8, 17};
    const int nd = (int)(sizeof dims / sizeof dims[0]);
    for (int a = 0; a < nd; ++a)
        for (int b = 0; b < nd; ++b)
            for (int c = 0; c < nd; ++c)
                for (int pad = 0; pad < 2; ++pad) {
                    const int M = dims[a], N = dims[b], K = dims[c];
                    if ((N == 0 || K == 0) && pad == 0) {
                        one_shape(M, N, K, 1, 1, 1);   /* ld >= 1 */
                        continue;
                    }
                    one_shape(M, N, K, pad, 3 * pad, 2 * pad);
                }
    /* identity: A (5x5) times I gives A exactly */
    {
        float A[25], I[25];
        double C[25];
        for (int i = 0; i < 25; ++i) { A[i] = (float)(i * 0.37 - 4.0); I[i] = (i % 6 == 0) ? 1.f : 0.f; }
        sgemm_ref_f64(5, 5, 5, A, 5, I, 5, C, 5);
        for (int i = 0; i < 25; ++i) CHECK(C[i] == (double)A[i]);
    }
    /* the micro-GEMM over exact-size A (4 x K) and B (K x 4) */
    for (int K = 0; K <= 1024; K = K ? 2 * K + 1 : 1) {
        float *A = xmalloc((size_t)4 * K * sizeof(float)), *B = xmalloc((size_t)K * 4 * sizeof(float));
        float C[16];
        for (int i = 0; i < 4 * K; ++i) { A[i] = (float)(i % 7) * 0.1f; B[i] = (float)(i % 5) * 0.2f; }
        micro4x4_seq_fma_f32(K, A, B, C);
        if (K == 0)
            for (int i = 0; i < 16; ++i) CHECK(C[i] == 0.f);
        free(A); free(B);
    }
    /* both decoders over every 16-bit pattern, into an exact-size buffer */
    {
        uint16_t *in = xmalloc(65536 * sizeof(uint16_t));
        float *out = xmalloc(65536 * sizeof(float));
        for (int i = 0; i < 65536; ++i) in[i] = (uint16_t)i;
        decode16_f32(1, 65536, in, out);
        CHECK(out[0x3f80] == 1.0f && out[0xc000] == -2.0f && isnan(out[0x7fc0]));
        decode16_f32(2, 65536, in, out);
        CHECK(out[0x3c00] == 1.0f && out[0x7bff] == 65504.0f && out[0x0001] == ldexpf(1.f, -24));
        free(in); free(out);
    }
    if (failures) fprintf(stderr, "%d checks failed\n", failures);
    return failures ? 1 : 0;
}
