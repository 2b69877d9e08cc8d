/*
 * oracle/sgemm_ref.c -- CPU oracle for single-precision row-major GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library
 * under register_lds_tiled_amd/) may include, link, load or call this file.
 * It is used by tests/, by the smoke check and by the CPU-baseline leg of the
 * benchmark, and by nothing else.  It shares no code, header, table or helper
 * with the HIP kernels.
 *
 * What it computes is the plain definition of the product that every page on
 * register/shared-memory tiling reaches, only faster:
 *
 *     C[i,j] = sum_{k=0}^{K-1} A[i,k] * B[k,j],   A: MxK, B: KxN, C: MxN,
 *     all row-major (element (r,c) of X at X[r*ldx + c]).
 *
 *   - the formula and the row-major indexing:
 *     "Micro Kernel 입문하기" (teach-meaning.tistory.com/1544), walkthrough
 *     section 2 (the accumulator c_ij is the sum over k of A[i,k]*B[k,j]) and
 *     sections 3-1 / 3-2 / 4 (A indexed row*K+col, B row*4+col, C row-major);
 *   - leading dimension of C: "누산 개념을 Grid-Block-Warp-Thread 계층에
 *     끼워넣기" (teach-meaning.tistory.com/1518), section 2 (the store uses
 *     row*ldc + col);
 *   - tiling, padding, double buffering and thread mapping change only the
 *     order in which the same products are summed, never the definition:
 *     "gemm_tiled_test" (teach-meaning.tistory.com/1542) sections 4-6, and
 *     "Register/Shared Memory Tiling" (ryotta.opik.net) "outer-product GEMM".
 *
 * Precision: every float input is widened to double (exact); each product of
 * two widened floats is exact in double (24+24 significant bits < 53); each
 * element's sum is accumulated in double in ascending k, starting from +0.0.
 * Build with -O2 -ffp-contract=off and no fast-math, so the compiler cannot
 * reassociate the sums.  OpenMP splits the work over rows of C only; no
 * element's arithmetic depends on the thread count.
 *
 * Second function: the single-thread 4x4 micro-GEMM of the first page in the
 * arithmetic its device performs -- fp32 accumulators, one fused multiply-add
 * per k in ascending k (C99 fmaf is correctly rounded).  The fused reading is
 * the one the tiled page writes out explicitly (fmaf in its section 5); the
 * printed output of the first page's example is reproduced to all digits by
 * it, and not by an unfused multiply-then-add.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

/* Number of OpenMP threads the oracle's parallel loops use. */
int oracle_num_threads(void) { return omp_get_max_threads(); }

/*
 * Full product in double: C[i*ldc + j] = sum_k A[i*lda + k] * B[k*ldb + j]
 * for 0 <= i < M, 0 <= j < N.  K == 0 gives the empty sum, 0.0.
 * The definition written out: for each (i, j), sum over k in ascending order.
 */
void sgemm_ref_f64(int M, int N, int K,
                   const float *A, long long lda,
                   const float *B, long long ldb,
                   double *C, long long ldc)
{
    #pragma omp parallel for schedule(dynamic, 1)
    for (int i = 0; i < M; ++i) {
        for (int j = 0; j < N; ++j) {
            double s = 0.0;
            for (int k = 0; k < K; ++k)
                s += (double)A[(size_t)i * lda + k] * (double)B[(size_t)k * ldb + j];
            C[(size_t)i * ldc + j] = s;
        }
    }
}

/*
 * Selected entries only: out[t] = C[rows[t], cols[t]] of the product above,
 * each computed by the same ascending-k double sum.  Lets a caller check
 * scattered outputs of a large product one by one.
 */
void sgemm_ref_f64_entries(int K,
                           const float *A, long long lda,
                           const float *B, long long ldb,
                           long long n, const long long *rows, const long long *cols,
                           double *out)
{
    #pragma omp parallel for schedule(static)
    for (long long t = 0; t < n; ++t) {
        const long long i = rows[t], j = cols[t];
        double s = 0.0;
        for (int k = 0; k < K; ++k)
            s += (double)A[(size_t)i * lda + k] * (double)B[(size_t)k * ldb + j];
        out[t] = s;
    }
}

/*
 * The first page's micro-GEMM in its own arithmetic: A is 4xK (row r at
 * A[r*K]), B is Kx4 (row k at B[k*4]), C is 4x4 row-major.  Each of the 16
 * accumulators starts at 0.0f and takes one fp32 fused multiply-add per k,
 * k ascending.
 */
void micro4x4_seq_fma_f32(int K, const float *A, const float *B, float *C)
{
    for (int r = 0; r < 4; ++r) {
        for (int j = 0; j < 4; ++j) {
            float c = 0.0f;
            for (int k = 0; k < K; ++k)
                c = fmaf(A[(size_t)r * K + k], B[(size_t)k * 4 + j], c);
            C[r * 4 + j] = c;
        }
    }
}

/*
 * The same product followed by the fused epilogue that the tiled page's
 * original kernel carries ("gemm_tiled_test", teach-meaning.tistory.com/1542,
 * opening paragraph: epilogue, bias and activation, removed from the test
 * kernel; the page does not define them further).  Reading taken: the BLAS
 * alpha/beta update, a bias added per output column, then an optional ReLU:
 *
 *     out[i,j] = act(alpha * S[i,j] + beta * Cin[i,j] + bias[j])
 *
 * with S[i,j] the ascending-k double sum above.  Cin is read only when
 * beta != 0 (so it may hold anything, NaN included, when beta == 0); bias
 * may be NULL (no bias).  act 0 is the identity; act 1 is ReLU taken as
 * (x < 0 ? 0 : x), which keeps NaN.  All in double.
 */
static double fused_epilogue(double s, long long i, long long j,
                             const float *Cin, long long ldc,
                             double alpha, double beta, const float *bias, int act)
{
    double v = alpha * s;
    if (beta != 0.0) v += beta * (double)Cin[(size_t)i * ldc + j];
    if (bias) v += (double)bias[j];
    if (act == 1 && v < 0.0) v = 0.0;
    return v;
}

/* Whole matrix; S is computed first into out, which must not overlap Cin. */
void sgemm_ex_ref_f64(int M, int N, int K,
                      const float *A, long long lda,
                      const float *B, long long ldb,
                      const float *Cin, long long ldc,
                      double alpha, double beta, const float *bias, int act,
                      double *out, long long ldo)
{
    sgemm_ref_f64(M, N, K, A, lda, B, ldb, out, ldo);
    #pragma omp parallel for schedule(static)
    for (int i = 0; i < M; ++i)
        for (int j = 0; j < N; ++j)
            out[(size_t)i * ldo + j] = fused_epilogue(out[(size_t)i * ldo + j], i, j, Cin, ldc,
                                                      alpha, beta, bias, act);
}

/* Selected entries out[t] = result[rows[t], cols[t]], for large products. */
void sgemm_ex_ref_f64_entries(int K,
                              const float *A, long long lda,
                              const float *B, long long ldb,
                              const float *Cin, long long ldc,
                              double alpha, double beta, const float *bias, int act,
                              long long n, const long long *rows, const long long *cols,
                              double *out)
{
    sgemm_ref_f64_entries(K, A, lda, B, ldb, n, rows, cols, out);
    for (long long t = 0; t < n; ++t)
        out[t] = fused_epilogue(out[t], rows[t], cols[t], Cin, ldc, alpha, beta, bias, act);
}

/*
 * 16-bit inputs.  The matrix-instruction path takes A and B in a 16-bit
 * floating-point format and accumulates in fp32 ("Register/Shared Memory
 * Tiling", ryotta.opik.net: advantages item 3 and related technologies tie
 * the tiling to tensor-core style instructions and half precision).  The
 * plain reading: the same sum as sgemm_ref_f64 over the values the 16-bit
 * inputs hold.  Each input is decoded to its exact value (both formats embed
 * in binary32, hence in double), then summed as above.
 *
 * fmt 1, bfloat16: the upper half of an IEEE binary32 -- the value is the
 *   binary32 whose bits are h followed by 16 zero bits.
 * fmt 2, IEEE binary16: sign bit, 5 exponent bits (bias 15), 10 fraction
 *   bits; exponent 0 is zero/subnormal (fraction * 2^-24), exponent 31 is
 *   Inf (fraction 0) or NaN.
 */
static float decode16(int fmt, uint16_t h)
{
    if (fmt == 1) {
        uint32_t u = (uint32_t)h << 16;
        float f;
        memcpy(&f, &u, sizeof f);
        return f;
    }
    const int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 0) v = ldexp((double)m, -24);
    else if (e == 31) v = m ? NAN : INFINITY;
    else v = ldexp((double)(m + 1024), e - 25);   /* (1 + m/2^10) * 2^(e-15) */
    return (float)(s ? -v : v);
}

/* out[i] = value of in[i] in format fmt (exact). */
void decode16_f32(int fmt, long long n, const uint16_t *in, float *out)
{
    for (long long i = 0; i < n; ++i) out[i] = decode16(fmt, in[i]);
}

/*
 * C[i*ldc + j] = sum_k a(i,k) * b(k,j) in double, ascending k, where a and b
 * are the decoded values of A[i*lda + k] and B[k*ldb + j].  Returns 0, or -1
 * if the scratch copies cannot be allocated.
 */
int gemm_lowp_ref_f64(int M, int N, int K,
                      const uint16_t *A, long long lda,
                      const uint16_t *B, long long ldb,
                      int fmt, double *C, long long ldc)
{
    float *a = malloc(sizeof(float) * ((size_t)M * K + 1));
    float *b = malloc(sizeof(float) * ((size_t)K * N + 1));
    if (!a || !b) { free(a); free(b); return -1; }
    for (int i = 0; i < M; ++i)
        for (int k = 0; k < K; ++k) a[(size_t)i * K + k] = decode16(fmt, A[(size_t)i * lda + k]);
    for (int k = 0; k < K; ++k)
        for (int j = 0; j < N; ++j) b[(size_t)k * N + j] = decode16(fmt, B[(size_t)k * ldb + j]);
    sgemm_ref_f64(M, N, K, a, K > 0 ? K : 1, b, N > 0 ? N : 1, C, ldc);
    free(a);
    free(b);
    return 0;
}
