/*
 * sgemm.h -- C ABI of the MI355X (gfx950) single-precision GEMM library
 * (libsgemm_mi355x.so), built from hand-written HIP kernels.
 *
 * Operation (every entry point below computes this, the 4x4 case of it, or,
 * for sgemm_f32_ex, this followed by a fused epilogue; gemm_bf16_f32 and
 * gemm_f16_f32 take A and B in 16-bit formats):
 *
 *     C[i,j] = sum_{k=0}^{K-1} A[i,k] * B[k,j]      0 <= i < M, 0 <= j < N
 *
 * with A (MxK), B (KxN) and C (MxN) single precision and row-major: element
 * (r,c) of X lives at X[r*ldx + c].  The sum is the accumulator that the
 * micro-GEMM page builds per output element ("Micro Kernel 입문하기",
 * teach-meaning.tistory.com/1544, walkthrough sections 2 and 3-1..4), and the
 * row*ld + col addressing of C is the store of "누산 개념을
 * Grid-Block-Warp-Thread 계층에 끼워넣기" (teach-meaning.tistory.com/1518),
 * section 2.  C is overwritten: the plain store of "gemm_tiled_test"
 * (teach-meaning.tistory.com/1542), section 6.  sgemm_f32_ex adds the fused
 * epilogue that page's opening paragraph says its original kernel carried
 * (alpha/beta, bias, activation); its reading is given at its declaration.
 *
 * How it is computed (results differ from the plain definition only in the
 * rounding order of the fp32 sums): one kernel launch covers all of C; each
 * workgroup owns one BM x BN block tile of C; the K axis is walked in BK-deep
 * slabs staged through LDS, double-buffered; within a workgroup each lane (or
 * each wave, on the matrix-core path) keeps a register tile of accumulators
 * updated by rank-1 outer products; the tile is stored once at the end.
 * (Page 2 section 1-2; "gemm_tiled_test" sections 1-6; "Register/Shared
 * Memory Tiling", ryotta.opik.net, sections on outer-product GEMM, tile
 * loading and double buffering.)
 *
 * Conventions shared by all entry points
 * --------------------------------------
 * - Pointers are DEVICE pointers (hipMalloc / torch CUDA tensors) owned by
 *   the caller.  The library allocates nothing and keeps no per-call state
 *   (it caches each device's compute-unit and XCD counts, read from the
 *   runtime on the first call that launches there); calls from several host
 *   threads are safe.
 * - Dimensions and leading dimensions are int; all address arithmetic inside
 *   the library is 64-bit.
 * - stream is a hipStream_t passed as void*; NULL means the null stream.
 *   Calls are stream-ordered and asynchronous: SGEMM_OK means the work was
 *   enqueued.  The caller synchronises before reading C.
 * - Every argument is validated before any HIP call; on a validation error
 *   nothing is launched and C is untouched.
 * - M == 0 or N == 0: nothing to do, returns SGEMM_OK without a launch.
 *   K == 0: A and B may be NULL; sgemm_f32 and sgemm_f32_path set
 *   C[0:M, 0:N] to 0 (the empty sum).
 * - C must not overlap A or B (the pages' kernels take all three pointers
 *   __restrict__); A and B may overlap each other.
 * - Result: within the fp32 rounding of some summation order of the exact
 *   products; integer-valued inputs whose partial sums stay below 2^24 in
 *   magnitude give the exact result on every path.
 */
#ifndef REGISTER_LDS_TILED_SGEMM_H
#define REGISTER_LDS_TILED_SGEMM_H

#ifdef __cplusplus
extern "C" {
#endif

/* Symbols of this ABI are the only ones the library exports. */
#ifndef SGEMM_API
#define SGEMM_API __attribute__((visibility("default")))
#endif

/* Return codes. */
#define SGEMM_OK             0
#define SGEMM_EINVAL_DIM    -1  /* M, N or K negative; micro-GEMM K < 0; C
                                   so large that one workgroup per 64 x 64 tile
                                   (256 threads each) would pass the 2^32 - 1
                                   threads of one launch; or a matrix whose
                                   byte extent from its pointer would pass the
                                   end of the address space                    */
#define SGEMM_EINVAL_LD     -2  /* lda < max(1,K), ldb < max(1,N) or ldc < max(1,N) */
#define SGEMM_EINVAL_PTR    -3  /* NULL pointer for a matrix with elements      */
#define SGEMM_EALIAS        -4  /* C's address range overlaps A's, B's or bias's */
#define SGEMM_EHIP          -5  /* the HIP runtime reported an error on launch  */
#define SGEMM_EINVAL_PATH   -6  /* unknown path selector                        */
#define SGEMM_EINVAL_ACT    -7  /* unknown activation selector (sgemm_f32_ex)   */

/* Activation selectors for sgemm_f32_ex. */
#define SGEMM_ACT_NONE        0 /* identity                                     */
#define SGEMM_ACT_RELU        1 /* x < 0 ? 0 : x  (NaN passes through)          */

/* Path selectors for sgemm_f32_path. */
#define SGEMM_PATH_AUTO       0 /* what sgemm_f32 uses: the matrix-core path;
                                   for A of at most 16 rows kernels that
                                   stream B once (9 to 16 aligned rows on the
                                   matrix cores, else on the vector ALU), and
                                   for B of at most 16 columns (A of more
                                   than 16 rows) vector-ALU kernels that
                                   stream A once */
#define SGEMM_PATH_VALU       1 /* per-lane TM x TN v_fma_f32 micro-kernel      */
#define SGEMM_PATH_MFMA       2 /* fp32 MFMA wave tiles (16x16x4 in the large
                                   wave-tile kernels, 32x32x2 in the others),
                                   for every shape                             */
#define SGEMM_PATH_VALU_PAGE  3 /* VALU path at the tiled page's own geometry:
                                   BM=BN=64, BK=16, 64 threads, 16x4 per thread,
                                   single-buffered ("gemm_tiled_test" section 7) */

/*
 * C = A.B, row-major, fp32, on the path the library picks for the shape.
 * A: M x K at A[i*lda + k]; B: K x N at B[k*ldb + j]; C: M x N at
 * C[i*ldc + j].  Returns SGEMM_OK or a negative code above.
 */
SGEMM_API int sgemm_f32(int M, int N, int K,
              const float *A, int lda,
              const float *B, int ldb,
              float *C, int ldc,
              void *stream);

/*
 * Same operation and contract as sgemm_f32 on an explicit path (one of
 * SGEMM_PATH_*), for tests and measurements that compare the paths.
 */
SGEMM_API int sgemm_f32_path(int M, int N, int K,
                   const float *A, int lda,
                   const float *B, int ldb,
                   float *C, int ldc,
                   void *stream, int path);

/*
 * Same operation and contract as sgemm_f32 on the VALU path at one of its
 * built tile configurations (tile = 0 .. sgemm_valu_tile_count() - 1): the
 * block tile BM x BN x BK, the wave tile WM x WN each wave of the block owns
 * (the warp tile of "누산 개념을 Grid-Block-Warp-Thread 계층에 끼워넣기",
 * teach-meaning.tistory.com/1518, section 2(2)), and the TM x TN register
 * tile of each lane (the thread tile, section 2(3); the MR x NR of "Micro
 * Kernel 입문하기", teach-meaning.tistory.com/1544, section 4, whose planned
 * comparison of register tiles this entry point serves).  Every
 * configuration sums each output over k in ascending order with one fused
 * multiply-add per k, so all of them return the same bits.  For tests and
 * measurements; SGEMM_PATH_VALU picks among the same configurations by
 * shape.  A tile outside the range -> SGEMM_EINVAL_PATH.
 */
SGEMM_API int sgemm_f32_valu_tile(int M, int N, int K,
                        const float *A, int lda,
                        const float *B, int ldb,
                        float *C, int ldc,
                        void *stream, int tile);

/* Number of VALU tile configurations sgemm_f32_valu_tile accepts. */
SGEMM_API int sgemm_valu_tile_count(void);

/*
 * Static text describing VALU tile configuration `tile` (block, waves, wave
 * tile, lanes, lane tile, LDS stages), or NULL outside 0 .. count - 1.
 */
SGEMM_API const char *sgemm_valu_tile_name(int tile);

/*
 * Fused form, on the default path's kernels (the same choice as sgemm_f32):
 *
 *     C[i,j] = act(alpha * sum_k A[i,k] * B[k,j] + beta * C[i,j] + bias[j])
 *
 * "gemm_tiled_test" (teach-meaning.tistory.com/1542), opening paragraph:
 * the page's test kernel is its original kernel with the epilogue, bias and
 * activation taken out, and the page leaves them undefined.  Reading taken
 * here: the BLAS alpha/beta update of C in place, one bias value per output
 * column, then act = SGEMM_ACT_NONE or SGEMM_ACT_RELU.  Each output is
 * computed once, in fp32, right after its dot product leaves the
 * accumulators, so the epilogue costs no extra pass over C.
 * - C is read only when beta != 0 (when beta == 0 it may hold anything,
 *   NaN included); it is then read and written in place, element by element.
 * - bias: NULL for none, else a device array of N floats that must not
 *   overlap C (SGEMM_EALIAS); it may overlap A or B.
 * - alpha multiplies the accumulated sum as is: alpha == 0 does not skip
 *   the product (NaN or Inf in A.B still propagates).
 * - K == 0: C = act(beta * C + bias) (the sum is the empty sum, 0).
 * - alpha == 1, beta == 0, bias == NULL, act == SGEMM_ACT_NONE runs exactly
 *   the kernel sgemm_f32 runs, the skinny-shape kernels included.
 * Other arguments, conventions and return codes as sgemm_f32; an act outside
 * SGEMM_ACT_* -> SGEMM_EINVAL_ACT.
 */
SGEMM_API int sgemm_f32_ex(int M, int N, int K,
                 const float *A, int lda,
                 const float *B, int ldb,
                 float *C, int ldc,
                 float alpha, float beta, const float *bias, int act,
                 void *stream);

/*
 * C = A.B with 16-bit floating-point inputs and fp32 accumulation and output,
 * on the matrix cores (v_mfma_f32_32x32x16_bf16 / _f16).  The pages tie the
 * register/LDS tiling to matrix instructions and half-precision inputs
 * ("Register/Shared Memory Tiling", ryotta.opik.net: advantages item 3,
 * related technologies); the reading taken is the plain one: the same sum as
 * above over the values the 16-bit inputs hold, accumulated in fp32.
 * - gemm_bf16_f32: A and B hold bfloat16 values (the upper 16 bits of an
 *   IEEE binary32); gemm_f16_f32: IEEE binary16.  Passed as raw 16-bit
 *   storage (const void *, two bytes per element); lda and ldb count
 *   elements.  C is fp32 and overwritten, as for sgemm_f32.
 * - Every product of two 16-bit values is exact in fp32, so the result is
 *   within the fp32 rounding of some summation order of the exact sum of the
 *   stored inputs; integer-valued inputs with partial sums below 2^24 give
 *   the exact result.
 * - Rows of A and B that are 16-byte aligned (base 16-byte aligned, lda and
 *   ldb multiples of 8) take the fast loader; any other layout is accepted
 *   and runs a slower one.
 * Conventions and return codes as sgemm_f32 (overlap checks use the 16-bit
 * extents of A and B).
 */
SGEMM_API int gemm_bf16_f32(int M, int N, int K,
                  const void *A, int lda,
                  const void *B, int ldb,
                  float *C, int ldc,
                  void *stream);
SGEMM_API int gemm_f16_f32(int M, int N, int K,
                 const void *A, int lda,
                 const void *B, int ldb,
                 float *C, int ldc,
                 void *stream);

/*
 * The micro-GEMM of "Micro Kernel 입문하기" (teach-meaning.tistory.com/1544),
 * section 2: one GPU thread holds the whole 4x4 tile of C in 16 registers and
 * walks k = 0..K-1 in order, loading column k of A (4 values) and row k of B
 * (4 values) and doing 16 fused multiply-adds (the fmaf form of the tiled
 * page's section 5).  The launch is one wave: its 64 lanes first stage
 * chunks of A's columns and B's rows in LDS with coalesced loads, and the
 * thread reads its operands from there.  Layouts are the page's: A is 4 x K with leading
 * dimension K (A[r*K + k]), B is K x 4 with leading dimension 4 (B[k*4 + j]),
 * C is 4 x 4 row-major (C[r*4 + j]).  Each output is the sequential fp32
 * fused sum in ascending k, so results are reproducible bit for bit.
 * K == 0 stores zeros.  K < 0 -> SGEMM_EINVAL_DIM; NULL A/B (K > 0) or NULL C
 * -> SGEMM_EINVAL_PTR; C overlapping A or B -> SGEMM_EALIAS.
 */
SGEMM_API int sgemm_micro4x4_f32(int K, const float *A, const float *B, float *C, void *stream);

/* Static description of a return code (never NULL). */
SGEMM_API const char *sgemm_status_string(int status);

/*
 * Detail of the last SGEMM_EHIP on the calling host thread (the HIP error
 * name and message), or "" if there was none.  Thread-local; valid until the
 * thread's next failing call.
 */
SGEMM_API const char *sgemm_last_error(void);

/* Version of this ABI; bumped when a signature or contract changes. */
SGEMM_API int sgemm_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* REGISTER_LDS_TILED_SGEMM_H */
