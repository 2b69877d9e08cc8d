/*
 * Drives the argument validation of libsgemm's C ABI (include/sgemm.h) in a
 * host build with AddressSanitizer and UndefinedBehaviorSanitizer: negative,
 * zero and extreme dimensions and leading dimensions, NULL pointers, every
 * overlap case and pointers near the top of the address space.  The
 * pointers are never dereferenced (validation is arithmetic on them); no
 * call here reaches a GPU.  Checks the documented return codes; exit status
 * 0 on success.
 */
#include <limits.h>
#include <stdint.h>
#include <stdio.h>

#include "sgemm.h"

static int failures = 0;
#define EXPECT(call, code)                                                          \
    do {                                                                            \
        const int st_ = (call);                                                     \
        if (st_ != (code)) {                                                        \
            fprintf(stderr, "line %d: %s returned %d, expected %d\n", __LINE__, #call, \
                    st_, (code));                                                   \
            ++failures;                                                             \
        }                                                                           \
    } while (0)

int main(void) {
    float *A = (float *)(uintptr_t)0x100000000ull, *B = (float *)(uintptr_t)0x200000000ull;
    float *C = (float *)(uintptr_t)0x300000000ull;
    float *top = (float *)(uintptr_t)(UINTPTR_MAX - 63);
    const int big = INT_MAX;
    for (int path = 0; path <= 3; ++path) {
        EXPECT(sgemm_f32_path(-1, 4, 4, A, 4, B, 4, C, 4, 0, path), SGEMM_EINVAL_DIM);
        EXPECT(sgemm_f32_path(4, -1, 4, A, 4, B, 4, C, 4, 0, path), SGEMM_EINVAL_DIM);
        EXPECT(sgemm_f32_path(4, 4, -1, A, 4, B, 4, C, 4, 0, path), SGEMM_EINVAL_DIM);
        EXPECT(sgemm_f32_path(4, 4, 8, A, 7, B, 4, C, 4, 0, path), SGEMM_EINVAL_LD);
        EXPECT(sgemm_f32_path(4, 8, 4, A, 4, B, 7, C, 8, 0, path), SGEMM_EINVAL_LD);
        EXPECT(sgemm_f32_path(4, 8, 4, A, 4, B, 8, C, 7, 0, path), SGEMM_EINVAL_LD);
        EXPECT(sgemm_f32_path(4, 4, 4, 0, 4, B, 4, C, 4, 0, path), SGEMM_EINVAL_PTR);
        EXPECT(sgemm_f32_path(4, 4, 4, A, 4, B, 4, 0, 4, 0, path), SGEMM_EINVAL_PTR);
        EXPECT(sgemm_f32_path(4, 4, 4, A, 4, B, 4, A + 15, 4, 0, path), SGEMM_EALIAS);
        EXPECT(sgemm_f32_path(4, 4, 4, A, 4, B, 4, B - 15, 4, 0, path), SGEMM_EALIAS);
        EXPECT(sgemm_f32_path(0, 4, 4, 0, 4, 0, 4, 0, 4, 0, path), SGEMM_OK);
        EXPECT(sgemm_f32_path(4, 0, 4, 0, 4, 0, 1, 0, 1, 0, path), SGEMM_OK);
        /* extreme sizes: refused by the grid limit or the address space, no overflow */
        EXPECT(sgemm_f32_path(big, big, big, A, big, B, big, C, big, 0, path), SGEMM_EINVAL_DIM);
        EXPECT(sgemm_f32_path(1 << 30, 64, big, A, big, B, big, C, big, 0, path), SGEMM_EINVAL_DIM);
        EXPECT(sgemm_f32_path(4, 4, 4, A, 4, B, 4, top, 4, 0, path), SGEMM_EINVAL_DIM);
        EXPECT(sgemm_f32_path(4, 4, 4, top, 4, B, 4, C, 4, 0, path), SGEMM_EINVAL_DIM);
    }
    EXPECT(sgemm_f32_path(4, 4, 4, A, 4, B, 4, C, 4, 0, 4), SGEMM_EINVAL_PATH);
    EXPECT(sgemm_f32_path(4, 4, 4, A, 4, B, 4, C, 4, 0, -1), SGEMM_EINVAL_PATH);
    EXPECT(sgemm_f32(-1, 4, 4, A, 4, B, 4, C, 4, 0), SGEMM_EINVAL_DIM);
    /* fused form */
    EXPECT(sgemm_f32_ex(4, 4, 4, A, 4, B, 4, C, 4, 1.f, 0.f, 0, 2, 0), SGEMM_EINVAL_ACT);
    EXPECT(sgemm_f32_ex(4, 4, 4, A, 4, B, 4, C, 4, 1.f, 0.f, C + 3, 1, 0), SGEMM_EALIAS);
    EXPECT(sgemm_f32_ex(4, 4, 4, A, 4, B, 4, C, 4, 1.f, 0.f, C - 3, 1, 0), SGEMM_EALIAS);
    EXPECT(sgemm_f32_ex(4, big, 4, A, 4, B, big, C, big, 1.f, 0.f, top, 1, 0), SGEMM_EINVAL_DIM);
    EXPECT(sgemm_f32_ex(0, 4, 4, 0, 4, 0, 4, 0, 4, 2.f, 1.f, C, 1, 0), SGEMM_OK);
    /* 16-bit inputs: extents of 2-byte elements */
    EXPECT(gemm_bf16_f32(4, 4, 4, A, 4, B, 4, (float *)((char *)A + 28), 4, 0), SGEMM_EALIAS);
    /* C right after A's 32 bytes: no overlap (the call then goes past validation) */
    if (gemm_f16_f32(4, 4, 4, A, 4, B, 4, (float *)((char *)A + 32), 4, 0) == SGEMM_EALIAS)
        ++failures;
    EXPECT(gemm_f16_f32(big, big, big, A, big, B, big, C, big, 0), SGEMM_EINVAL_DIM);
    /* VALU tiles */
    EXPECT(sgemm_f32_valu_tile(4, 4, 4, A, 4, B, 4, C, 4, 0, -1), SGEMM_EINVAL_PATH);
    EXPECT(sgemm_f32_valu_tile(4, 4, 4, A, 4, B, 4, C, 4, 0, sgemm_valu_tile_count()),
           SGEMM_EINVAL_PATH);
    EXPECT(sgemm_f32_valu_tile(big, big, big, A, big, B, big, C, big, 0, 0), SGEMM_EINVAL_DIM);
    if (sgemm_valu_tile_name(-1) != 0 || sgemm_valu_tile_name(0) == 0) ++failures;
    /* micro-GEMM */
    EXPECT(sgemm_micro4x4_f32(-1, A, B, C, 0), SGEMM_EINVAL_DIM);
    EXPECT(sgemm_micro4x4_f32(8, 0, B, C, 0), SGEMM_EINVAL_PTR);
    EXPECT(sgemm_micro4x4_f32(8, A, B, A + 4, 0), SGEMM_EALIAS);
    EXPECT(sgemm_micro4x4_f32(big, A, B, top, 0), SGEMM_EINVAL_DIM);
    EXPECT(sgemm_micro4x4_f32(big, top, B, C, 0), SGEMM_EINVAL_DIM);
    /* strings */
    for (int code = -8; code <= 1; ++code)
        if (sgemm_status_string(code) == 0) ++failures;
    if (sgemm_abi_version() != 4) ++failures;
    if (failures) fprintf(stderr, "%d checks failed\n", failures);
    return failures ? 1 : 0;
}
