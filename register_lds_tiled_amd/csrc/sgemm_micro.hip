// sgemm_micro.hip -- the one-thread 4x4 micro-GEMM ("Micro Kernel 입문하기",
// teach-meaning.tistory.com/1544, sections 1-2 and the walkthrough).
//
// One thread keeps the whole 4x4 tile of C in 16 registers.  For each k in
// ascending order it loads column k of A (4 values, rows K apart) and row k
// of B (4 contiguous values) and applies the 4x4 outer product with 16 fused
// multiply-adds; C is written once at the end.  Each output is therefore the
// sequential fp32 fused sum over k, which makes the result reproducible bit
// for bit.  The k loop is unrolled by 8 (the page's unroll knob, section 3);
// unrolling moves loads earlier but leaves every accumulator's chain of
// fused multiply-adds in the same order.
#include "tiles.h"

namespace sgemm {
namespace {

__global__ __launch_bounds__(64)
void micro4x4_kernel(int K, const float* __restrict__ A, const float* __restrict__ B,
                     float* __restrict__ C) {
    if (threadIdx.x != 0) return;
    float c[4][4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int j = 0; j < 4; ++j) c[r][j] = 0.f;

#pragma unroll 8
    for (int k = 0; k < K; ++k) {
        float a[4], b[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) a[r] = A[(long long)r * K + k];
#pragma unroll
        for (int j = 0; j < 4; ++j) b[j] = B[(long long)k * 4 + j];
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int j = 0; j < 4; ++j) c[r][j] = __builtin_fmaf(a[r], b[j], c[r][j]);
    }

#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int j = 0; j < 4; ++j) C[r * 4 + j] = c[r][j];
}

}  // namespace

hipError_t launch_micro4x4(int K, const float* A, const float* B, float* C,
                           hipStream_t stream) {
    // One workgroup of one thread, as the page launches it.
    hipLaunchKernelGGL(micro4x4_kernel, dim3(1), dim3(1), 0, stream, K, A, B, C);
    return hipGetLastError();
}

}  // namespace sgemm
