// sgemm_micro.hip -- the one-thread 4x4 micro-GEMM ("Micro Kernel 입문하기",
// teach-meaning.tistory.com/1544, sections 1-2 and the walkthrough).
//
// One thread keeps the whole 4x4 tile of C in 16 registers.  For each k in
// ascending order it takes column k of A (4 values, rows K apart) and row k
// of B (4 contiguous values) and applies the 4x4 outer product with 16 fused
// multiply-adds; C is written once at the end.  Each output is therefore the
// sequential fp32 fused sum over k, which makes the result reproducible bit
// for bit.  The k loop is unrolled by 8 (the page's unroll knob, section 3);
// unrolling moves loads earlier but leaves every accumulator's chain of
// fused multiply-adds in the same order.
//
// gfx950 choice (not on the page): the thread's operands reach it through
// LDS.  Read straight from global memory, every step of the single thread
// waited a full memory latency (about 58 us for K = 1024); here the
// workgroup's 64 lanes first copy a chunk of A's columns and B's rows into
// LDS with coalesced loads, then lane 0 alone runs the page's loop over it.
// Only the loads change; the arithmetic is the page's, in the page's order.
#include <cstdint>

#include "tiles.h"

namespace sgemm {
namespace {

constexpr int MICRO_KC = 1024;   // k per LDS chunk: 2 x 16 KB

__global__ __launch_bounds__(64)
void micro4x4_kernel(int K, const float* __restrict__ A, const float* __restrict__ B,
                     float* __restrict__ C) {
    __shared__ float4 Acol[MICRO_KC];   // Acol[k] = A[0..3][k0 + k]
    __shared__ float4 Brow[MICRO_KC];   // Brow[k] = B[k0 + k][0..3]
    const int lane = threadIdx.x;
    const bool bvec = (reinterpret_cast<uintptr_t>(B) & 15) == 0;
    float c[4][4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int j = 0; j < 4; ++j) c[r][j] = 0.f;

    for (int k0 = 0; k0 < K; k0 += MICRO_KC) {
        const int kc = min(MICRO_KC, K - k0);
        __syncthreads();   // the previous chunk has been consumed
        if constexpr (kLdsPoison) {
            for (int k = lane; k < kc; k += 64) {
                lds_poison_f4(&Acol[k]);
                lds_poison_f4(&Brow[k]);
            }
        }
#pragma unroll 4
        for (int k = lane; k < kc; k += 64) {
            const long long kk = (long long)k0 + k;
            Acol[k] = make_float4(A[kk], A[(long long)K + kk], A[2LL * K + kk], A[3LL * K + kk]);
            if (bvec) {
                Brow[k] = *reinterpret_cast<const float4*>(B + 4 * kk);
            } else {
                Brow[k] = make_float4(B[4 * kk], B[4 * kk + 1], B[4 * kk + 2], B[4 * kk + 3]);
            }
        }
        __syncthreads();
        if (lane == 0) {
#pragma unroll 8
            for (int k = 0; k < kc; ++k) {
                const float4 av = Acol[k], bv = Brow[k];
                const float a[4] = {av.x, av.y, av.z, av.w}, b[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int j = 0; j < 4; ++j) c[r][j] = __builtin_fmaf(a[r], b[j], c[r][j]);
            }
        }
    }

    if (lane == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int j = 0; j < 4; ++j) C[r * 4 + j] = c[r][j];
    }
}

}  // namespace

hipError_t launch_micro4x4(int K, const float* A, const float* B, float* C,
                           hipStream_t stream) {
    // One workgroup of one wave: its lanes stage the operands, lane 0
    // computes the whole 4x4 tile, as the page's single thread does.
    hipLaunchKernelGGL(micro4x4_kernel, dim3(1), dim3(64), 0, stream, K, A, B, C);
    return hipGetLastError();
}

}  // namespace sgemm
