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
// workgroup's 64 lanes copy chunks of A's columns and B's rows into LDS
// with coalesced loads, and lane 0 alone runs the page's loop over them.
// The chunks are double-buffered: the 64 lanes' loads of chunk c + 1 are in
// flight while lane 0 multiplies chunk c, so only the first chunk's latency
// shows, and the single thread's 16 v_fma_f32 per k bound the rest (K =
// 1024: 43.3 us, against 45.4 with one chunk loaded before the loop).
// Only the loads change; the arithmetic is the page's, in the page's order.
#include <cstdint>

#include "tiles.h"

namespace sgemm {
namespace {

constexpr int MICRO_KC = 256;   // k per LDS chunk, 4 per lane

__global__ __launch_bounds__(64)
void micro4x4_kernel(int K, const float* __restrict__ A, const float* __restrict__ B,
                     float* __restrict__ C) {
    __shared__ float4 Acol[2][MICRO_KC];   // Acol[b][k] = A[0..3][k0 + k]
    __shared__ float4 Brow[2][MICRO_KC];   // Brow[b][k] = B[k0 + k][0..3]
    const int lane = threadIdx.x;
    const bool bvec = (reinterpret_cast<uintptr_t>(B) & 15) == 0;
    float c[4][4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int j = 0; j < 4; ++j) c[r][j] = 0.f;

    // this lane's k of a chunk at k0: k0 + lane + 64 i, i < 4
    float4 ra[4], rb[4];
    auto load = [&](int k0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const long long kk = (long long)k0 + lane + 64 * i;
            if (kk >= K) continue;
            ra[i] = make_float4(A[kk], A[(long long)K + kk], A[2LL * K + kk], A[3LL * K + kk]);
            rb[i] = bvec ? *reinterpret_cast<const float4*>(B + 4 * kk)
                         : make_float4(B[4 * kk], B[4 * kk + 1], B[4 * kk + 2], B[4 * kk + 3]);
        }
    };
    auto store = [&](int buf, int k0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int k = lane + 64 * i;
            if ((long long)k0 + k >= K) continue;
            Acol[buf][k] = ra[i];
            Brow[buf][k] = rb[i];
        }
    };

    const int nch = (K + MICRO_KC - 1) / MICRO_KC;
    if (nch > 0) {
        load(0);
        store(0, 0);
    }
    __syncthreads();
    for (int ch = 0; ch < nch; ++ch) {
        const int cur = ch & 1, k0 = ch * MICRO_KC, kc = min(MICRO_KC, K - k0);
        const bool more = ch + 1 < nch;
        if (kLdsPoison && more) {   // buffer cur ^ 1, retired by the last barrier
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                lds_poison_f4(&Acol[cur ^ 1][lane + 64 * i]);
                lds_poison_f4(&Brow[cur ^ 1][lane + 64 * i]);
            }
        }
        if (more) load(k0 + MICRO_KC);
        if (lane == 0) {
#pragma unroll 8
            for (int k = 0; k < kc; ++k) {
                const float4 av = Acol[cur][k], bv = Brow[cur][k];
                const float a[4] = {av.x, av.y, av.z, av.w}, b[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int j = 0; j < 4; ++j) c[r][j] = __builtin_fmaf(a[r], b[j], c[r][j]);
            }
        }
        if (more) store(cur ^ 1, k0 + MICRO_KC);
        __syncthreads();   // chunk cur consumed, chunk cur ^ 1 in LDS
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
