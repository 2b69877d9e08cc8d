// sgemm_skinny.hip -- fp32 C = A.B when A has at most 16 rows or B at most
// 16 columns.
//
// The same sum as the tiled kernels ("Register/Shared Memory Tiling",
// ryotta.opik.net: the output tile of a block held in registers across the
// K loop), shaped for a product that is bound by reading B: with M <= 16,
// 2MNK flops fall on 4KN bytes of B, at most 8 flops per byte, far below
// the 157.3 TFLOP/s : 8 TB/s balance of the chip.  A tile of 64 columns
// times all of A's rows would waste most of a matrix-core tile, so this
// kernel stays on the vector ALU and is built to stream B once at HBM rate:
//  * a workgroup owns 64 columns of C; its 16 waves split K into 16
//    contiguous slices, and each lane accumulates its column of C for the
//    rows of A over its wave's slice;
//  * for one k a wave reads 64 consecutive floats of B's row k (256 bytes,
//    coalesced); up to 8 rows, A[i][k] (the same for the whole wave) comes
//    by scalar loads, the k loop unrolled so that several rows of B are in
//    flight per wave (as many as the scalar registers for A allow); from 9
//    rows on A comes through LDS (skinny_m16_kernel);
//  * the 16 partial sums of each output are added through LDS in wave
//    order, so the result does not depend on timing.
#include "tiles.h"

namespace sgemm {
namespace {

constexpr int SK_WAVES = 16;   // waves per workgroup, one slice of K each
constexpr int SK_COLS = 64;    // columns of C per workgroup

// Up to 8 rows (MB = 1, 2, 4, 8; 9 to 16 rows take skinny_m16_kernel).  A
// wave takes at most 8 rows of A (RW); were there more, RH waves would share
// a slice of K.  Rows of B in flight per wave: the unrolled step holds
// RW x UNROLL values of A in scalar registers, kept within 64 of them.
template <int MB>
struct SkCfg {
    static constexpr int RW = MB < 8 ? MB : 8;          // rows of A per wave
    static constexpr int RH = MB / RW;                  // waves per slice of K
    static constexpr int SLICES = SK_WAVES / RH;        // slices of K
    static constexpr int UNROLL = 64 / RW;
};

template <int MB>
__global__ __launch_bounds__(64 * SK_WAVES)
void skinny_m_kernel(GemmArgs p) {
    using Cfg = SkCfg<MB>;
    constexpr int RW = Cfg::RW, RH = Cfg::RH, SLICES = Cfg::SLICES, UNROLL = Cfg::UNROLL;
    __shared__ float part[SLICES][MB][SK_COLS];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int slice = wave / RH, r0 = (wave % RH) * RW;
    const long long col = (long long)blockIdx.x * SK_COLS + lane;
    const bool in = col < p.N;
    // a column past N reads column 0 of B (always there) and is not stored
    const float* __restrict__ bcol = p.B + (in ? col : 0);
    const long long kper = ((long long)p.K + SLICES - 1) / SLICES;
    const int k0 = (int)min((long long)p.K, slice * kper), k1 = (int)min((long long)p.K, k0 + kper);
    // rows past M repeat row M - 1 (their sums are not stored)
    const float* __restrict__ arow[RW];
#pragma unroll
    for (int i = 0; i < RW; ++i) arow[i] = p.A + (long long)min(r0 + i, p.M - 1) * p.lda;

    float acc[RW];
#pragma unroll
    for (int i = 0; i < RW; ++i) acc[i] = 0.f;
    int k = k0;
    for (; k + UNROLL <= k1; k += UNROLL) {
        float b[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) b[u] = bcol[(long long)(k + u) * p.ldb];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u)
#pragma unroll
            for (int i = 0; i < RW; ++i) acc[i] = __builtin_fmaf(arow[i][k + u], b[u], acc[i]);
    }
    for (; k < k1; ++k) {
        const float b = bcol[(long long)k * p.ldb];
#pragma unroll
        for (int i = 0; i < RW; ++i) acc[i] = __builtin_fmaf(arow[i][k], b, acc[i]);
    }

#pragma unroll
    for (int i = 0; i < RW; ++i) part[slice][r0 + i][lane] = acc[i];
    __syncthreads();
    // output (i, c) of the tile: the slices added in order
    for (int o = threadIdx.x; o < MB * SK_COLS; o += 64 * SK_WAVES) {
        const int i = o / SK_COLS, c = o % SK_COLS;
        const long long cc = (long long)blockIdx.x * SK_COLS + c;
        if (i >= p.M || cc >= p.N) continue;
        float s = part[0][i][c];
#pragma unroll
        for (int w = 1; w < SLICES; ++w) s += part[w][i][c];
        p.C[(long long)i * p.ldc + cc] = s;
    }
}

// 9 to 16 rows: the same plan with a wave per slice of K holding all 16
// rows, and A brought in by vector loads instead of scalar ones: per step
// of 16 k a lane loads 4 values of A (row lane / 4, k 4 (lane % 4) ..) with
// the step's rows of B and writes them to the wave's own corner of LDS,
// whence every lane reads them back as broadcasts.  (Scalar loads of 16
// rows held the waves at 3.4 TB/s, a step's loads of A waiting behind each
// other.)  The corner is private to its wave, so a wave-scope release and
// acquire around a wave barrier orders each step's writes before the reads
// and the reads before the next step's writes; they cost no instruction.
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__global__ __launch_bounds__(64 * SK_WAVES)
void skinny_m16_kernel(GemmArgs p) {
    constexpr int MB = 16, U = 16;
    __shared__ float part[SK_WAVES][MB][SK_COLS];
    __shared__ __attribute__((aligned(16))) float ast[SK_WAVES][MB * U];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const long long col = (long long)blockIdx.x * SK_COLS + lane;
    const float* __restrict__ bcol = p.B + (col < p.N ? col : 0);
    const long long kper = ((long long)p.K + SK_WAVES - 1) / SK_WAVES;
    const int k0 = (int)min((long long)p.K, wave * kper), k1 = (int)min((long long)p.K, k0 + kper);
    // this lane's share of a step's A: row ar (past M: row M - 1), k ak .. ak + 3
    const int ar = lane >> 2, ak = 4 * (lane & 3);
    const float* __restrict__ amine = p.A + (long long)min(ar, p.M - 1) * p.lda + ak;
    float* const corner = ast[wave];
    float acc[MB];
#pragma unroll
    for (int i = 0; i < MB; ++i) acc[i] = 0.f;
    int k = k0;
    for (; k + U <= k1; k += U) {
        float b[U], av[4];
#pragma unroll
        for (int u = 0; u < U; ++u) b[u] = bcol[(long long)(k + u) * p.ldb];
#pragma unroll
        for (int e = 0; e < 4; ++e) av[e] = amine[k + e];
        *reinterpret_cast<float4*>(&corner[ar * U + ak]) = make_float4(av[0], av[1], av[2], av[3]);
        wave_sync();
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int u = 0; u < U; u += 4) {
                const float4 a4 = *reinterpret_cast<const float4*>(&corner[i * U + u]);
                acc[i] = __builtin_fmaf(a4.x, b[u], acc[i]);
                acc[i] = __builtin_fmaf(a4.y, b[u + 1], acc[i]);
                acc[i] = __builtin_fmaf(a4.z, b[u + 2], acc[i]);
                acc[i] = __builtin_fmaf(a4.w, b[u + 3], acc[i]);
            }
        wave_sync();
    }
    for (; k < k1; ++k) {
        const float bk = bcol[(long long)k * p.ldb];
#pragma unroll
        for (int i = 0; i < MB; ++i) acc[i] = __builtin_fmaf(p.A[(long long)min(i, p.M - 1) * p.lda + k], bk, acc[i]);
    }
#pragma unroll
    for (int i = 0; i < MB; ++i) part[wave][i][lane] = acc[i];
    __syncthreads();
    for (int o = threadIdx.x; o < MB * SK_COLS; o += 64 * SK_WAVES) {
        const int i = o / SK_COLS, c = o % SK_COLS;
        const long long cc = (long long)blockIdx.x * SK_COLS + c;
        if (i >= p.M || cc >= p.N) continue;
        float s = part[0][i][c];
#pragma unroll
        for (int w = 1; w < SK_WAVES; ++w) s += part[w][i][c];
        p.C[(long long)i * p.ldc + cc] = s;
    }
}

template <int MB>
hipError_t launch_mb(const GemmArgs& a, hipStream_t stream) {
    const long long blocks = ((long long)a.N + SK_COLS - 1) / SK_COLS;
    hipLaunchKernelGGL((skinny_m_kernel<MB>), dim3((unsigned)blocks), dim3(64 * SK_WAVES), 0, stream, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// B with 1 or 2 columns: reading A bounds the product the same way.  A
// wave owns 16 rows of A (16 x NB partial sums per lane) and walks
// all of K for them, its lanes splitting each 256-k step: lane l takes
// k = kb + l + 64e, e < 4, so every load of A is 64 consecutive floats of
// one row (coalesced); the lane's rows of B (1 or 2 floats each) come
// from the L2.  The 64 lanes' partial sums are then added by a butterfly
// of lane exchanges (the same order on every run) and stored.  k past K
// contributes zero (both factors are set to zero, so no NaN from 0 x Inf).
template <int NB>
struct SknCfg {
    static constexpr int R = 16;   // rows of A per wave (R x NB <= 64 sums)
};

template <int NB>
__global__ __launch_bounds__(256)
void skinny_n_kernel(GemmArgs p) {
    constexpr int R = SknCfg<NB>::R;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const long long row0 = ((long long)blockIdx.x * 4 + wave) * R;
    if (row0 >= p.M) return;   // whole waves; no barrier follows
    // rows past M repeat row M - 1 and columns past N column N - 1 (not stored)
    const float* __restrict__ arow[R];
#pragma unroll
    for (int i = 0; i < R; ++i) arow[i] = p.A + min(row0 + i, (long long)p.M - 1) * p.lda;
    float acc[R][NB];
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = 0.f;
    for (long long kb = 0; kb < p.K; kb += 256) {
        float a[4][R], bv[4][NB];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const long long k = kb + lane + 64 * e;
            const bool ok = k < p.K;
            const long long kk = ok ? k : 0;
#pragma unroll
            for (int i = 0; i < R; ++i) a[e][i] = arow[i][kk];
            const float* __restrict__ brow = p.B + kk * p.ldb;
#pragma unroll
            for (int j = 0; j < NB; ++j) bv[e][j] = brow[min(j, p.N - 1)];
            if (!ok) {
#pragma unroll
                for (int i = 0; i < R; ++i) a[e][i] = 0.f;
#pragma unroll
                for (int j = 0; j < NB; ++j) bv[e][j] = 0.f;
            }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int i = 0; i < R; ++i)
#pragma unroll
                for (int j = 0; j < NB; ++j) acc[i][j] = __builtin_fmaf(a[e][i], bv[e][j], acc[i][j]);
    }
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            float v = acc[i][j];
#pragma unroll
            for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
            acc[i][j] = v;
        }
    // lane i NB + j stores output (i, j)
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
            if (lane == i * NB + j && row0 + i < p.M && j < p.N) p.C[(row0 + i) * p.ldc + j] = acc[i][j];
}

// 3 to 16 columns: the workgroup's 4 waves walk the same 256-k steps and
// share each step's rows of B, copied once into LDS (consecutive threads
// read consecutive elements of B, so the copy is coalesced where B's rows
// are), double-buffered so that one barrier per step suffices; a lane then
// reads its four rows of B from LDS (rows padded by 4 floats).  A wave owns
// R rows of A (at most 64 / NB).  (Each lane reading its own rows of B from the L2
// bounded 8 columns at 2.2 TB/s and 16 at 0.6; this copy reaches 5.3 and
// 3.7.)
template <int NB, int R>
__global__ __launch_bounds__(256)
void skinny_n_lds_kernel(GemmArgs p) {
    constexpr int SB = NB + 4;
    __shared__ __attribute__((aligned(16))) float bs[2][256 * SB];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const long long row0 = ((long long)blockIdx.x * 4 + wave) * R;
    // rows past M repeat row M - 1 (not stored); every wave takes part in
    // the copies and barriers
    const float* __restrict__ arow[R];
#pragma unroll
    for (int i = 0; i < R; ++i) arow[i] = p.A + min(row0 + i, (long long)p.M - 1) * p.lda;
    float acc[R][NB];
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = 0.f;
    // element q of a step's 256 x NB block of B: row q / NB, column q % NB;
    // past K or N it is zero
    auto copy_b = [&](long long kb, int buf) {
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            const int q = (int)threadIdx.x + 256 * u, r = q / NB, j = q % NB;
            const long long k = kb + r;
            const bool ok = k < p.K && j < p.N;
            const float v = p.B[(ok ? k : 0) * p.ldb + (ok ? j : 0)];
            bs[buf][r * SB + j] = ok ? v : 0.f;
        }
    };
    int buf = 0;
    if (p.K > 0) copy_b(0, 0);
    __syncthreads();
    for (long long kb = 0; kb < p.K; kb += 256) {
        if (kb + 256 < p.K) copy_b(kb + 256, buf ^ 1);
        float a[4][R];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const long long k = kb + lane + 64 * e;
            const bool ok = k < p.K;
#pragma unroll
            for (int i = 0; i < R; ++i) {
                const float v = arow[i][ok ? k : 0];
                a[e][i] = ok ? v : 0.f;
            }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float* brow = &bs[buf][(lane + 64 * e) * SB];
            float bv[NB];
#pragma unroll
            for (int j = 0; j < NB; j += 4) {
                const float4 t = *reinterpret_cast<const float4*>(brow + j);
                bv[j] = t.x; bv[j + 1] = t.y; bv[j + 2] = t.z; bv[j + 3] = t.w;
            }
#pragma unroll
            for (int i = 0; i < R; ++i)
#pragma unroll
                for (int j = 0; j < NB; ++j) acc[i][j] = __builtin_fmaf(a[e][i], bv[j], acc[i][j]);
        }
        __syncthreads();   // this step's buffer is free; the next one is in LDS
        buf ^= 1;
    }
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            float v = acc[i][j];
#pragma unroll
            for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
            acc[i][j] = v;
        }
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
            if (lane == i * NB + j && row0 + i < p.M && j < p.N) p.C[(row0 + i) * p.ldc + j] = acc[i][j];
}

// R = 64 / NB rows of A per wave, or (up to 8 columns) a quarter of that
// when it would leave fewer than 4096 waves (16 per CU) to hide the latency
// of the reads of A: 8192x4x8192 3.3 -> 4.4 TB/s.  With 16 columns one row
// per wave reads B from LDS 16 times per element of A and loses (3.0 -> 1.6).
// Workgroups of 4 waves of R rows each: the grid's threads must stay within
// the 32-bit launch limit, else the matrix-core path takes the shape.
template <int R>
bool skinny_grid_fits(const GemmArgs& a) {
    return ((long long)a.M + 4 * R - 1) / (4 * R) * 256 <= 0xFFFFFFFFll;
}

template <int NB, int R>
hipError_t launch_nb_lds_r(const GemmArgs& a, hipStream_t stream) {
    if (!skinny_grid_fits<R>(a)) return launch_mfma(a, stream);
    const long long blocks = ((long long)a.M + 4 * R - 1) / (4 * R);
    hipLaunchKernelGGL((skinny_n_lds_kernel<NB, R>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}
template <int NB>
hipError_t launch_nb_lds(const GemmArgs& a, hipStream_t stream) {
    constexpr int R = 64 / NB;
    if constexpr (R >= 8) {
        if ((long long)a.M < 4096LL * R) return launch_nb_lds_r<NB, R / 4>(a, stream);
    }
    return launch_nb_lds_r<NB, R>(a, stream);
}

template <int NB>
hipError_t launch_nb(const GemmArgs& a, hipStream_t stream) {
    constexpr int R = SknCfg<NB>::R;
    if (!skinny_grid_fits<R>(a)) return launch_mfma(a, stream);
    const long long blocks = ((long long)a.M + 4 * R - 1) / (4 * R);
    hipLaunchKernelGGL((skinny_n_kernel<NB>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

// (each launcher checks that its grid fits the 32-bit launch limit and
// hands the shape to the matrix-core path where it does not: with 9 to 16
// columns from 2^28 rows on)
bool skinny_n_fits(const GemmArgs& a) {
    return a.N >= 1 && a.N <= 16 && a.M > 16 && !a.epi;
}

hipError_t launch_skinny_n(const GemmArgs& a, hipStream_t stream) {
    if (!skinny_n_fits(a)) return hipErrorInvalidValue;
    if (a.N <= 1) return launch_nb<1>(a, stream);
    if (a.N <= 2) return launch_nb<2>(a, stream);
    if (a.N <= 4) return launch_nb_lds<4>(a, stream);
    if (a.N <= 8) return launch_nb_lds<8>(a, stream);
    return launch_nb_lds<16>(a, stream);
}

// (the grid's thread count within the 32-bit launch limit)
bool skinny_m_fits(const GemmArgs& a) {
    return a.M >= 1 && a.M <= 16 && !a.epi &&
           ((long long)a.N + SK_COLS - 1) / SK_COLS * 64 * SK_WAVES <= 0xFFFFFFFFll;
}

hipError_t launch_skinny_m(const GemmArgs& a, hipStream_t stream) {
    if (!skinny_m_fits(a)) return hipErrorInvalidValue;
    if (a.M <= 1) return launch_mb<1>(a, stream);
    if (a.M <= 2) return launch_mb<2>(a, stream);
    if (a.M <= 4) return launch_mb<4>(a, stream);
    if (a.M <= 8) return launch_mb<8>(a, stream);
    const long long blocks = ((long long)a.N + SK_COLS - 1) / SK_COLS;
    hipLaunchKernelGGL(skinny_m16_kernel, dim3((unsigned)blocks), dim3(64 * SK_WAVES), 0, stream, a);
    return hipGetLastError();
}

}  // namespace sgemm
