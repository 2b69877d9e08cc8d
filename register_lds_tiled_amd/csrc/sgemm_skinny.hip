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
//    rows on A comes through LDS (skinny_m16_kernel); from 4 rows, where
//    64-column workgroups would leave many CUs idle, a workgroup takes 32
//    or 16 columns and each wave's lanes split its slice of K once more
//    (skinny_m_split_kernel);
//  * the 16 partial sums of each output are added through LDS in wave
//    order, so the result does not depend on timing.
#include <cstdint>

#include "tiles.h"

namespace sgemm {
namespace {

constexpr int SK_WAVES = 16;   // waves per workgroup, one slice of K each
constexpr int SK_COLS = 64;    // columns of C per workgroup

// The operand that is read once -- B when A has few rows, A when B has few
// columns -- is loaded with the nontemporal hint (NT) when it is larger than
// the chip's 256 MB last-level cache: it then streams through the caches
// without displacing the small operand that every workgroup reads again
// (65536 x 4 x 8192, A 2 GB: 4.8 -> 6.1 TB/s; 16384 x 4 x 8192, 512 MB:
// 5.0 -> 5.4).  An operand that fits (8192 x 1 x 8192, 256 MB) is read
// without the hint: back-to-back products then find part of it still in
// that cache (6.1 TB/s, against 4.1 with the hint).
constexpr long long SK_NT_BYTES = 256LL << 20;

template <bool NT>
__device__ __forceinline__ float stream_load(const float* p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}
typedef float sk_f4 __attribute__((ext_vector_type(4)));
template <bool NT>
__device__ __forceinline__ float4 stream_load4(const float* p) {
    if constexpr (NT) {
        const sk_f4 t = __builtin_nontemporal_load(reinterpret_cast<const sk_f4*>(p));
        return make_float4(t[0], t[1], t[2], t[3]);
    } else {
        return *reinterpret_cast<const float4*>(p);
    }
}

// Output (row, col) of C from its finished sum: the plain product, or with
// the fused epilogue (sgemm_f32_ex: alpha, beta * C, bias, ReLU, the
// expression of fused_out), chosen per call -- a uniform branch at the
// store, outside every loop.  C is read only when beta != 0.
__device__ __forceinline__ void sk_store(const GemmArgs& p, long long row, long long col, float s) {
    float* const c = p.C + row * p.ldc + col;
    if (p.epi) {
        const float c_in = p.beta != 0.f ? *c : 0.f;
        const float bias_j = p.bias != nullptr ? p.bias[col] : 0.f;
        s = fused_out(p, s, c_in, bias_j);
    }
    *c = s;
}

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

template <int MB, bool NT>
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
        for (int u = 0; u < UNROLL; ++u) b[u] = stream_load<NT>(bcol + (long long)(k + u) * p.ldb);
#pragma unroll
        for (int u = 0; u < UNROLL; ++u)
#pragma unroll
            for (int i = 0; i < RW; ++i) acc[i] = __builtin_fmaf(arow[i][k + u], b[u], acc[i]);
    }
    for (; k < k1; ++k) {
        const float b = stream_load<NT>(bcol + (long long)k * p.ldb);
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
        sk_store(p, i, cc, s);
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

template <bool NT>
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
        // (debug build: the previous step's second wave_sync retired the
        // corner)
        if constexpr (kLdsPoison) lds_poison_f4(&corner[ar * U + ak]);
        float b[U], av[4];
#pragma unroll
        for (int u = 0; u < U; ++u) b[u] = stream_load<NT>(bcol + (long long)(k + u) * p.ldb);
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
        const float bk = stream_load<NT>(bcol + (long long)k * p.ldb);
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
        sk_store(p, i, cc, s);
    }
}

// B's bytes (the operand the few-row kernels stream) and A's (the one the
// few-column kernels stream) against the last-level cache
static bool b_streams(const GemmArgs& a) { return 4LL * a.K * a.N > SK_NT_BYTES; }
static bool a_streams(const GemmArgs& a) { return 4LL * a.M * a.K > SK_NT_BYTES; }

// Few rows of A and few columns of C (fewer 64-column blocks than CUs, e.g.
// 8 x 8192 x 8192: 128 workgroups for 256 CUs): a workgroup owns 64 / H
// columns and each wave's slice of K is split once more between its H lane
// groups (lane = h (64 / H) + c: column c, the h-th U-long run of each
// H U-long step), so that the grid has H times the workgroups.  A comes
// through the wave's corner of LDS as in the 16-row kernel (the lane groups
// read different k there); B's rows come as H runs of 64 / H consecutive
// floats per load.  The partial sums of the waves and lane groups are added
// in a fixed order (wave, then group).
template <int MB, int H, bool NT>
__global__ __launch_bounds__(64 * SK_WAVES)
void skinny_m_split_kernel(GemmArgs p) {
    constexpr int COLS = SK_COLS / H, U = 16, KS = H * U;
    __shared__ float part[SK_WAVES][H][MB][COLS];
    __shared__ __attribute__((aligned(16))) float ast[SK_WAVES][MB * KS];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c = lane % COLS, h = lane / COLS;
    const long long col = (long long)blockIdx.x * COLS + c;
    // a column past N reads column 0 of B (always there) and is not stored
    const float* __restrict__ bcol = p.B + (col < p.N ? col : 0);
    const long long kper = ((long long)p.K + SK_WAVES - 1) / SK_WAVES;
    const int k0 = (int)min((long long)p.K, wave * kper), k1 = (int)min((long long)p.K, k0 + kper);
    float* const corner = ast[wave];
    float acc[MB];
#pragma unroll
    for (int i = 0; i < MB; ++i) acc[i] = 0.f;
    int k = k0;
    for (; k + KS <= k1; k += KS) {
        if constexpr (kLdsPoison) {
#pragma unroll
            for (int e0 = 0; e0 < MB * KS; e0 += 64)
                if (MB * KS % 64 == 0 || e0 + lane < MB * KS) lds_poison_f1(&corner[e0 + lane]);
        }
        float b[U];
#pragma unroll
        for (int u = 0; u < U; ++u) b[u] = stream_load<NT>(bcol + (long long)(k + h * U + u) * p.ldb);
        // the step's A (MB rows x KS k; rows past M repeat row M - 1)
#pragma unroll
        for (int e0 = 0; e0 < MB * KS; e0 += 64) {
            const int e = e0 + lane;
            if (MB * KS % 64 == 0 || e < MB * KS) {
                const int r = e / KS, kk = e % KS;
                corner[e] = p.A[(long long)min(r, p.M - 1) * p.lda + k + kk];
            }
        }
        wave_sync();
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int u = 0; u < U; u += 4) {
                const float4 a4 = *reinterpret_cast<const float4*>(&corner[i * KS + h * U + u]);
                acc[i] = __builtin_fmaf(a4.x, b[u], acc[i]);
                acc[i] = __builtin_fmaf(a4.y, b[u + 1], acc[i]);
                acc[i] = __builtin_fmaf(a4.z, b[u + 2], acc[i]);
                acc[i] = __builtin_fmaf(a4.w, b[u + 3], acc[i]);
            }
        wave_sync();
    }
    // the slice's tail: lane group h takes every H-th k
    for (int kk = k + h; kk < k1; kk += H) {
        const float bk = stream_load<NT>(bcol + (long long)kk * p.ldb);
#pragma unroll
        for (int i = 0; i < MB; ++i) acc[i] = __builtin_fmaf(p.A[(long long)min(i, p.M - 1) * p.lda + kk], bk, acc[i]);
    }
#pragma unroll
    for (int i = 0; i < MB; ++i) part[wave][h][i][c] = acc[i];
    __syncthreads();
    for (int o = threadIdx.x; o < MB * COLS; o += 64 * SK_WAVES) {
        const int i = o / COLS, cc = o % COLS;
        const long long gc = (long long)blockIdx.x * COLS + cc;
        if (i >= p.M || gc >= p.N) continue;
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < SK_WAVES; ++w)
#pragma unroll
            for (int g = 0; g < H; ++g) s = w == 0 && g == 0 ? part[0][0][i][cc] : s + part[w][g][i][cc];
        sk_store(p, i, gc, s);
    }
}

template <int MB, int H>
hipError_t launch_m_split(const GemmArgs& a, hipStream_t stream) {
    const long long blocks = ((long long)a.N + SK_COLS / H - 1) / (SK_COLS / H);
    if (b_streams(a))
        hipLaunchKernelGGL((skinny_m_split_kernel<MB, H, true>), dim3((unsigned)blocks), dim3(64 * SK_WAVES), 0,
                           stream, a);
    else
        hipLaunchKernelGGL((skinny_m_split_kernel<MB, H, false>), dim3((unsigned)blocks), dim3(64 * SK_WAVES), 0,
                           stream, a);
    return hipGetLastError();
}

// 9 to 16 rows of A, on the matrix cores.  The vector-ALU kernels above
// read every row of A once per k for each lane, from LDS, which bounds them
// there (16 x 8192 x 8192: 3.3 TB/s).  One v_mfma_f32_16x16x4_f32 takes
// 16 rows x 4 k of A and 4 k x 16 columns of B, one element of each per
// lane, so a wave keeps its A (row lane % 16, k group lane / 16) in
// registers, four k per lane per 16 k, and B goes from memory straight into
// the MFMA operands: lane (c = lane % 16, q = lane / 16) loads row
// k + 4q + s of B at columns n0 + NJ c .. NJ c + NJ - 1 (a float4, float2
// or float for 64-, 32- or 16-column workgroups), and component j feeds
// block j, whose column c is n0 + NJ c + j.  Nothing goes through LDS but
// the partial sums: the 16 waves of a workgroup take slices of K and their
// sums are added in a fixed order (wave 0 first), as in the kernels above.
// Slices are whole iterations of U 16-k groups except the last, whose
// short iteration reads k past K as zero in both factors.  A row past M
// repeats row M - 1 (never stored).  A is read four floats at a time where
// its rows are 16-byte aligned (AX4), else one at a time.  B likewise: a
// group load where B's rows are aligned to it and N is a multiple of NJ
// (BV; a lane wholly past N then reads column 0), else NJ loads of one
// float, a column past N reading column 0.  Outputs past N are not stored.
typedef float sk_f2 __attribute__((ext_vector_type(2)));
template <int NJ, bool NT>
__device__ __forceinline__ sk_f4 load_bgroup(const float* p) {
    if constexpr (NJ == 4) {
        if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const sk_f4*>(p));
        else return *reinterpret_cast<const sk_f4*>(p);
    } else if constexpr (NJ == 2) {
        sk_f2 t;
        if constexpr (NT) t = __builtin_nontemporal_load(reinterpret_cast<const sk_f2*>(p));
        else t = *reinterpret_cast<const sk_f2*>(p);
        return sk_f4{t[0], t[1], 0.f, 0.f};
    } else {
        return sk_f4{stream_load<NT>(p), 0.f, 0.f, 0.f};
    }
}

// B's group one float at a time (rows not aligned to the group), each
// column from its own offset in the row (a column past N reads column 0)
template <int NJ, bool NT>
__device__ __forceinline__ sk_f4 load_bgroup_el(const float* row, const int (&off)[NJ]) {
    sk_f4 v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < NJ; ++j) v[j] = stream_load<NT>(row + off[j]);
    return v;
}

template <int COLS, bool NT, bool AX4, bool BV>
__global__ __launch_bounds__(64 * SK_WAVES)
void skinny_m_mfma_kernel(GemmArgs p) {
    constexpr int NJ = COLS / 16;   // 16 x 16 blocks of C per wave
    constexpr int U = 8 / NJ;       // 16-k groups per iteration: 512 bytes of B in flight per lane
    static_assert(NJ == 4 || NJ == 2 || NJ == 1, "64, 32 or 16 columns");
    __shared__ float part[SK_WAVES][16][COLS];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c = lane & 15, q = lane >> 4;
    const long long n0 = (long long)blockIdx.x * COLS;
    const long long K = p.K;
    // slices of whole iterations (16 U k), so that only the last slice has
    // a short iteration
    const long long kper = ((K + SK_WAVES - 1) / SK_WAVES + 16 * U - 1) / (16 * U) * (16 * U);
    const long long k0 = min(K, wave * kper), k1 = min(K, k0 + kper);
    const long long col = n0 + NJ * c;
    const float* __restrict__ arow = p.A + (long long)min(c, p.M - 1) * p.lda + 4 * q;
    const float* __restrict__ brow = p.B + 4LL * q * p.ldb;
    const float* __restrict__ bcol = brow + (col < p.N ? col : 0);
    int boff[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) boff[j] = col + j < p.N ? (int)col + j : 0;
    // row r of the lane's B group (r counted from the lane's first row 4q)
    auto load_b = [&](long long r) {
        if constexpr (BV) return load_bgroup<NJ, NT>(bcol + r * p.ldb);
        else return load_bgroup_el<NJ, NT>(brow + r * p.ldb, boff);
    };
    sk_f4 acc[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[j] = sk_f4{0.f, 0.f, 0.f, 0.f};
    auto mma = [&](const float4& a, const sk_f4 (&b)[4]) {
        const float av[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[s], b[s][j], acc[j], 0, 0, 0);
    };
    long long k = k0;
    for (; k + 16 * U <= k1; k += 16 * U) {
        float4 a[U];
        sk_f4 b[U][4];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if constexpr (AX4) {
                a[u] = *reinterpret_cast<const float4*>(arow + k + 16 * u);
            } else {
                const float* const ak = arow + k + 16 * u;
                a[u] = make_float4(ak[0], ak[1], ak[2], ak[3]);
            }
#pragma unroll
            for (int s = 0; s < 4; ++s) b[u][s] = load_b(k + 16 * u + s);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) mma(a[u], b[u]);
    }
    if (k < k1) {
        // the last slice's short iteration: k past k1 is zero in A and in
        // B (its addresses go to k0, always inside the matrices)
        float4 a[U];
        sk_f4 b[U][4];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float ae[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const long long kk = k + 16 * u + e;   // (the lane's k is kk + 4q)
                const bool in = kk + 4 * q < k1;
                const float av = arow[in ? kk : k0 - 4 * q];
                ae[e] = in ? av : 0.f;
                const sk_f4 bv = load_b(in ? kk : k0 - 4 * q);
                b[u][e] = in ? bv : sk_f4{0.f, 0.f, 0.f, 0.f};
            }
            a[u] = make_float4(ae[0], ae[1], ae[2], ae[3]);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) mma(a[u], b[u]);
    }
    // block j, register r: row 4q + r, column NJ c + j of the workgroup
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) part[wave][4 * q + r][NJ * c + j] = acc[j][r];
    __syncthreads();
    for (int o = threadIdx.x; o < 16 * COLS; o += 64 * SK_WAVES) {
        const int i = o / COLS, cc = o % COLS;
        if (i >= p.M || n0 + cc >= p.N) continue;
        float sum = part[0][i][cc];
#pragma unroll
        for (int w = 1; w < SK_WAVES; ++w) sum += part[w][i][cc];
        sk_store(p, i, n0 + cc, sum);
    }
}

// B's loads of NJ columns need its rows aligned to them and N a multiple of
// NJ (always so for NJ = 1); A is read four floats at a time where its rows
// are 16-byte aligned (AX4), else one at a time.
static bool m_mfma_b_fits(const GemmArgs& a, int nj) {
    const uintptr_t ub = reinterpret_cast<uintptr_t>(a.B);
    return (ub & (4 * nj - 1)) == 0 && a.ldb % nj == 0 && a.N % nj == 0;
}
static bool m_mfma_a16(const GemmArgs& a) {
    return (reinterpret_cast<uintptr_t>(a.A) & 15) == 0 && a.lda % 4 == 0;
}

template <int COLS, bool NT, bool AX4>
void launch_m_mfma_a(const GemmArgs& a, hipStream_t stream) {
    const long long blocks = ((long long)a.N + COLS - 1) / COLS;
    if (COLS == 16 || m_mfma_b_fits(a, COLS / 16))   // (16 columns: one float per lane, always fits)
        hipLaunchKernelGGL((skinny_m_mfma_kernel<COLS, NT, AX4, true>), dim3((unsigned)blocks),
                           dim3(64 * SK_WAVES), 0, stream, a);
    else if constexpr (COLS != 16 && !NT)   // (the launcher streams no misaligned B)
        hipLaunchKernelGGL((skinny_m_mfma_kernel<COLS, NT, AX4, false>), dim3((unsigned)blocks),
                           dim3(64 * SK_WAVES), 0, stream, a);
}
template <int COLS, bool NT>
void launch_m_mfma_nt(const GemmArgs& a, hipStream_t stream) {
    if (m_mfma_a16(a)) launch_m_mfma_a<COLS, NT, true>(a, stream);
    else launch_m_mfma_a<COLS, NT, false>(a, stream);
}
template <int COLS>
hipError_t launch_m_mfma(const GemmArgs& a, hipStream_t stream) {
    if (b_streams(a)) launch_m_mfma_nt<COLS, true>(a, stream);
    else launch_m_mfma_nt<COLS, false>(a, stream);
    return hipGetLastError();
}

// The split form from 4 rows of A, where its grid stays within one round of
// one workgroup per CU and keeps clearly more of the CUs busy than the
// 64-column one (at least 0.15 more of them), with the fewer lane groups on
// a tie: 8 x 8192 x 8192 3.7 -> 5.7 TB/s, 16 x 8192 x 8192 2.8 -> 3.3,
// 16 x 4096 x 8192 1.4 -> 2.0, 4 x 8192 x 8192 5.6 -> 5.8.  Below 4 rows the
// 64-column kernel keeps 64 / rows rows of B in flight per lane and stays
// ahead (1 x 8192 x 8192: 6.3 against 6.1), and so does it where the split
// grid would need a second round (8 x 12000 x 3000: 188 workgroups at 4.4
// TB/s, against 3.1 for 750 of 16 columns).
static double sk_fill(long long blocks, long long cus) {
    const long long rounds = (blocks + cus - 1) / cus;
    return (double)blocks / (double)(rounds * cus);
}
template <int MB>
bool launch_m_narrow(const GemmArgs& a, hipStream_t stream, hipError_t& err) {
    if constexpr (MB < 4) {
        return false;
    } else {
        const long long cus = a.cus > 0 ? a.cus : 256;
        const long long b64 = ((long long)a.N + SK_COLS - 1) / SK_COLS;
        const long long b32 = ((long long)a.N + 31) / 32, b16 = ((long long)a.N + 15) / 16;
        const double f1 = sk_fill(b64, cus);
        const double f2 = b32 <= cus ? sk_fill(b32, cus) : 0.0, f4 = b16 <= cus ? sk_fill(b16, cus) : 0.0;
        if (f2 >= f4 && f2 >= f1 + 0.15) {
            err = launch_m_split<MB, 2>(a, stream);
            return true;
        }
        if (f4 > f2 && f4 >= f1 + 0.15) {
            err = launch_m_split<MB, 4>(a, stream);
            return true;
        }
        return false;
    }
}

template <int MB>
hipError_t launch_mb(const GemmArgs& a, hipStream_t stream) {
    const long long blocks = ((long long)a.N + SK_COLS - 1) / SK_COLS;
    if (b_streams(a))
        hipLaunchKernelGGL((skinny_m_kernel<MB, true>), dim3((unsigned)blocks), dim3(64 * SK_WAVES), 0, stream, a);
    else
        hipLaunchKernelGGL((skinny_m_kernel<MB, false>), dim3((unsigned)blocks), dim3(64 * SK_WAVES), 0, stream, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// B with 1 or 2 columns: reading A bounds the product the same way.  A
// wave owns R rows of A (R x NB partial sums per lane) and walks
// all of K for them, its lanes splitting each 256-k step: lane l takes
// k = kb + l + 64e, e < 4, so every load of A is 64 consecutive floats of
// one row (coalesced); the lane's rows of B (1 or 2 floats each) come
// from the L2.  The 64 lanes' partial sums are then added by a butterfly
// of lane exchanges (the same order on every run) and stored.  k past K
// contributes zero (both factors are set to zero, so no NaN from 0 x Inf).
// R rows of A per wave (R x NB <= 64 sums): 16, or 8 or 4 where 16 would
// leave too many CUs idle (the launcher).
template <int NB, int R, bool NT>
__global__ __launch_bounds__(256)
void skinny_n_kernel(GemmArgs p) {
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
            for (int i = 0; i < R; ++i) a[e][i] = stream_load<NT>(arow[i] + kk);
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
            if (lane == i * NB + j && row0 + i < p.M && j < p.N) sk_store(p, row0 + i, j, acc[i][j]);
}

// 3 to 16 columns: the workgroup's 4 waves walk the same 256-k steps and
// share each step's rows of B, copied once into LDS (consecutive threads
// read consecutive elements of B, so the copy is coalesced where B's rows
// are), double-buffered so that one barrier per step suffices; a lane then
// reads its four rows of B from LDS (rows padded by 4 floats).  A wave owns
// R rows of A (at most 64 / NB).  (Each lane reading its own rows of B from the L2
// bounded 8 columns at 2.2 TB/s and 16 at 0.6; this copy reaches 5.3 and
// 3.7.)
template <int NB, int R, bool NT>
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
    // debug build: the words copy_b(.., buf) is about to write
    auto poison_b = [&](int buf) {
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            const int q = (int)threadIdx.x + 256 * u;
            lds_poison_f1(&bs[buf][(q / NB) * SB + q % NB]);
        }
    };
    int buf = 0;
    if (p.K > 0) copy_b(0, 0);
    __syncthreads();
    for (long long kb = 0; kb < p.K; kb += 256) {
        // (the barrier ending the previous step retired buffer buf ^ 1)
        if (kLdsPoison && kb + 256 < p.K) poison_b(buf ^ 1);
        if (kb + 256 < p.K) copy_b(kb + 256, buf ^ 1);
        float a[4][R];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const long long k = kb + lane + 64 * e;
            const bool ok = k < p.K;
#pragma unroll
            for (int i = 0; i < R; ++i) {
                const float v = stream_load<NT>(arow[i] + (ok ? k : 0));
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
            if (lane == i * NB + j && row0 + i < p.M && j < p.N) sk_store(p, row0 + i, j, acc[i][j]);
}

// 3 to 8 columns with A's rows 16-byte aligned: the same plan with 16-byte
// loads of A.  A lane takes four consecutive k of a row per load, k = kb +
// 4 (l + 64 v) + c for c < 4 and v < KV, so one instruction brings 1 KB of
// a row for the wave instead of 256 bytes.  The step's rows of B are laid
// out in LDS to match: the NB values of row kb + 4 (l + 64 v) + c sit as
// NB / 4 float4 at ((v 4 + c) NB / 4 + jq) 64 + l, so the lanes of a wave
// read consecutive 16-byte words (no bank conflict).  The last, partial
// step of K loads element by element, each k past K as zero.
template <int NB, int R, int KV, bool NT>
__global__ __launch_bounds__(256)
void skinny_n_vec_kernel(GemmArgs p) {
    constexpr int NQ = NB / 4, STEP = 256 * KV;
    static_assert(NB % 4 == 0 && R * NB <= 64, "float4 column groups; one output per lane");
    __shared__ float4 bs[2][KV * 4 * NQ * 64];
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
    // element q of a step's STEP x NB block of B: row r = q / NB, column
    // j = q % NB (zero past K or N)
    auto copy_b = [&](long long kb, int buf) {
        float* const dst = reinterpret_cast<float*>(bs[buf]);
#pragma unroll
        for (int u = 0; u < KV * NB; ++u) {
            const int q = (int)threadIdx.x + 256 * u, r = q / NB, j = q % NB;
            const long long k = kb + r;
            const bool ok = k < p.K && j < p.N;
            const float v = p.B[(ok ? k : 0) * p.ldb + (ok ? j : 0)];
            const int vv = r >> 8, l = (r & 255) >> 2, c = r & 3;
            dst[(((vv * 4 + c) * NQ + (j >> 2)) * 64 + l) * 4 + (j & 3)] = ok ? v : 0.f;
        }
    };
    auto poison_b = [&](int buf) {
        float* const dst = reinterpret_cast<float*>(bs[buf]);
#pragma unroll
        for (int u = 0; u < KV * NB; ++u) {
            const int q = (int)threadIdx.x + 256 * u, r = q / NB, j = q % NB;
            const int vv = r >> 8, l = (r & 255) >> 2, c = r & 3;
            lds_poison_f1(&dst[(((vv * 4 + c) * NQ + (j >> 2)) * 64 + l) * 4 + (j & 3)]);
        }
    };
    auto fma_step = [&](int buf, const float4 (&a)[KV][R]) {
#pragma unroll
        for (int v = 0; v < KV; ++v)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                float bv[NB];
#pragma unroll
                for (int jq = 0; jq < NQ; ++jq) {
                    const float4 t = bs[buf][((v * 4 + c) * NQ + jq) * 64 + lane];
                    bv[4 * jq] = t.x; bv[4 * jq + 1] = t.y; bv[4 * jq + 2] = t.z; bv[4 * jq + 3] = t.w;
                }
#pragma unroll
                for (int i = 0; i < R; ++i) {
                    const float av = c == 0 ? a[v][i].x : c == 1 ? a[v][i].y : c == 2 ? a[v][i].z : a[v][i].w;
#pragma unroll
                    for (int j = 0; j < NB; ++j) acc[i][j] = __builtin_fmaf(av, bv[j], acc[i][j]);
                }
            }
    };
    int buf = 0;
    if (p.K > 0) copy_b(0, 0);
    __syncthreads();
    long long kb = 0;
    for (; kb + STEP <= p.K; kb += STEP) {
        if (kLdsPoison && kb + STEP < p.K) poison_b(buf ^ 1);
        if (kb + STEP < p.K) copy_b(kb + STEP, buf ^ 1);
        float4 a[KV][R];
#pragma unroll
        for (int v = 0; v < KV; ++v)
#pragma unroll
            for (int i = 0; i < R; ++i) a[v][i] = stream_load4<NT>(arow[i] + kb + 4 * (lane + 64 * v));
        fma_step(buf, a);
        __syncthreads();   // this step's buffer is free; the next one is in LDS
        buf ^= 1;
    }
    if (kb < p.K) {
        float4 a[KV][R];
#pragma unroll
        for (int v = 0; v < KV; ++v)
#pragma unroll
            for (int i = 0; i < R; ++i) {
                const long long k = kb + 4 * (lane + 64 * v);
                float e[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) e[c] = k + c < p.K ? stream_load<NT>(arow[i] + k + c) : 0.f;
                a[v][i] = make_float4(e[0], e[1], e[2], e[3]);
            }
        fma_step(buf, a);
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
            if (lane == i * NB + j && row0 + i < p.M && j < p.N) sk_store(p, row0 + i, j, acc[i][j]);
}

// The 4-byte form (A's rows not 16-byte aligned, or 9 to 16 columns):
// R = 64 / NB rows of A per wave, or a quarter of that -- always at 4
// columns, at 8 when it would leave fewer than 4096 waves (16 per CU) to
// hide the latency of the reads of A: 8192x4x8192 3.3 -> 4.4 TB/s.  With 16 columns one row
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
    if (a_streams(a))
        hipLaunchKernelGGL((skinny_n_lds_kernel<NB, R, true>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((skinny_n_lds_kernel<NB, R, false>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}
template <int NB>
hipError_t launch_nb_lds(const GemmArgs& a, hipStream_t stream) {
    constexpr int R = 64 / NB;
    // 4 columns: 4 rows per wave at any M (this kernel at 65536 x 4 x 8192:
    // 6.2 TB/s with 4 rows, 5.8 with 16)
    if constexpr (NB == 4) {
        return launch_nb_lds_r<NB, R / 4>(a, stream);
    } else {
        if constexpr (R >= 8) {
            if ((long long)a.M < 4096LL * R) return launch_nb_lds_r<NB, R / 4>(a, stream);
        }
        return launch_nb_lds_r<NB, R>(a, stream);
    }
}

// 16-byte loads: 4 columns take 2 rows per wave and 4 loads per row per
// step (65536 x 4 x 8192: 6.1 TB/s, against 5.8 with 4-byte loads; 8192 x
// 4 x 8192: 5.1 against 4.5), 8 columns 8 rows and one load (65536 x 8 x
// 8192: 5.9 TB/s, against 5.7)
template <int NB>
struct SkvCfg;
template <>
struct SkvCfg<4> { static constexpr int R = 2, KV = 4; };
template <>
struct SkvCfg<8> { static constexpr int R = 8, KV = 1; };

template <int NB>
hipError_t launch_nb_vec(const GemmArgs& a, hipStream_t stream) {
    constexpr int R = SkvCfg<NB>::R, KV = SkvCfg<NB>::KV;
    if (!skinny_grid_fits<R>(a)) return launch_mfma(a, stream);
    const long long blocks = ((long long)a.M + 4 * R - 1) / (4 * R);
    if (a_streams(a))
        hipLaunchKernelGGL((skinny_n_vec_kernel<NB, R, KV, true>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((skinny_n_vec_kernel<NB, R, KV, false>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

// A's rows start on 16-byte boundaries
static bool a_rows_16b(const GemmArgs& a) {
    return (reinterpret_cast<uintptr_t>(a.A) & 15) == 0 && a.lda % 4 == 0;
}

template <int NB, int R>
hipError_t launch_nb_r(const GemmArgs& a, hipStream_t stream) {
    if (!skinny_grid_fits<R>(a)) return launch_mfma(a, stream);
    const long long blocks = ((long long)a.M + 4 * R - 1) / (4 * R);
    if (a_streams(a))
        hipLaunchKernelGGL((skinny_n_kernel<NB, R, true>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((skinny_n_kernel<NB, R, false>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}
// The most rows per wave whose grid keeps at least half the CUs busy (one
// column) or all of them (two), else 4: 4096 x 1 x 16384 1.8 -> 2.4 TFLOP/s,
// 2048 x 2 x 2048 1.3 -> 2.1, 8192 x 2 x 8192 5.5 -> 6.0; 8192 x 1 x 8192
// keeps 16 rows on half the CUs (3.0 against 2.9 at 8 rows on all).
template <int NB>
hipError_t launch_nb(const GemmArgs& a, hipStream_t stream) {
    const long long cus = a.cus > 0 ? a.cus : 256;
    const long long need = NB == 1 ? (cus + 1) / 2 : cus;
    auto blocks = [&](int r) { return ((long long)a.M + 4 * r - 1) / (4 * r); };
    if (blocks(16) >= need) return launch_nb_r<NB, 16>(a, stream);
    if (blocks(8) >= need) return launch_nb_r<NB, 8>(a, stream);
    return launch_nb_r<NB, 4>(a, stream);
}

}  // namespace

// (each launcher checks that its grid fits the 32-bit launch limit and
// hands the shape to the matrix-core path where it does not: with 9 to 16
// columns from 2^28 rows on)
bool skinny_n_fits(const GemmArgs& a) {
    return a.N >= 1 && a.N <= 16 && a.M > 16;
}

hipError_t launch_skinny_n(const GemmArgs& a, hipStream_t stream) {
    if (!skinny_n_fits(a)) return hipErrorInvalidValue;
    if (a.N <= 1) return launch_nb<1>(a, stream);
    if (a.N <= 2) return launch_nb<2>(a, stream);
    if (a.N <= 4) return a_rows_16b(a) ? launch_nb_vec<4>(a, stream) : launch_nb_lds<4>(a, stream);
    // (8 columns below 32768 rows: 8 rows per wave would leave too few
    // waves; the 4-byte kernel then takes 2)
    if (a.N <= 8)
        return a_rows_16b(a) && a.M >= 32768 ? launch_nb_vec<8>(a, stream) : launch_nb_lds<8>(a, stream);
    return launch_nb_lds<16>(a, stream);
}

// (the grid's thread count within the 32-bit launch limit)
bool skinny_m_fits(const GemmArgs& a) {
    return a.M >= 1 && a.M <= 16 &&
           ((long long)a.N + SK_COLS - 1) / SK_COLS * 64 * SK_WAVES <= 0xFFFFFFFFll;
}

hipError_t launch_skinny_m(const GemmArgs& a, hipStream_t stream) {
    if (!skinny_m_fits(a)) return hipErrorInvalidValue;
    hipError_t err = hipSuccess;
    if (a.M <= 1) return launch_m_narrow<1>(a, stream, err) ? err : launch_mb<1>(a, stream);
    if (a.M <= 2) return launch_m_narrow<2>(a, stream, err) ? err : launch_mb<2>(a, stream);
    if (a.M <= 4) return launch_m_narrow<4>(a, stream, err) ? err : launch_mb<4>(a, stream);
    if (a.M <= 8) return launch_m_narrow<8>(a, stream, err) ? err : launch_mb<8>(a, stream);
    {
        // 9 to 16 rows on the matrix cores where the loads are aligned: 64
        // columns per workgroup, or 32 or 16 where that keeps clearly more
        // CUs busy within one round (the wider on a tie)
        const long long cus = a.cus > 0 ? a.cus : 256;
        const long long b64 = ((long long)a.N + 63) / 64, b32 = ((long long)a.N + 31) / 32;
        const long long b16 = ((long long)a.N + 15) / 16;
        const double f1 = sk_fill(b64, cus);
        const double f2 = b32 <= cus ? sk_fill(b32, cus) : 0.0, f4 = b16 <= cus ? sk_fill(b16, cus) : 0.0;
        int nj = f2 >= f4 && f2 >= f1 + 0.15 ? 2 : f4 > f2 && f4 >= f1 + 0.15 ? 1 : 4;
        // a narrower workgroup walks more k per iteration (128 / nj): wider
        // ones where K would leave a quarter of the 16 waves without one
        // (12 x 4096 x 1000: 8.8 TFLOP/s at 16 columns, 16.4 at 32)
        while (nj < 4 && a.K < 12 * 128 / nj) nj *= 2;
        // B's rows not aligned to its groups: each lane reads its columns
        // one float at a time.  Its four loads then touch the same lines,
        // which the caches must hold between them, so a B streamed past the
        // last-level cache stays with the vector-ALU kernels (16 x 65535 x
        // 8192: 18.4 TFLOP/s this way, 34.0 there; 16 x 8191 x 8192, not
        // streamed: 29.8 against 20.1).
        if (nj == 1 || m_mfma_b_fits(a, nj) || !b_streams(a)) {
            if (nj == 4) return launch_m_mfma<64>(a, stream);
            if (nj == 2) return launch_m_mfma<32>(a, stream);
            return launch_m_mfma<16>(a, stream);
        }
    }
    if (launch_m_narrow<16>(a, stream, err)) return err;
    const long long blocks = ((long long)a.N + SK_COLS - 1) / SK_COLS;
    if (b_streams(a))
        hipLaunchKernelGGL(skinny_m16_kernel<true>, dim3((unsigned)blocks), dim3(64 * SK_WAVES), 0, stream, a);
    else
        hipLaunchKernelGGL(skinny_m16_kernel<false>, dim3((unsigned)blocks), dim3(64 * SK_WAVES), 0, stream, a);
    return hipGetLastError();
}

}  // namespace sgemm
