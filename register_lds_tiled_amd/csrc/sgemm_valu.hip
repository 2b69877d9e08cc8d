// sgemm_valu.hip -- fp32 C = A.B with per-lane register tiles on the vector ALU.
//
// The register/shared-memory tiled GEMM as the pages lay it out, level by
// level:
//  * grid -> block tile: workgroup (tile_m, tile_n) owns
//    C[m0:m0+BM, n0:n0+BN]; one launch covers all of C
//    ("누산 개념을 Grid-Block-Warp-Thread 계층에 끼워넣기",
//    teach-meaning.tistory.com/1518, sections 1 and 2(1); "gemm_tiled_test",
//    teach-meaning.tistory.com/1542, section 1);
//  * block tile -> wave tile: the block's waves form a WAVES_M x WAVES_N grid,
//    wave (wr, wc) owning the WM x WN sub-tile at (wr WM, wc WN) -- the warp
//    tile of the hierarchy page, section 2(2), sized for 64-lane waves;
//  * wave tile -> lane tile: the wave's 64 lanes form an LM x LN grid and
//    each lane owns TM x TN outputs of the wave tile in registers (the
//    thread tile, section 2(3); MR x NR of "Micro Kernel 입문하기",
//    teach-meaning.tistory.com/1544, section 4);
//  * K walked in BK-deep slabs; the block's A slab (BM x BK) and B slab
//    (BK x BN) are loaded cooperatively by all threads into LDS, with zero
//    fill outside the matrix ("gemm_tiled_test" sections 2-4; "Register/Shared
//    Memory Tiling", ryotta.opik.net, tile-loading section);
//  * for every k of the slab a lane loads TM values of A's column and TN
//    values of B's row and does the TM x TN rank-1 update with fused
//    multiply-adds ("gemm_tiled_test" section 5; page 4 outer-product GEMM
//    and register-level detail; the one-thread 4x4 case is the micro-kernel
//    page's section 2);
//  * optional double buffering: STAGES = 2 computes on one LDS stage while
//    the next slab is in flight (page 4, double-buffering sections);
//  * plain guarded store at the end ("gemm_tiled_test" section 6).
//
// gfx950 choices (not on the pages):
//  * A is written to LDS transposed, k-major (As[k][m]), so a lane's TM
//    A values for one k are contiguous and come in float4 reads, as B's are.
//  * A lane's TM rows are TM/4 groups of 4 rows spread 4 LM apart inside the
//    wave tile (and likewise its TN columns, 4 LN apart), so the float4 reads
//    of neighbouring lanes hit consecutive 16-byte words: lanes of one lane
//    row read the same A word (a broadcast) and consecutive B words, with no
//    LDS bank conflicts.
//  * LDS rows are padded by 4 floats.
//  * Double buffering stages the next slab in registers: global loads for
//    slab t+1 are issued before the FMAs of slab t and written to the other
//    LDS stage afterwards, so one barrier per slab suffices.
//  * The FMAs are scalar v_fma_f32 (this library is built with packed fp32
//    disabled).
//
// Each lane's sum runs over k in ascending order with one fused multiply-add
// per k, whatever the tile configuration: every configuration gives the same
// bits.
#include <cstdint>

#include "tiles.h"

namespace sgemm {
namespace {

template <int BM_, int BN_, int BK_, int WM_, int WN_, int TM_, int TN_, int STAGES_,
          int MINW_ = 2, int KU_ = 8>
struct ValuCfg {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, TM = TM_, TN = TN_;
    static constexpr int WM = WM_, WN = WN_;
    static constexpr int STAGES = STAGES_;
    static constexpr int MINW = MINW_;                  // min waves per SIMD (launch bounds)
    static constexpr int KU = KU_;                      // unroll of the k loop over a slab
    static constexpr int WAVES_M = BM / WM, WAVES_N = BN / WN;
    static constexpr int NW = WAVES_M * WAVES_N;        // waves per workgroup
    static constexpr int NT = 64 * NW;                  // threads per workgroup
    static constexpr int LM = WM / TM, LN = WN / TN;    // lane grid of a wave tile
    static constexpr int GM = TM / 4, GN = TN / 4;
    static constexpr int SA = BM + 4;           // LDS row (one k) of A^T
    static constexpr int SB = BN + 4;           // LDS row (one k) of B
    static constexpr int A_TOT = BM * BK / 4;          // float4 of A per slab
    static constexpr int B_TOT = BK * BN / 4;          // float4 of B per slab
    static constexpr int A_F4 = (A_TOT + NT - 1) / NT;
    static constexpr int B_F4 = (B_TOT + NT - 1) / NT;
    static_assert(BM % WM == 0 && BN % WN == 0, "whole wave tiles");
    static_assert(WM % TM == 0 && WN % TN == 0 && LM * LN == 64, "64 lanes per wave tile");
    static_assert(TM % 4 == 0 && TN % 4 == 0, "register tile is whole float4 groups");
    static_assert(BK % 4 == 0, "BK multiple of 4");
    static_assert(A_TOT % NT == 0 || A_TOT < NT, "A float4s spread evenly or one each");
    static_assert(B_TOT % NT == 0 || B_TOT < NT, "B float4s spread evenly or one each");
    static_assert(STAGES == 1 || STAGES == 2, "one or two LDS stages");
    static_assert(STAGES * BK * (SA + SB) * 4 <= 64 * 1024, "static LDS of one workgroup");
};

constexpr int GROUP_M = 8;

template <class Cfg, bool VA, bool VB>
__global__ __launch_bounds__(Cfg::NT, Cfg::MINW)
void sgemm_valu_kernel(GemmArgs p, int tiles_m, int tiles_n) {
    constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK, TM = Cfg::TM, TN = Cfg::TN;
    constexpr int STAGES = Cfg::STAGES, NT = Cfg::NT;
    constexpr int LM = Cfg::LM, LN = Cfg::LN;
    constexpr int GM = Cfg::GM, GN = Cfg::GN, SA = Cfg::SA, SB = Cfg::SB;
    __shared__ __attribute__((aligned(16))) float As[STAGES][BK * SA];
    __shared__ __attribute__((aligned(16))) float Bs[STAGES][BK * SB];

    int tm, tn;
    tile_coords(blockIdx.x, tiles_m, tiles_n, GROUP_M, p.xcds, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int M = p.M, N = p.N, K = p.K;
    const int tid = threadIdx.x;
    // wave tile (wm, wn) in the block; lane (lr, lc) in the wave tile
    const int wave = tid >> 6, lane = tid & 63;
    const int wm = (wave / Cfg::WAVES_N) * Cfg::WM, wn = (wave % Cfg::WAVES_N) * Cfg::WN;
    const int lr = lane / LN, lc = lane % LN;
    const int arow = wm + 4 * lr, bcol = wn + 4 * lc;   // first row / column of the lane

    int a_row[Cfg::A_F4], a_col[Cfg::A_F4], b_row[Cfg::B_F4], b_col[Cfg::B_F4];
#pragma unroll
    for (int i = 0; i < Cfg::A_F4; ++i) {
        const int idx = tid + i * NT;
        a_row[i] = idx / (BK / 4);
        a_col[i] = (idx % (BK / 4)) * 4;
    }
#pragma unroll
    for (int i = 0; i < Cfg::B_F4; ++i) {
        const int idx = tid + i * NT;
        b_row[i] = idx / (BN / 4);
        b_col[i] = (idx % (BN / 4)) * 4;
    }
    const float* __restrict__ Ablk = p.A + (long long)m0 * p.lda;
    const float* __restrict__ Bblk = p.B + n0;
    const int mrem = M - m0, nrem = N - n0;
    const bool m_full = mrem >= BM, n_full = nrem >= BN;

    float4 ra[Cfg::A_F4], rb[Cfg::B_F4];
    auto load_slab = [&](int k0) {
        const bool k_full = (K - k0) >= BK;
#pragma unroll
        for (int i = 0; i < Cfg::A_F4; ++i)
            if (Cfg::A_TOT >= NT || tid < Cfg::A_TOT)
                ra[i] = load4<VA>(Ablk + k0, p.lda, a_row[i], a_col[i], mrem, K - k0,
                                  m_full && k_full);
#pragma unroll
        for (int i = 0; i < Cfg::B_F4; ++i)
            if (Cfg::B_TOT >= NT || tid < Cfg::B_TOT)
                rb[i] = load4<VB>(Bblk + (long long)k0 * p.ldb, p.ldb, b_row[i], b_col[i],
                                  K - k0, nrem, n_full && k_full);
    };
    auto store_slab = [&](int st) {
#pragma unroll
        for (int i = 0; i < Cfg::A_F4; ++i) {   // transpose: A[m][k] -> As[k][m]
            if (Cfg::A_TOT < NT && tid >= Cfg::A_TOT) continue;
            float* d = &As[st][a_col[i] * SA + a_row[i]];
            d[0] = ra[i].x; d[SA] = ra[i].y; d[2 * SA] = ra[i].z; d[3 * SA] = ra[i].w;
        }
#pragma unroll
        for (int i = 0; i < Cfg::B_F4; ++i)
            if (Cfg::B_TOT >= NT || tid < Cfg::B_TOT)
                *reinterpret_cast<float4*>(&Bs[st][b_row[i] * SB + b_col[i]]) = rb[i];
    };

    // debug build: the words store_slab(st) is about to write
    auto poison_slab = [&](int st) {
#pragma unroll
        for (int i = 0; i < Cfg::A_F4; ++i) {
            if (Cfg::A_TOT < NT && tid >= Cfg::A_TOT) continue;
#pragma unroll
            for (int e = 0; e < 4; ++e) lds_poison_f1(&As[st][(a_col[i] + e) * SA + a_row[i]]);
        }
#pragma unroll
        for (int i = 0; i < Cfg::B_F4; ++i)
            if (Cfg::B_TOT >= NT || tid < Cfg::B_TOT) lds_poison_f4(&Bs[st][b_row[i] * SB + b_col[i]]);
    };

    float acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = 0.f;

    // Unrolling the k loop by KU (the micro-kernel page's unroll knob) lets
    // the LDS reads of the next k overlap the FMAs of this one; unrolling the
    // whole slab makes the compiler hoist every read and spill.
    auto compute = [&](int st) {
#pragma unroll Cfg::KU
        for (int kk = 0; kk < BK; ++kk) {
            float a[TM], b[TN];
#pragma unroll
            for (int g = 0; g < GM; ++g) {
                const float4 v = *reinterpret_cast<const float4*>(
                    &As[st][kk * SA + arow + g * 4 * LM]);
                a[4 * g + 0] = v.x; a[4 * g + 1] = v.y; a[4 * g + 2] = v.z; a[4 * g + 3] = v.w;
            }
#pragma unroll
            for (int g = 0; g < GN; ++g) {
                const float4 v = *reinterpret_cast<const float4*>(
                    &Bs[st][kk * SB + bcol + g * 4 * LN]);
                b[4 * g + 0] = v.x; b[4 * g + 1] = v.y; b[4 * g + 2] = v.z; b[4 * g + 3] = v.w;
            }
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
        }
    };

    const int nslab = (K + BK - 1) / BK;
    if constexpr (STAGES == 2) {
        if (nslab > 0) {
            load_slab(0);
            store_slab(0);
            __syncthreads();
        }
        for (int t = 0; t < nslab; ++t) {
            const int cur = t & 1;
            // (the barrier ending iteration t - 1 retired stage cur ^ 1)
            if (kLdsPoison && t + 1 < nslab) poison_slab(cur ^ 1);
            if (t + 1 < nslab) load_slab((t + 1) * BK);
            compute(cur);
            if (t + 1 < nslab) store_slab(cur ^ 1);
            __syncthreads();
        }
    } else {
        // Single LDS stage, as the tiled page's test kernel runs: load,
        // barrier, compute, barrier.
        for (int t = 0; t < nslab; ++t) {
            if (kLdsPoison) poison_slab(0);
            load_slab(t * BK);
            store_slab(0);
            __syncthreads();
            compute(0);
            __syncthreads();
        }
    }

    // Epilogue: lane rows m0 + arow + 4 LM gi + (0..3), columns
    // n0 + bcol + 4 LN gj + (0..3).
    const bool vec_c = ((p.ldc & 3) == 0) && ((reinterpret_cast<uintptr_t>(p.C) & 15) == 0);
#pragma unroll
    for (int gi = 0; gi < GM; ++gi) {
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            const int i = 4 * gi + ii;
            const int row = m0 + arow + gi * 4 * LM + ii;
            if (row >= M) continue;
            float* crow = p.C + (long long)row * p.ldc;
#pragma unroll
            for (int gj = 0; gj < GN; ++gj) {
                const int col = n0 + bcol + gj * 4 * LN;
                const int j = 4 * gj;
                if (vec_c && col + 3 < N) {
                    store_c4(crow + col, acc[i][j], acc[i][j + 1], acc[i][j + 2], acc[i][j + 3]);
                } else {
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj)
                        if (col + jj < N) store_c(crow + col + jj, acc[i][j + jj]);
                }
            }
        }
    }
}

template <class Cfg>
hipError_t launch_cfg(const GemmArgs& a, hipStream_t stream) {
    constexpr int BM = Cfg::BM, BN = Cfg::BN;
    const int tiles_m = (a.M + BM - 1) / BM;
    const int tiles_n = (a.N + BN - 1) / BN;
    const dim3 grid((unsigned)(tiles_m * tiles_n)), block(Cfg::NT);
    const bool va = (a.lda % 4 == 0) && ((reinterpret_cast<uintptr_t>(a.A) & 15) == 0);
    const bool vb = (a.ldb % 4 == 0) && ((reinterpret_cast<uintptr_t>(a.B) & 15) == 0);
    if (va && vb)
        hipLaunchKernelGGL((sgemm_valu_kernel<Cfg, true, true>), grid, block, 0, stream, a, tiles_m, tiles_n);
    else if (va)
        hipLaunchKernelGGL((sgemm_valu_kernel<Cfg, true, false>), grid, block, 0, stream, a, tiles_m, tiles_n);
    else if (vb)
        hipLaunchKernelGGL((sgemm_valu_kernel<Cfg, false, true>), grid, block, 0, stream, a, tiles_m, tiles_n);
    else
        hipLaunchKernelGGL((sgemm_valu_kernel<Cfg, false, false>), grid, block, 0, stream, a, tiles_m, tiles_n);
    return hipGetLastError();
}

// The built VALU tile configurations: block BM x BN x BK, waves of WM x WN,
// lanes of TM x TN (MR x NR), LDS stages.  They span the register tiles
// the micro-kernel page plans to compare (4x4, 8x4, 16x8; section 4 items 2
// and 4) plus the tiled page's 16x4 and the square and wide 8x8 / 8x16, at
// several block sizes, wave counts and slab depths.
using V0 = ValuCfg<128, 128, 16, 64, 64, 8, 8, 2, 3>;     // 4 waves, 8x8
using V1 = ValuCfg<64, 64, 16, 32, 32, 4, 4, 2, 4>;       // 4 waves, 4x4
using V2 = ValuCfg<128, 64, 16, 64, 32, 8, 4, 2, 4>;      // 4 waves, 8x4
using V3 = ValuCfg<128, 128, 16, 64, 64, 16, 4, 2, 3>;    // 4 waves, 16x4
using V4 = ValuCfg<256, 128, 16, 128, 64, 16, 8, 2, 2>;   // 4 waves, 16x8
using V5 = ValuCfg<128, 128, 16, 64, 32, 8, 4, 2, 4>;     // 8 waves, 8x4
using V6 = ValuCfg<64, 128, 16, 64, 64, 8, 8, 2, 3>;      // 2 waves, 8x8
using V7 = ValuCfg<128, 256, 16, 64, 128, 8, 16, 2, 2>;   // 4 waves, 8x16
using V8 = ValuCfg<64, 64, 16, 64, 64, 16, 4, 1, 1, 16>;  // the tiled page's kernel
using V9 = ValuCfg<128, 64, 16, 64, 64, 8, 8, 2, 3>;      // 2 waves, 8x8
using V10 = ValuCfg<64, 64, 16, 32, 64, 8, 4, 2, 4>;      // 2 waves, 8x4
using V11 = ValuCfg<64, 64, 32, 32, 32, 4, 4, 2, 4>;      // 4 waves, 4x4, 32-k slabs
using V12 = ValuCfg<128, 64, 16, 32, 32, 4, 4, 2, 2>;     // 8 waves, 4x4
using V13 = ValuCfg<64, 128, 16, 32, 32, 4, 4, 2, 2>;     // 8 waves, 4x4
using V14 = ValuCfg<64, 64, 16, 64, 32, 8, 4, 2, 4>;      // 2 waves, 8x4 (64-row waves)

struct TileInfo {
    const char* name;
    hipError_t (*launch)(const GemmArgs&, hipStream_t);
};

const TileInfo kTiles[] = {
    {"128x128x16 waves 2x2 of 64x64 lanes 8x8 of 8x8 stages 2", launch_cfg<V0>},
    {"64x64x16 waves 2x2 of 32x32 lanes 8x8 of 4x4 stages 2", launch_cfg<V1>},
    {"128x64x16 waves 2x2 of 64x32 lanes 8x8 of 8x4 stages 2", launch_cfg<V2>},
    {"128x128x16 waves 2x2 of 64x64 lanes 4x16 of 16x4 stages 2", launch_cfg<V3>},
    {"256x128x16 waves 2x2 of 128x64 lanes 8x8 of 16x8 stages 2", launch_cfg<V4>},
    {"128x128x16 waves 2x4 of 64x32 lanes 8x8 of 8x4 stages 2", launch_cfg<V5>},
    {"64x128x16 waves 1x2 of 64x64 lanes 8x8 of 8x8 stages 2", launch_cfg<V6>},
    {"128x256x16 waves 2x2 of 64x128 lanes 8x8 of 8x16 stages 2", launch_cfg<V7>},
    {"64x64x16 waves 1x1 of 64x64 lanes 4x16 of 16x4 stages 1", launch_cfg<V8>},
    {"128x64x16 waves 2x1 of 64x64 lanes 8x8 of 8x8 stages 2", launch_cfg<V9>},
    {"64x64x16 waves 2x1 of 32x64 lanes 4x16 of 8x4 stages 2", launch_cfg<V10>},
    {"64x64x32 waves 2x2 of 32x32 lanes 8x8 of 4x4 stages 2", launch_cfg<V11>},
    {"128x64x16 waves 4x2 of 32x32 lanes 8x8 of 4x4 stages 2", launch_cfg<V12>},
    {"64x128x16 waves 2x4 of 32x32 lanes 8x8 of 4x4 stages 2", launch_cfg<V13>},
    {"64x64x16 waves 1x2 of 64x32 lanes 8x8 of 8x4 stages 2", launch_cfg<V14>},
};
constexpr int kNumTiles = sizeof(kTiles) / sizeof(kTiles[0]);

}  // namespace

int valu_tile_count() { return kNumTiles; }

const char* valu_tile_name(int tile) {
    return tile >= 0 && tile < kNumTiles ? kTiles[tile].name : nullptr;
}

hipError_t launch_valu_tile(const GemmArgs& a, int tile, hipStream_t stream) {
    if (tile < 0 || tile >= kNumTiles) return hipErrorInvalidValue;
    return kTiles[tile].launch(a, stream);
}

// Tuned VALU path, from interleaved sweeps of every configuration on
// MI355X (median GFLOP/s): 128x128 blocks of 4 waves of 64x64 with 8x8 per
// lane where the grid has at least 4 such tiles per CU (8192^3 87,050;
// 4096^3 85,610: then up to 4 workgroups share a CU and hide each other's
// waits), else 64x64 blocks of 4 waves of 32x32 with 4x4 per lane, whose
// grid is four times larger (3072^3 73,890 against 65,705; 2048^3 71,665
// against 41,640), with 32-k slabs (half the barriers) where even the
// 128x128 grid would leave CUs idle (1536^3 53,226 against 51,612 for 16-k
// slabs; 1024^3 35,239 against 34,130; 1000x1500x777 39,474 against
// 37,299; at 3072^3 the 16-k slabs lead, 71,946 against 70,999).
hipError_t launch_valu(const GemmArgs& a, hipStream_t stream) {
    const long long t128 = ((long long)a.M + 127) / 128 * (((long long)a.N + 127) / 128);
    if (t128 >= 4LL * a.cus) return launch_cfg<V0>(a, stream);
    if (t128 < a.cus) return launch_cfg<V11>(a, stream);
    return launch_cfg<V1>(a, stream);
}

// The tiled page's measured geometry ("gemm_tiled_test" section 7): BM=BN=64,
// BK=16, 64 threads (16 x 4), 16 x 4 outputs per thread, one LDS stage.
hipError_t launch_valu_page(const GemmArgs& a, hipStream_t stream) {
    return launch_cfg<V8>(a, stream);
}

}  // namespace sgemm
