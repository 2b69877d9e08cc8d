// sgemm_mfma.hip -- fp32 C = A.B on the CDNA4 matrix cores.
//
// Same hierarchy as the register/LDS-tiled method ("Register/Shared Memory
// Tiling", ryotta.opik.net: outer-product GEMM, cooperative tile loading,
// double buffering; "gemm_tiled_test", teach-meaning.tistory.com/1542,
// sections 1-6): a workgroup owns a BM x BN tile of C, walks K in BK-deep
// slabs staged through LDS, and keeps the tile in registers until one final
// store.  The step that differs is the innermost one: instead of each lane
// doing a TM x TN scalar outer product, each wave owns a WM x WN sub-tile
// ("warp tile", "누산 개념을 Grid-Block-Warp-Thread 계층에 끼워넣기",
// teach-meaning.tistory.com/1518, section 2) held as (WM/32) x (WN/32)
// accumulator blocks of v_mfma_f32_32x32x2_f32.  One such instruction is a
// rank-2 update of a 32x32 block (2048 fused multiply-adds, fp32 in and out):
// the same outer-product accumulation, done by the matrix core for the whole
// wave.  The pages note that the tiling maps onto matrix instructions
// (page 4, advantages, item 3).
//
// Operand layouts of v_mfma_f32_32x32x2_f32 (wave64, one VGPR per operand):
//   A (32 x 2): lane l holds A[l % 32][l / 32]
//   B (2 x 32): lane l holds B[l / 32][l % 32]
//   D (32 x 32, 16 VGPRs): register r of lane l holds
//       D[8*(r/4) + 4*(l/32) + r%4][l % 32]
// Because the order of the k terms does not change the sum's value (only its
// rounding), the BK values of a slab are split between the two lane halves:
// MFMA step s feeds lane half h with k = h*(BK/2) + s.  A lane therefore
// reads BK/2 consecutive k of one A row (float4 LDS reads) and BK/2 rows of
// one B column.
//
// LDS (per stage): As[BM][BK+4] (rows of A, k contiguous) and Bs[BK][BN+4]
// (rows of B, n contiguous).  The +4 float pads make the A float4 reads of a
// wave and the B column reads of both lane halves fall in distinct banks.
//
// Loader: every thread moves float4s from global memory into registers for
// slab t+1 before computing slab t, then writes them to the other LDS stage
// after; one barrier per slab.  Rows past M, columns past N and k past K are
// loaded as zero, so partial tiles compute the same sums as full ones and
// the store is guarded by row < M && col < N ("gemm_tiled_test" section 3,
// zero-padding after the boundary check).
#include "tiles.h"

namespace sgemm {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));

template <int BM, int BN, int BK, int WM, int WN>
struct MfmaCfg {
    static constexpr int WAVES_M = BM / WM;
    static constexpr int WAVES_N = BN / WN;
    static constexpr int NT = WAVES_M * WAVES_N * 64;  // threads per workgroup
    static constexpr int FM = WM / 32;                  // 32x32 blocks per wave, M
    static constexpr int FN = WN / 32;                  // 32x32 blocks per wave, N
    static constexpr int KH = BK / 2;                   // k per lane half per slab
    static constexpr int SA = BK + 4;                   // LDS row of A (floats)
    static constexpr int SB = BN + 4;                   // LDS row of B (floats)
    static constexpr int A_F4 = BM * BK / 4 / NT;       // float4 of A per thread
    static constexpr int B_F4 = BK * BN / 4 / NT;       // float4 of B per thread
    static constexpr int LDS_FLOATS = 2 * (BM * SA + BK * SB);
    static_assert(BM % WM == 0 && BN % WN == 0, "wave tiles must tile the block");
    static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile is whole 32x32 blocks");
    static_assert(BK % 8 == 0, "BK/2 must be a multiple of 4 (float4 A reads)");
    static_assert((BM * BK / 4) % NT == 0 && (BK * BN / 4) % NT == 0,
                  "loader float4s must divide evenly over the threads");
    static_assert(LDS_FLOATS * 4 <= 160 * 1024, "LDS budget of one CU");
};

constexpr int GROUP_M = 8;

template <int BM, int BN, int BK, int WM, int WN, bool VA, bool VB>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64, 2)
void sgemm_mfma_kernel(GemmArgs p, int tiles_m, int tiles_n) {
    using Cfg = MfmaCfg<BM, BN, BK, WM, WN>;
    constexpr int NT = Cfg::NT, FM = Cfg::FM, FN = Cfg::FN, KH = Cfg::KH;
    constexpr int SA = Cfg::SA, SB = Cfg::SB;
    __shared__ __attribute__((aligned(16))) float As[2][BM * SA];
    __shared__ __attribute__((aligned(16))) float Bs[2][BK * SB];

    int tm, tn;
    tile_coords(blockIdx.x, tiles_m, tiles_n, GROUP_M, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int M = p.M, N = p.N, K = p.K;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = (wave / Cfg::WAVES_N) * WM;
    const int wn = (wave % Cfg::WAVES_N) * WN;
    const int li = lane & 31, lh = lane >> 5;

    // Per-thread loader coordinates inside the tile (fixed over the K loop).
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
    const int mrem = M - m0, nrem = N - n0;   // rows/cols of this tile inside C
    const bool m_full = mrem >= BM, n_full = nrem >= BN;

    float4 ra[Cfg::A_F4], rb[Cfg::B_F4];
    auto load_slab = [&](int k0) {
        const bool k_full = (K - k0) >= BK;
#pragma unroll
        for (int i = 0; i < Cfg::A_F4; ++i)
            ra[i] = load4<VA>(Ablk + k0, p.lda, a_row[i], a_col[i], mrem, K - k0,
                              m_full && k_full);
#pragma unroll
        for (int i = 0; i < Cfg::B_F4; ++i)
            rb[i] = load4<VB>(Bblk + (long long)k0 * p.ldb, p.ldb, b_row[i], b_col[i],
                              K - k0, nrem, n_full && k_full);
    };
    auto store_slab = [&](int st) {
#pragma unroll
        for (int i = 0; i < Cfg::A_F4; ++i)
            *reinterpret_cast<float4*>(&As[st][a_row[i] * SA + a_col[i]]) = ra[i];
#pragma unroll
        for (int i = 0; i < Cfg::B_F4; ++i)
            *reinterpret_cast<float4*>(&Bs[st][b_row[i] * SB + b_col[i]]) = rb[i];
    };

    floatx16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int nslab = (K + BK - 1) / BK;
    if (nslab > 0) {
        load_slab(0);
        store_slab(0);
        __syncthreads();
    }
    for (int t = 0; t < nslab; ++t) {
        const int cur = t & 1;
        if (t + 1 < nslab) load_slab((t + 1) * BK);

        float a[FM][KH], b[FN][KH];
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const float* src = &As[cur][(wm + i * 32 + li) * SA + lh * KH];
#pragma unroll
            for (int q = 0; q < KH / 4; ++q) {
                const float4 v = *reinterpret_cast<const float4*>(src + 4 * q);
                a[i][4 * q + 0] = v.x; a[i][4 * q + 1] = v.y;
                a[i][4 * q + 2] = v.z; a[i][4 * q + 3] = v.w;
            }
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const float* src = &Bs[cur][(lh * KH) * SB + wn + j * 32 + li];
#pragma unroll
            for (int s = 0; s < KH; ++s) b[j][s] = src[s * SB];
        }
#pragma unroll
        for (int s = 0; s < KH; ++s)
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i][s], b[j][s],
                                                                     acc[i][j], 0, 0, 0);

        if (t + 1 < nslab) store_slab(cur ^ 1);
        __syncthreads();
    }

    // Epilogue: plain guarded store of the register tile.
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int col = n0 + wn + j * 32 + li;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + wm + i * 32 + 8 * (r / 4) + 4 * lh + (r % 4);
                if (row < M && col < N) p.C[(long long)row * p.ldc + col] = acc[i][j][r];
            }
        }
    }
}

template <int BM, int BN, int BK, int WM, int WN>
hipError_t launch_cfg(const GemmArgs& a, hipStream_t stream) {
    using Cfg = MfmaCfg<BM, BN, BK, WM, WN>;
    const int tiles_m = (a.M + BM - 1) / BM;
    const int tiles_n = (a.N + BN - 1) / BN;
    const dim3 grid((unsigned)(tiles_m * tiles_n)), block(Cfg::NT);
    const bool va = (a.lda % 4 == 0) && ((reinterpret_cast<uintptr_t>(a.A) & 15) == 0);
    const bool vb = (a.ldb % 4 == 0) && ((reinterpret_cast<uintptr_t>(a.B) & 15) == 0);
    if (va && vb)
        hipLaunchKernelGGL((sgemm_mfma_kernel<BM, BN, BK, WM, WN, true, true>), grid, block, 0, stream, a, tiles_m, tiles_n);
    else if (va)
        hipLaunchKernelGGL((sgemm_mfma_kernel<BM, BN, BK, WM, WN, true, false>), grid, block, 0, stream, a, tiles_m, tiles_n);
    else if (vb)
        hipLaunchKernelGGL((sgemm_mfma_kernel<BM, BN, BK, WM, WN, false, true>), grid, block, 0, stream, a, tiles_m, tiles_n);
    else
        hipLaunchKernelGGL((sgemm_mfma_kernel<BM, BN, BK, WM, WN, false, false>), grid, block, 0, stream, a, tiles_m, tiles_n);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_mfma(const GemmArgs& a, hipStream_t stream) {
    return launch_cfg<128, 128, 16, 64, 64>(a, stream);
}

}  // namespace sgemm
