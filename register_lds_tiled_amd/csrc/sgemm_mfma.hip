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

template <int BM_, int BN_, int BK_, int WM_, int WN_, int MINW_ = 2, int GROUP_M_ = 8,
          bool XCD_ = true, int PADB_ = 4, int P_ = 1, bool PF_ = false>
struct MfmaCfg {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_;
    static constexpr int P = P_;                         // slabs in flight in registers
    static constexpr bool PF = PF_;                      // 3 LDS stages + fragment prefetch
    static constexpr int STAGES = PF ? 3 : 2;            // LDS stages
    static constexpr int MINW = MINW_;                   // min waves per SIMD (launch bounds)
    static constexpr int GROUP_M = GROUP_M_;             // tile rows per raster group
    static constexpr bool XCD = XCD_;                    // XCD-aware workgroup remap
    static constexpr int WAVES_M = BM / WM;
    static constexpr int WAVES_N = BN / WN;
    static constexpr int NT = WAVES_M * WAVES_N * 64;  // threads per workgroup
    static constexpr int FM = WM / 32;                  // 32x32 blocks per wave, M
    static constexpr int FN = WN / 32;                  // 32x32 blocks per wave, N
    static constexpr int KH = BK / 2;                   // k per lane half per slab
    static constexpr int SA = BK + 4;                   // LDS row of A (floats)
    static constexpr int SB = BN + PADB_;               // LDS row of B (floats)
    static constexpr int A_TOT = BM * BK / 4;           // float4 of A per slab
    static constexpr int B_TOT = BK * BN / 4;           // float4 of B per slab
    static constexpr int A_F4 = (A_TOT + NT - 1) / NT;  // float4 of A per thread
    static constexpr int B_F4 = (B_TOT + NT - 1) / NT;  // float4 of B per thread
    static constexpr int LDS_FLOATS = STAGES * (BM * SA + BK * SB);
    static_assert(BM % WM == 0 && BN % WN == 0, "wave tiles must tile the block");
    static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile is whole 32x32 blocks");
    static_assert(BK % 8 == 0, "BK/2 must be a multiple of 4 (float4 A reads)");
    static_assert(A_TOT % NT == 0 || A_TOT < NT, "A float4s spread evenly or one each");
    static_assert(B_TOT % NT == 0 || B_TOT < NT, "B float4s spread evenly or one each");
    static_assert(LDS_FLOATS * 4 <= 160 * 1024, "LDS budget of one CU");
    static_assert(PADB_ % 2 == 0, "B rows stay 8-byte aligned");
    static_assert(!PF || P == 1, "fragment prefetch runs with one register staging set");
};

template <class Cfg, bool VA, bool VB>
__global__ __launch_bounds__(Cfg::NT, Cfg::MINW)
void sgemm_mfma_kernel(GemmArgs p, int tiles_m, int tiles_n) {
    constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK, WM = Cfg::WM, WN = Cfg::WN;
    constexpr int NT = Cfg::NT, FM = Cfg::FM, FN = Cfg::FN, KH = Cfg::KH;
    constexpr int SA = Cfg::SA, SB = Cfg::SB;
    __shared__ __attribute__((aligned(16))) float As[Cfg::STAGES][BM * SA];
    __shared__ __attribute__((aligned(16))) float Bs[Cfg::STAGES][BK * SB];

    int tm, tn;
    tile_coords(blockIdx.x, tiles_m, tiles_n, Cfg::GROUP_M, Cfg::XCD, tm, tn);
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

    using RegA = float4[Cfg::A_F4];
    using RegB = float4[Cfg::B_F4];
    auto load_slab = [&](int k0, RegA& ra, RegB& rb) {
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
    auto store_slab = [&](int st, const RegA& ra, const RegB& rb) {
#pragma unroll
        for (int i = 0; i < Cfg::A_F4; ++i)
            if (Cfg::A_TOT >= NT || tid < Cfg::A_TOT)
                *reinterpret_cast<float4*>(&As[st][a_row[i] * SA + a_col[i]]) = ra[i];
#pragma unroll
        for (int i = 0; i < Cfg::B_F4; ++i) {
            if (Cfg::B_TOT < NT && tid >= Cfg::B_TOT) continue;
            float* d = &Bs[st][b_row[i] * SB + b_col[i]];
            if constexpr (SB % 4 == 0) {
                *reinterpret_cast<float4*>(d) = rb[i];
            } else {   // rows only 8-byte aligned
                d[0] = rb[i].x; d[1] = rb[i].y; d[2] = rb[i].z; d[3] = rb[i].w;
            }
        }
    };

    floatx16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // One slab: each wave reads its A rows (float4) and B columns from LDS
    // stage st into registers, then applies BK/2 rank-2 MFMA updates to each
    // accumulator block.
    struct Frag {
        float a[FM][KH], b[FN][KH];
    };
    auto read_frags = [&](int st, Frag& f) {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const float* src = &As[st][(wm + i * 32 + li) * SA + lh * KH];
#pragma unroll
            for (int q = 0; q < KH / 4; ++q) {
                const float4 v = *reinterpret_cast<const float4*>(src + 4 * q);
                f.a[i][4 * q + 0] = v.x; f.a[i][4 * q + 1] = v.y;
                f.a[i][4 * q + 2] = v.z; f.a[i][4 * q + 3] = v.w;
            }
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const float* src = &Bs[st][(lh * KH) * SB + wn + j * 32 + li];
#pragma unroll
            for (int s = 0; s < KH; ++s) f.b[j][s] = src[s * SB];
        }
    };
    auto mma = [&](const Frag& f) {
#pragma unroll
        for (int s = 0; s < KH; ++s)
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(f.a[i][s], f.b[j][s],
                                                                     acc[i][j], 0, 0, 0);
    };

    constexpr int P = Cfg::P;
    float4 ra[P][Cfg::A_F4], rb[P][Cfg::B_F4];
    const int nslab = (K + BK - 1) / BK;
    if constexpr (!Cfg::PF) {
        // Two LDS stages.  Slab s is staged in register set s % P, written to
        // LDS stage s % 2 at the end of iteration s - 1 and computed in
        // iteration s.  The global loads of slab t + P are issued at the start
        // of iteration t into the set slab t has left, so each load has P
        // slabs of compute to land.  One barrier per slab orders this
        // iteration's LDS writes before the next iteration's reads, and this
        // iteration's reads of stage t % 2 before iteration t + 1 writes it.
        if (nslab > 0) {
            load_slab(0, ra[0], rb[0]);
            store_slab(0, ra[0], rb[0]);
#pragma unroll
            for (int q = 1; q < P; ++q)
                if (q < nslab) load_slab(q * BK, ra[q], rb[q]);
            __syncthreads();
        }
        for (int t0 = 0; t0 < nslab; t0 += P) {
#pragma unroll
            for (int u = 0; u < P; ++u) {
                const int t = t0 + u;
                if (t >= nslab) break;
                if (t + P < nslab) load_slab((t + P) * BK, ra[u], rb[u]);
                Frag f;
                read_frags(t & 1, f);
                mma(f);
                if (t + 1 < nslab) store_slab((t + 1) & 1, ra[(u + 1) % P], rb[(u + 1) % P]);
                __syncthreads();
            }
        }
    } else {
        // Three LDS stages.  Slab s lives in stage s % 3; it is written in
        // iteration s - 2, its fragments are read into registers in iteration
        // s - 1 (while the MFMAs of slab s - 1 run) and consumed in iteration
        // s, so no wave waits on LDS after the barrier.  The barrier at the
        // end of iteration t publishes slab t + 2 before iteration t + 1 reads
        // it, and separates the last reads of a stage (iteration s - 1) from
        // its next writes (iteration s + 1).
        Frag f[2];
        if (nslab > 0) {
            load_slab(0, ra[0], rb[0]);
            store_slab(0, ra[0], rb[0]);
        }
        if (nslab > 1) {
            load_slab(BK, ra[0], rb[0]);
            store_slab(1, ra[0], rb[0]);
        }
        __syncthreads();
        if (nslab > 0) read_frags(0, f[0]);
        int s_cur = 0;
        for (int t0 = 0; t0 < nslab; t0 += 2) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int t = t0 + u;
                if (t >= nslab) break;
                const int s_nxt = s_cur == 2 ? 0 : s_cur + 1;
                const int s_wr = s_nxt == 2 ? 0 : s_nxt + 1;
                if (t + 2 < nslab) load_slab((t + 2) * BK, ra[0], rb[0]);
                if (t + 1 < nslab) read_frags(s_nxt, f[u ^ 1]);
                mma(f[u]);
                if (t + 2 < nslab) store_slab(s_wr, ra[0], rb[0]);
                __syncthreads();
                s_cur = s_nxt;
            }
        }
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

template <class Cfg>
hipError_t launch_cfg(const GemmArgs& a, hipStream_t stream) {
    constexpr int BM = Cfg::BM, BN = Cfg::BN;
    const int tiles_m = (a.M + BM - 1) / BM;
    const int tiles_n = (a.N + BN - 1) / BN;
    const dim3 grid((unsigned)(tiles_m * tiles_n)), block(Cfg::NT);
    const bool va = (a.lda % 4 == 0) && ((reinterpret_cast<uintptr_t>(a.A) & 15) == 0);
    const bool vb = (a.ldb % 4 == 0) && ((reinterpret_cast<uintptr_t>(a.B) & 15) == 0);
    if (va && vb)
        hipLaunchKernelGGL((sgemm_mfma_kernel<Cfg, true, true>), grid, block, 0, stream, a, tiles_m, tiles_n);
    else if (va)
        hipLaunchKernelGGL((sgemm_mfma_kernel<Cfg, true, false>), grid, block, 0, stream, a, tiles_m, tiles_n);
    else if (vb)
        hipLaunchKernelGGL((sgemm_mfma_kernel<Cfg, false, true>), grid, block, 0, stream, a, tiles_m, tiles_n);
    else
        hipLaunchKernelGGL((sgemm_mfma_kernel<Cfg, false, false>), grid, block, 0, stream, a, tiles_m, tiles_n);
    return hipGetLastError();
}

}  // namespace

// Tile table, chosen by measured GFLOP/s on MI355X (256 CUs):
//  * large grids: 256x256 block, 16 waves of 64x64 (4 MFMA blocks each) --
//    the most operand reuse per LDS byte and per L2 byte;
//  * mid-size: 64x128 block, 8 waves of 32x32 -- enough workgroups to keep
//    two per CU resident;
//  * small / ragged: 64x64 block, 4 waves of 32x32 -- the most workgroups.
// A class is taken when its grid still gives every CU at least two
// workgroups' worth of tiles.
using MfmaLarge = MfmaCfg<256, 256, 16, 64, 64, 1>;
using MfmaMid = MfmaCfg<64, 128, 16, 32, 32, 2>;
using MfmaSmall = MfmaCfg<64, 64, 16, 32, 32, 2>;

static long long tiles_of(const GemmArgs& a, int bm, int bn) {
    return ((long long)a.M + bm - 1) / bm * (((long long)a.N + bn - 1) / bn);
}

hipError_t launch_mfma(const GemmArgs& a, hipStream_t stream) {
    if (tiles_of(a, 256, 256) >= 512) return launch_cfg<MfmaLarge>(a, stream);
    if (tiles_of(a, 64, 128) >= 512) return launch_cfg<MfmaMid>(a, stream);
    return launch_cfg<MfmaSmall>(a, stream);
}

}  // namespace sgemm
