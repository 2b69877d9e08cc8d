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
// after; one barrier per slab.  k past K is loaded as zero, so the K tail
// adds nothing ("gemm_tiled_test" section 3, zero-padding after the boundary
// check); rows past M and columns past N are read from in-range addresses
// instead (see the kernel), which only reaches accumulators of C entries
// that the store, guarded by row < M && col < N, never writes.
#include <algorithm>
#include <type_traits>
#include <utility>

#include "lds_dma.h"
#include "tiles.h"

namespace sgemm {
namespace {

template <int BM_, int BN_, int BK_, int WM_, int WN_, int MINW_ = 2, int GROUP_M_ = 8,
          bool XCD_ = true, int PADB_ = 4, int P_ = 1, int KC_ = 0>
struct MfmaCfg {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_;
    static constexpr int P = P_;                         // slabs in flight in registers
    static constexpr int STAGES = 2;                     // LDS stages
    // MFMA steps per fragment chunk: 0 = read the whole slab's fragments up
    // front; otherwise read chunk c + 1 while chunk c multiplies, with
    // scheduling fences so the compiler keeps that order.
    static constexpr int KC = KC_ == 0 ? BK_ / 2 : KC_;
    static constexpr bool CHUNKED = KC_ != 0;
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
    static_assert((BK / 2) % KC == 0 && KC % 4 == 0, "chunks of whole float4 A reads");
};

template <class Cfg, bool VA, bool VB, bool EPI>
__global__ __launch_bounds__(Cfg::NT, Cfg::MINW)
void sgemm_mfma_kernel(GemmArgs p, int tiles_m, int tiles_n) {
    constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK, WM = Cfg::WM, WN = Cfg::WN;
    constexpr int NT = Cfg::NT, FM = Cfg::FM, FN = Cfg::FN, KH = Cfg::KH;
    constexpr int SA = Cfg::SA, SB = Cfg::SB;
    __shared__ __attribute__((aligned(16))) float As[Cfg::STAGES][BM * SA];
    __shared__ __attribute__((aligned(16))) float Bs[Cfg::STAGES][BK * SB];

    int tm, tn;
    tile_coords(blockIdx.x, tiles_m, tiles_n, Cfg::GROUP_M, Cfg::XCD ? p.xcds : 1, tm, tn);
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
    // Edge tiles.  Row r of A only feeds row r of C, and column j of B only
    // column j of C; rows and columns past the matrix edge are never stored.
    // So a lane whose A row lies past M loads row M - 1 instead, and a lane
    // whose B float4 lies wholly past N loads the tile's first four columns
    // (when the tile has four inside N): in-range addresses, ordinary vector
    // loads, garbage confined to discarded accumulators.  A B float4 that
    // straddles N, one past N in a tile with fewer than four columns inside
    // it, and the K tail (where every C entry sums the product) keep the
    // element-wise zero-filling load.  The LDS destinations stay a_row, b_col.
    int a_src[Cfg::A_F4], b_src[Cfg::B_F4];
    bool b_whole[Cfg::B_F4];
#pragma unroll
    for (int i = 0; i < Cfg::A_F4; ++i) a_src[i] = min(a_row[i], mrem - 1);
#pragma unroll
    for (int i = 0; i < Cfg::B_F4; ++i) {
        b_whole[i] = b_col[i] + 4 <= nrem || (b_col[i] >= nrem && nrem >= 4);
        b_src[i] = b_col[i] >= nrem ? 0 : b_col[i];
    }

    using RegA = float4[Cfg::A_F4];
    using RegB = float4[Cfg::B_F4];
    auto load_slab = [&](int k0, RegA& ra, RegB& rb) {
        const bool k_full = (K - k0) >= BK;
#pragma unroll
        for (int i = 0; i < Cfg::A_F4; ++i)
            if (Cfg::A_TOT >= NT || tid < Cfg::A_TOT)
                ra[i] = load4<VA>(Ablk + k0, p.lda, a_src[i], a_col[i], mrem, K - k0, k_full);
#pragma unroll
        for (int i = 0; i < Cfg::B_F4; ++i)
            if (Cfg::B_TOT >= NT || tid < Cfg::B_TOT)
                rb[i] = load4<VB>(Bblk + (long long)k0 * p.ldb, p.ldb, b_row[i], b_src[i],
                                  K - k0, nrem, k_full && b_whole[i]);
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
    // debug build: the words store_slab(st, ..) is about to write
    auto poison_slab = [&](int st) {
#pragma unroll
        for (int i = 0; i < Cfg::A_F4; ++i)
            if (Cfg::A_TOT >= NT || tid < Cfg::A_TOT) lds_poison_f4(&As[st][a_row[i] * SA + a_col[i]]);
#pragma unroll
        for (int i = 0; i < Cfg::B_F4; ++i)
            if (Cfg::B_TOT >= NT || tid < Cfg::B_TOT) lds_poison_f4(&Bs[st][b_row[i] * SB + b_col[i]]);
    };

    floatx16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    // Fused form with beta != 0: read C's previous values now, so the reads
    // overlap the main loop (wave tiles of up to two blocks; larger ones have
    // no registers to spare and read C at the store).
    constexpr bool PRE_C = EPI && FM * FN <= 2;
    floatx16 cin[FM][FN];
    if constexpr (PRE_C) load_c_tile(p, cin, m0 + wm, n0 + wn, li, lh);

    // One slab from LDS stage st: each wave reads its A rows (float4) and B
    // columns into registers and applies BK/2 rank-2 MFMA updates to each
    // accumulator block.  Fragments come in chunks of KC MFMA steps.
    constexpr int KC = Cfg::KC, NC = KH / KC;
    struct Chunk {
        float a[FM][KC], b[FN][KC];
    };
    auto read_chunk = [&](int st, int c, Chunk& f) {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const float* src = &As[st][(wm + i * 32 + li) * SA + lh * KH + c * KC];
#pragma unroll
            for (int q = 0; q < KC / 4; ++q) {
                const float4 v = *reinterpret_cast<const float4*>(src + 4 * q);
                f.a[i][4 * q + 0] = v.x; f.a[i][4 * q + 1] = v.y;
                f.a[i][4 * q + 2] = v.z; f.a[i][4 * q + 3] = v.w;
            }
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const float* src = &Bs[st][(lh * KH + c * KC) * SB + wn + j * 32 + li];
#pragma unroll
            for (int s = 0; s < KC; ++s) f.b[j][s] = src[s * SB];
        }
    };
    auto mma_chunk = [&](const Chunk& f) {
#pragma unroll
        for (int s = 0; s < KC; ++s)
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(f.a[i][s], f.b[j][s],
                                                                     acc[i][j], 0, 0, 0);
    };
    auto compute = [&](int st) {
        if constexpr (!Cfg::CHUNKED) {
            Chunk f;
            read_chunk(st, 0, f);
            mma_chunk(f);
        } else {
            Chunk f[2];
            read_chunk(st, 0, f[0]);
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                if (c + 1 < NC) read_chunk(st, c + 1, f[(c + 1) & 1]);
                __builtin_amdgcn_sched_barrier(0);
                mma_chunk(f[c & 1]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    // Two LDS stages.  Slab s is staged in register set s % P, written to LDS
    // stage s % 2 at the end of iteration s - 1 and computed in iteration s.
    // The global loads of slab t + P are issued at the start of iteration t
    // into the set slab t has left, so each load has P slabs of compute to
    // land.  One barrier per slab orders this iteration's LDS writes before
    // the next iteration's reads, and this iteration's reads of stage t % 2
    // before iteration t + 1 writes it.
    constexpr int P = Cfg::P;
    float4 ra[P][Cfg::A_F4], rb[P][Cfg::B_F4];
    const int nslab = (K + BK - 1) / BK;
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
            // (debug build: stage (t + 1) & 1, retired by the barrier
            // ending iteration t - 1)
            if (kLdsPoison && t + 1 < nslab) poison_slab((t + 1) & 1);
            if (t + P < nslab) load_slab((t + P) * BK, ra[u], rb[u]);
            compute(t & 1);
            if (t + 1 < nslab) store_slab((t + 1) & 1, ra[(u + 1) % P], rb[(u + 1) % P]);
            __syncthreads();
        }
    }

    store_tile<EPI, FM, FN, PRE_C>(p, acc, cin, m0 + wm, n0 + wn, li, lh);
}

// ---------------------------------------------------------------------------
// Direct-to-LDS variant.  Same block/wave/MFMA structure, but the tile loader
// is gfx950's global_load_lds_dwordx4: every lane names a 16-byte global
// chunk and the memory system writes it straight into LDS at
// (wave-uniform base) + 16 * lane, with no staging registers and no
// ds_write.  Three LDS stages: stage t + 2 is requested while stage t is
// multiplied, so every load has two stages of MFMA work to arrive in.  (The
// pages' next-step plan puts an asynchronous copy pipeline into the
// micro-kernel and names pipeline prefetching; this is that, on CDNA4.)
//
// K split inside the workgroup (KS > 1): the waves form KS groups, each a
// full copy of the BM x BN wave grid.  A stage holds KS consecutive 16-deep
// sub-slabs of K and group g multiplies sub-slab g, so a tile runs KS times
// as many waves, each over 1/KS of K, which gives grids with few tiles more
// waves per SIMD to hide the per-slab latency with.  At the end the groups
// g > 0 leave their accumulators in LDS and group 0 adds them in the fixed
// order g = 1, 2, ... before the store: deterministic, and the fused
// epilogue still sees the whole sum.  (The pages' next steps name split-K
// for shapes with few tiles.)
//
// Because the DMA fills 64 consecutive chunks per instruction, the LDS tiles
// are dense and bank conflicts are avoided by XOR-swizzling 16-byte chunks
// instead of padding rows.  Within one sub-slab:
//   A (BM x 16): chunk c of row r sits at chunk c ^ (((r >> 1) ^ (r >> 3)) & 3)
//                -- the float4 reads of 8 (or 16) consecutive rows then hit
//                distinct banks;
//   B (16 x BN): chunk c of row k sits at chunk c ^ (8 * (k >= 8)) -- the two
//                lane halves of a B read (k and k + 8) land 128 bytes apart.
// Stages that cross the matrix edge (edge tiles, the K tail) take a register
// loader that zero-fills and writes the same swizzled layout; matrices whose
// rows are not 16-byte aligned never reach this kernel.
template <int BM_, int BN_, int WM_, int WN_, int MINW_ = 1, int KS_ = 1, int STAGES_ = 3,
          bool MID_ = false, int GROUP_M_ = 8>
struct DmaCfg {
    static constexpr int BM = BM_, BN = BN_, BK = 16, WM = WM_, WN = WN_;
    static constexpr int MINW = MINW_, KS = KS_, GROUP_M = GROUP_M_;
    static constexpr int KSLAB = KS * BK;              // k per stage
    // LDS buffers; stage t + STAGES - 1 is requested while stage t multiplies.
    static constexpr int STAGES = STAGES_;
    // Where the stage's barrier sits: after all its MFMAs (false; three
    // stages), or between their two halves, with the next stage's first
    // operands read during the second half (true).
    static constexpr bool MID = MID_;
    static constexpr bool XCD = true;
    static constexpr int WAVES_N = BN / WN;
    static constexpr int NWT = (BM / WM) * (BN / WN);  // waves of one group
    static constexpr int NW = NWT * KS;                // waves per workgroup
    static constexpr int NT = NW * 64;
    static constexpr int FM = WM / 32, FN = WN / 32, KH = BK / 2;
    static constexpr int CA = BK / 4;                  // 16-byte chunks per A row
    static constexpr int CB = BN / 4;                  // chunks per B row
    static constexpr int A_SUB = BM * CA / 64;         // DMA instructions per sub-slab
    static constexpr int B_SUB = BK * CB / 64;
    static constexpr int A_INS = KS * A_SUB, B_INS = KS * B_SUB;  // per stage
    static constexpr int SA = KS * BM * BK, SB = KS * BK * BN;    // floats per stage
    static constexpr int LDS_FLOATS = STAGES * (SA + SB);
    static constexpr int RED_FLOATS = (KS - 1) * BM * BN;         // K-split partial sums
    static_assert(BM % WM == 0 && BN % WN == 0 && WM % 32 == 0 && WN % 32 == 0, "tiles");
    static_assert((BM * CA) % 64 == 0 && (BK * CB) % 64 == 0, "whole DMA instructions");
    static_assert(BN % 64 == 0, "B swizzle flips chunk bit 3 inside 16-chunk groups");
    static_assert(LDS_FLOATS * 4 <= 160 * 1024, "LDS budget of one CU");
    static_assert(RED_FLOATS <= LDS_FLOATS, "partial sums fit in the stage buffers");
    static_assert(NT <= 1024, "workgroup size");
    static_assert(STAGES >= 3, "the schedule keeps two stages ahead of the one being read");
    static_assert(MID || STAGES == 3, "the end-of-stage schedule is written for three stages");
};

__device__ __forceinline__ int swz_a(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }


template <class Cfg, bool EPI>
__global__ __launch_bounds__(Cfg::NT, Cfg::MINW)
void sgemm_mfma_dma_kernel(GemmArgs p, int tiles_m, int tiles_n) {
    constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK, WM = Cfg::WM, WN = Cfg::WN;
    constexpr int NW = Cfg::NW, NWT = Cfg::NWT, FM = Cfg::FM, FN = Cfg::FN, KH = Cfg::KH;
    constexpr int CA = Cfg::CA, CB = Cfg::CB, KSLAB = Cfg::KSLAB;
    constexpr int SA = Cfg::SA, SB = Cfg::SB, STAGES = Cfg::STAGES;
    // Stages of A, then stages of B; at the end, the K-split partial sums.
    __shared__ __attribute__((aligned(16))) float lds[Cfg::LDS_FLOATS];
    float* const As = lds;
    float* const Bs = lds + STAGES * SA;

    int tm, tn;
    tile_coords(blockIdx.x, tiles_m, tiles_n, Cfg::GROUP_M, Cfg::XCD ? p.xcds : 1, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int M = p.M, N = p.N, K = p.K;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int grp = wave / NWT, wt = wave % NWT;       // K-split group, wave in group
    const int wm = (wt / Cfg::WAVES_N) * WM;
    const int wn = (wt % Cfg::WAVES_N) * WN;
    const int li = lane & 31, lh = lane >> 5;
    const float* __restrict__ Ablk = p.A + (long long)m0 * p.lda;
    const float* __restrict__ Bblk = p.B + n0;
    const int mrem = M - m0, nrem = N - n0;
    const bool mn_full = mrem >= BM && nrem >= BN;
    // DMA instructions this wave issues per stage (wave-uniform).
    const int n_dma = (Cfg::A_INS % NW == 0 && Cfg::B_INS % NW == 0)
        ? Cfg::A_INS / NW + Cfg::B_INS / NW
        : (wave < Cfg::A_INS ? (Cfg::A_INS - wave + NW - 1) / NW : 0) +
          (wave < Cfg::B_INS ? (Cfg::B_INS - wave + NW - 1) / NW : 0);
    const unsigned as_base = lds_addr(As), bs_base = lds_addr(Bs);

    // Instruction q of a stage covers sub-slab g = q / A_SUB (or B_SUB) and
    // 64 chunks of it; its LDS destination is q * 256 floats into the stage,
    // i.e. sub-slab g occupies floats [g * BM * BK, (g + 1) * BM * BK) of an
    // A stage and [g * BK * BN, (g + 1) * BK * BN) of a B stage.
    // Full stage at k0 into stage st: pure DMA, n_dma instructions per wave.
    auto issue_full = [&](int k0, int st) {
        for (int q = wave; q < Cfg::A_INS; q += NW) {
            const int g = q / Cfg::A_SUB, P = (q % Cfg::A_SUB) * 64 + lane;
            const int r = P / CA, c = (P % CA) ^ swz_a(P / CA);
            lds_dma16(Ablk + (long long)r * p.lda + k0 + g * BK + 4 * c,
                      __builtin_amdgcn_readfirstlane(as_base + 4u * (unsigned)(st * SA + q * 256)));
        }
        for (int q = wave; q < Cfg::B_INS; q += NW) {
            const int g = q / Cfg::B_SUB, P = (q % Cfg::B_SUB) * 64 + lane;
            const int k = P / CB, c = (P % CB) ^ ((k / KH) << 3);
            lds_dma16(Bblk + (long long)(k0 + g * BK + k) * p.ldb + 4 * c,
                      __builtin_amdgcn_readfirstlane(bs_base + 4u * (unsigned)(st * SB + q * 256)));
        }
    };
    // Any stage (edge tiles, the K tail) into stage st with ordinary loads:
    // elements outside the matrix are written as zeros.  Completes before
    // returning except for the ds_writes (ordered by the next barrier).
    auto issue_edge = [&](int k0, int st) {
        if constexpr (kLdsPoison) {   // debug build: the chunks written below
            for (int q = wave; q < Cfg::A_INS; q += NW) lds_poison_f4(&As[st * SA + q * 256 + lane * 4]);
            for (int q = wave; q < Cfg::B_INS; q += NW) lds_poison_f4(&Bs[st * SB + q * 256 + lane * 4]);
        }
        for (int q = wave; q < Cfg::A_INS; q += NW) {
            const int g = q / Cfg::A_SUB, P = (q % Cfg::A_SUB) * 64 + lane;
            const int r = P / CA, c = (P % CA) ^ swz_a(P / CA);
            const int kg = k0 + g * BK + 4 * c, krem = K - kg;
            const float* gp = Ablk + (long long)r * p.lda + kg;
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (r < mrem) {
                if (0 < krem) v.x = gp[0];
                if (1 < krem) v.y = gp[1];
                if (2 < krem) v.z = gp[2];
                if (3 < krem) v.w = gp[3];
            }
            *reinterpret_cast<float4*>(&As[st * SA + q * 256 + lane * 4]) = v;
        }
        for (int q = wave; q < Cfg::B_INS; q += NW) {
            const int g = q / Cfg::B_SUB, P = (q % Cfg::B_SUB) * 64 + lane;
            const int k = P / CB, c = (P % CB) ^ ((k / KH) << 3);
            const int kg = k0 + g * BK + k;
            const float* gp = Bblk + (long long)kg * p.ldb + 4 * c;
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (kg < K) {
                if (4 * c + 0 < nrem) v.x = gp[0];
                if (4 * c + 1 < nrem) v.y = gp[1];
                if (4 * c + 2 < nrem) v.z = gp[2];
                if (4 * c + 3 < nrem) v.w = gp[3];
            }
            *reinterpret_cast<float4*>(&Bs[st * SB + q * 256 + lane * 4]) = v;
        }
    };
    // Barrier that orders LDS traffic: wait until at most `inflight` of this
    // wave's DMA instructions are outstanding and its ds_writes are done,
    // then s_barrier.  The empty asm statements keep the compiler from
    // moving LDS accesses across it.
    auto lds_barrier = [&](int inflight) {
        asm volatile("" ::: "memory");
        wait_vmcnt(inflight);
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };

    floatx16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    // Fused form with beta != 0: read C's previous values now, so the reads
    // overlap the main loop (wave tiles of up to two blocks; larger ones have
    // no registers to spare and read C at the store).
    constexpr bool PRE_C = EPI && FM * FN <= 2;
    floatx16 cin[FM][FN];
    if constexpr (PRE_C) {
        if (grp == 0) load_c_tile(p, cin, m0 + wm, n0 + wn, li, lh);   // only group 0 stores
    }

    // Fragment addresses (floats, inside this group's sub-slab of a stage).
    const int a_sub = grp * BM * BK, b_sub = grp * BK * BN;
    int a_off[FM], a_swz[FM], b_off[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        a_off[i] = a_sub + (wm + i * 32 + li) * BK;
        a_swz[i] = swz_a(wm + i * 32 + li);
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int col = wn + j * 32 + li;
        b_off[j] = b_sub + lh * KH * BN + ((((col >> 2) ^ (lh << 3)) << 2) | (col & 3));
    }
    // Operands of one half of a sub-slab: half h is MFMA steps 4h .. 4h+3,
    // i.e. k = 8lh + 4h + e for lane half lh -- one float4 of each A row
    // (chunk 2lh + h) and four values down each B column.
    struct Half {
        float a[FM][4], b[FN][4];
    };
    auto read_half = [&](int st, int h, Half& f) {
        const float* as = &As[st * SA];
        const float* bs = &Bs[st * SB];
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const float4 v = *reinterpret_cast<const float4*>(
                &as[a_off[i] + 4 * ((lh * 2 + h) ^ a_swz[i])]);
            f.a[i][0] = v.x; f.a[i][1] = v.y; f.a[i][2] = v.z; f.a[i][3] = v.w;
        }
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) f.b[j][e] = bs[b_off[j] + (4 * h + e) * BN];
    };
    auto mma_half = [&](const Half& f) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(f.a[i][e], f.b[j][e],
                                                                     acc[i][j], 0, 0, 0);
    };

    if constexpr (!Cfg::MID) {
        // Three stages, one barrier per stage after all its MFMAs; interior
        // tiles, the K tail and edge tiles in loops of their own.
        // One sub-slab from stage st: each wave reads its A rows (float4) and B
        // columns and applies BK/2 rank-2 MFMA updates to every accumulator block.
        auto compute = [&](int st, auto&& between) {
            const float* as = &As[st * SA];
            const float* bs = &Bs[st * SB];
            float fa[FM][KH], fb[FN][KH];
#pragma unroll
            for (int i = 0; i < FM; ++i) {
#pragma unroll
                for (int q = 0; q < KH / 4; ++q) {
                    const int c = (lh * (KH / 4) + q) ^ a_swz[i];
                    const float4 v = *reinterpret_cast<const float4*>(&as[a_off[i] + 4 * c]);
                    fa[i][4 * q + 0] = v.x; fa[i][4 * q + 1] = v.y;
                    fa[i][4 * q + 2] = v.z; fa[i][4 * q + 3] = v.w;
                }
            }
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int s = 0; s < KH; ++s) fb[j][s] = bs[b_off[j] + s * BN];
            between();   // e.g. request a later stage while the reads are in flight
#pragma unroll
            for (int s = 0; s < KH; ++s)
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[i][s], fb[j][s],
                                                                         acc[i][j], 0, 0, 0);
        };

        if (mn_full) {
            // Interior tile: full stages stream through three LDS stages by DMA.
            // Iteration t reads stage t's fragments, requests stage t + 2 into the
            // buffer stage t - 1 used (every wave finished reading it before the
            // previous barrier), multiplies, then waits until stage t + 1 has
            // landed.
            const int nfull = K / KSLAB;
            if (nfull > 0) issue_full(0, 0);
            if (nfull > 1) issue_full(KSLAB, 1);
            lds_barrier(nfull > 1 ? n_dma : 0);
            int st = 0;
            for (int t = 0; t < nfull; ++t) {
                const int st2 = st == 0 ? 2 : st - 1;   // (st + 2) % 3
                const bool more = t + 2 < nfull;
                compute(st, [&] { if (more) issue_full((t + 2) * KSLAB, st2); });
                lds_barrier(more ? n_dma : 0);
                st = st == 2 ? 0 : st + 1;
            }
            if (K % KSLAB) {   // the K tail: one stage with zero fill
                issue_edge(nfull * KSLAB, 0);
                lds_barrier(0);
                compute(0, [] {});
            }
        } else {
            // Tile crossing the matrix edge: one stage, load / barrier / compute /
            // barrier per step.
            const int nslab = (K + KSLAB - 1) / KSLAB;
            for (int t = 0; t < nslab; ++t) {
                issue_edge(t * KSLAB, 0);
                lds_barrier(0);
                compute(0, [] {});
                lds_barrier(0);
            }
        }
    } else {
        // One pipeline for every tile: S = STAGES LDS buffers, stage t + D
        // (D = S - 1) requested while stage t multiplies, into the buffer
        // stage t - 1 used (every wave finished reading it before the previous
        // barrier), and one barrier per stage between the two halves of its
        // MFMA steps.  Iteration t (stage t's first-half operands f0 already
        // read):
        //   1. read the second-half operands f1 of stage t;
        //   2. request stage t + D;
        //   3. multiply the first half (f0);
        //   4. wait until stage t + 1 has landed (stages t + 2 .. t + D may
        //      stay in flight), barrier, read its first-half operands into
        //      f0 -- their latency hides behind
        //   5. the second half's MFMAs (f1).
        // Whole stages of interior tiles come by DMA; stages that cross an
        // edge of the matrix come through the register loader, which
        // completes before it returns (its ds_writes are ordered by the next
        // barrier).  sched_barrier keeps the compiler from sinking the reads
        // of step 1 below the MFMAs of step 3.
        constexpr int S = Cfg::STAGES, D = S - 1;
        const int nstage = (K + KSLAB - 1) / KSLAB;
        const int nfull = mn_full ? K / KSLAB : 0;    // stages 0 .. nfull-1 by DMA
        auto issue = [&](int t, int st) {
            if (t < nfull) issue_full(t * KSLAB, st);
            else issue_edge(t * KSLAB, st);
        };
        // DMA instructions of this wave still allowed in flight once stage u
        // has landed: those of the DMA stages u + 1 .. min(last requested,
        // nfull - 1).
        auto inflight_after = [&](int u, int last) {
            const int hi = min(last, nfull - 1);
            return hi > u ? (hi - u) * n_dma : 0;
        };
#pragma unroll
        for (int u = 0; u < D; ++u)
            if (u < nstage) issue(u, u);
        lds_barrier(inflight_after(0, D - 1));
        Half f0, f1;
        if (nstage > 0) read_half(0, 0, f0);
        int st = 0, st_req = D;   // buffer of stage t; buffer for stage t + D
        for (int t = 0; t < nstage; ++t) {
            const int st1 = st + 1 == S ? 0 : st + 1;
            read_half(st, 1, f1);
            if (t + D < nstage) issue(t + D, st_req);
            st_req = st_req + 1 == S ? 0 : st_req + 1;
            __builtin_amdgcn_sched_barrier(0);
            mma_half(f0);
            if (t + 1 < nstage) {
                lds_barrier(inflight_after(t + 1, t + D));
                read_half(st1, 0, f0);
            }
            __builtin_amdgcn_sched_barrier(0);
            mma_half(f1);
            st = st1;
        }
    }

    if constexpr (Cfg::KS > 1) {
        // Partial sums of groups 1.. KS-1 through LDS (lane-contiguous, no
        // bank conflicts); group 0 adds them in order and stores.
        constexpr int PER_WAVE = FM * FN * 16 * 64;
        lds_barrier(0);   // every wave is done reading the stages
        if (grp > 0) {
            float* dst = lds + ((grp - 1) * NWT + wt) * PER_WAVE + lane;
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) dst[((i * FN + j) * 16 + r) * 64] = acc[i][j][r];
        }
        lds_barrier(0);
        if (grp > 0) return;
        for (int g = 1; g < Cfg::KS; ++g) {
            const float* src = lds + ((g - 1) * NWT + wt) * PER_WAVE + lane;
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[i][j][r] += src[((i * FN + j) * 16 + r) * 64];
        }
    }
    store_tile<EPI, FM, FN, PRE_C>(p, acc, cin, m0 + wm, n0 + wn, li, lh);
}

bool rows_16b_aligned(const GemmArgs& a) {
    return (a.lda % 4 == 0) && (a.ldb % 4 == 0) &&
           ((reinterpret_cast<uintptr_t>(a.A) & 15) == 0) &&
           ((reinterpret_cast<uintptr_t>(a.B) & 15) == 0);
}

// The DMA kernel copies whole 16-byte chunks, so A's and B's rows must be
// 16-byte aligned; anything else is refused here.
template <class Cfg>
hipError_t launch_dma_cfg(const GemmArgs& a, hipStream_t stream) {
    if (!rows_16b_aligned(a)) return hipErrorInvalidValue;
    const int tiles_m = (a.M + Cfg::BM - 1) / Cfg::BM;
    const int tiles_n = (a.N + Cfg::BN - 1) / Cfg::BN;
    const dim3 grid((unsigned)(tiles_m * tiles_n)), block(Cfg::NT);
    if (a.epi)
        hipLaunchKernelGGL((sgemm_mfma_dma_kernel<Cfg, true>), grid, block, 0, stream, a, tiles_m, tiles_n);
    else
        hipLaunchKernelGGL((sgemm_mfma_dma_kernel<Cfg, false>), grid, block, 0, stream, a, tiles_m, tiles_n);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Large wave tiles.  A BM x BM tile (BM = 256, 128 or 64) computed by 4
// waves, one per SIMD: 2 x 2 waves of BM/2 x BM/2 (4 x 1 of 16 x 64 at BM =
// 64), each holding its sub-tile as accumulator blocks of
// v_mfma_f32_16x16x4_f32 -- 64 blocks, 256 accumulator registers per lane
// at BM = 256.  The few-wave, large-wave-tile design reaches the
// fp32 matrix peak only if the single wave of each SIMD never leaves the
// matrix pipe idle, so everything else is shaped around the MFMA stream:
//  * tiles come by direct-to-LDS DMA into two LDS buffers of SUBS 16-deep
//    sub-slabs, interleaved one instruction at a time with the MFMAs;
//  * every operand read is a 16-byte ds_read_b128.  A (rows of 16 k, chunk
//    c of row r at chunk c ^ ((r >> 2) & 3)) gives lane (q, li) four
//    consecutive k of its row: one float4 per row block serves the four MFMA
//    steps of a sub-slab, with k = 4q + s at step s.  B is read along n:
//    lane li takes columns 4li .. 4li+3 of a 64-column group, and those four
//    columns belong to four different accumulator blocks (block j holds
//    columns 64(j/4) + 4li + j%4 of the wave tile), so one float4 feeds four
//    MFMAs.  The output then comes out as float4 rows as well;
//  * operand reads for the next step or sub-slab run between the current
//    MFMAs, into the other half of a double-buffered register set;
//  * one barrier per stage, taken PRE MFMAs into the stage's last step: the
//    next stage has landed and every wave has read the current buffer; the
//    next stage's first operands are read between the remaining MFMAs.
// The order of MFMAs, reads and DMA is fixed by a scheduling fence after
// every MFMA.  The MFMA is written as inline assembly with its accumulator
// bound to AGPRs: through the builtin, the register allocator kept part of
// the 64 accumulators in VGPRs and copied them in and out on every
// iteration.  The compiler does not see these MFMAs, so the kernel supplies
// the wait states they need itself: a pause after the accumulators are
// zeroed and before they are read for the store, and no operand register is
// overwritten less than RB MFMAs after its last reader.
//
// Shapes.  Any M, N, K, alignment and leading dimension below 2^22; all
// of it is handled without touching the main loop:
//  * ragged M and N: a DMA lane whose A row lies past M reads row M - 1, one
//    whose B column (or chunk) lies past N reads the tile's first column.
//    Those values reach only accumulators of C entries that are never
//    stored, and the store is guarded (row < M, col < N);
//  * any K: the k range is shifted so that the stages start at k = -shift
//    and end exactly at K, shift = (2 KST - K % 2 KST) % 2 KST (whole pairs
//    of stages) or, in configurations built for odd stage counts, (KST -
//    K % KST) % KST (at least two stages).  Both LDS buffers are zeroed
//    first and the DMA lanes of negative k are switched off, so those k add
//    nothing; every later stage is whole;
//  * A rows that are not 16-byte aligned (or K % 4 != 0): A comes by the
//    4-byte form of the DMA, 64 floats per instruction, into the same
//    swizzled layout (four times the instructions, no alignment needed);
//    likewise B when its rows are not 16-byte aligned or N % 4 != 0 (a
//    16-byte chunk could then reach past the last row's end);
//  * C rows that are not 16-byte aligned, or N % 4 != 0: the four
//    consecutive columns a lane holds are stored one by one.
typedef float floatx4 __attribute__((ext_vector_type(4)));

template <int BM_, int SUBS_, bool LATE_, int PRE_ = 4, int GROUP_M_ = 8, int DFRAC_ = 2,
          int BN_ = BM_, bool ODD_ = false>
struct BigCfg {
    static constexpr int BM = BM_, BN = BN_, SUBS = SUBS_, PRE = PRE_, GROUP_M = GROUP_M_;
    // ODD: also built for odd stage counts (early DMA only), so that the k
    // shift stays below one stage
    static constexpr bool ODD = ODD_;
    // Where the DMA goes: LATE, stage t + 2's right after the barrier in
    // stage t's last step (a whole stage to land); else stage t + 1's, spread
    // over the first 1/DFRAC of stage t.
    static constexpr bool LATE = LATE_;
    static constexpr int NW = 4, NT = 256;
    // wave grid: 2 x 2 waves of BM/2 x BN/2; at BM = 64, 4 x 1 of 16 x BN
    // (a wave tile of 64 or 96 columns keeps the vector B reads)
    static constexpr int WAVES_N = BM >= 128 ? 2 : 1, WAVES_M = NW / WAVES_N;
    static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
    static constexpr int FBM = WM / 16, FBN = WN / 16;        // 16x16 blocks per wave
    // B reads per step: NB4 float4 (each feeding four blocks) and, when the
    // wave tile has 32 columns more than a multiple of 64, one float2
    // feeding the last two blocks
    static constexpr int NB4 = FBN / 4, NB2 = (FBN % 4) / 2;
    static constexpr int NB = NB4 + NB2;
    static constexpr int NMF = FBM * FBN;                     // MFMAs per step
    static constexpr int KST = 16 * SUBS;                     // k per stage
    static constexpr int STEPS = 4 * SUBS;                    // MFMA steps per stage
    static constexpr int SA = BM * KST, SB = KST * BN;        // floats per stage
    // A and B DMA per stage and per wave, 16-byte or 4-byte form
    static constexpr int aq(bool x4) { return (x4 ? BM * SUBS / 16 : BM * SUBS / 4) / NW; }
    static constexpr int bq(bool x4) { return (x4 ? KST * BN / 256 : KST * BN / 64) / NW; }
    static constexpr int ndma(bool ax4, bool bx4) { return aq(ax4) + bq(bx4); }
    // early DMA: the first STEPS / DFRAC steps, or as many as its
    // instructions need at one per MFMA
    static constexpr int dsteps(bool ax4, bool bx4) {
        return STEPS / DFRAC_ > (ndma(ax4, bx4) + NMF - 1) / NMF ? STEPS / DFRAC_
                                                                  : (ndma(ax4, bx4) + NMF - 1) / NMF;
    }
    static constexpr int dgap(bool ax4, bool bx4) { return dsteps(ax4, bx4) * NMF / ndma(ax4, bx4); }
    // Operand reads of a step start RB MFMAs in, so an operand register is
    // rewritten at least RB MFMAs after its last reader; in the last step
    // they follow the barrier every OS-th MFMA.
    static constexpr int RB = NMF >= 8 ? 4 : 1, OS = NMF >= 16 ? 2 : 1;
    // A pair of DMA forms is built where its instructions fit the schedule:
    // with late DMA, after the reads of the stage's last step; with early
    // DMA, one per MFMA over less than a stage.  The 4-byte A form at BM =
    // 128 also does not fit the registers of the two waves per SIMD the
    // compiler budgets that tile, so it is not built there.
    static constexpr bool late_fits(int nd) { return PRE + 1 + OS * (NB + FBM + nd - 1) < NMF; }
    static constexpr bool fits(bool ax4, bool bx4) {
        return (ax4 || BM != 128) &&
               (LATE ? late_fits(ndma(ax4, bx4))
                     : dsteps(ax4, bx4) < STEPS && dgap(ax4, bx4) >= 1);
    }
    // Waves per SIMD the kernel can run at: 1 when its LDS leaves room for
    // one workgroup per CU (told to the compiler, which otherwise may keep
    // a two-wave register budget it can never use).
    static constexpr int MAXW = 2 * (SA + SB) * 4 > 80 * 1024 ? 1 : 2;
    static_assert(BM == 256 || BM == 128 || BM == 64, "tile");
    static_assert((FBN % 4 == 0 || FBN % 4 == 2) && NMF >= 4,
                  "float4 B reads feed four blocks, a float2 two");
    static_assert((BM * SUBS / 16) % NW == 0 && (KST * BN / 256) % NW == 0 &&
                  (KST * BN / 64) % NW == 0 && BN % 32 == 0, "whole DMA instructions");
    static_assert(2 * (SA + SB) * 4 <= 160 * 1024, "two stages in LDS");
    static_assert(fits(true, true) && PRE >= 1 && RB + NB + FBM <= NMF, "ops fit their steps");
    static_assert(PRE + 1 + OS * (NB + FBM - 1) < NMF, "reads fit the last step");
    static_assert(!ODD || !LATE, "odd stage counts with the early DMA only");
};

__device__ __forceinline__ int swz_big(int r) { return (r >> 2) & 3; }



template <class Cfg, bool AX4, bool BX4, bool CX4, bool EPI, bool ODD>
__global__ __launch_bounds__(256, 1) __attribute__((amdgpu_waves_per_eu(1, Cfg::MAXW)))
void sgemm_mfma_big_kernel(GemmArgs p, int tiles_m, int tiles_n, int shift) {
    constexpr int BM = Cfg::BM, BN = Cfg::BN, FBM = Cfg::FBM, FBN = Cfg::FBN, SUBS = Cfg::SUBS;
    constexpr int SA = Cfg::SA, SB = Cfg::SB, BQ = Cfg::bq(BX4), KST = Cfg::KST;
    constexpr int AQ = Cfg::aq(AX4), NDMA = Cfg::ndma(AX4, BX4), DGAP = Cfg::dgap(AX4, BX4);
    constexpr int STEPS = Cfg::STEPS, NB = Cfg::NB, PRE = Cfg::PRE, NMF = Cfg::NMF;
    constexpr int RB = Cfg::RB, OS = Cfg::OS;
    __shared__ __attribute__((aligned(16))) float lds[2 * (SA + SB)];
    float* const As = lds;
    float* const Bs = lds + 2 * SA;

    int tm, tn;
    tile_coords(blockIdx.x, tiles_m, tiles_n, Cfg::GROUP_M, p.xcds, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int M = p.M, N = p.N;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = (wave / Cfg::WAVES_N) * Cfg::WM, wn = (wave % Cfg::WAVES_N) * Cfg::WN;
    const int q = lane >> 4, li = lane & 15;
    const unsigned as_base = __builtin_amdgcn_readfirstlane(lds_addr(As));
    const unsigned bs_base = __builtin_amdgcn_readfirstlane(lds_addr(Bs));

    // DMA sources: a scalar base (the tile's first row of A, or first
    // column of B, at the stage's first k) and a 32-bit byte offset per
    // lane that stays fixed for the whole loop, so the loop computes
    // addresses on the scalar unit only (a vector instruction between the
    // MFMAs costs the matrix pipe about 14 cycles).  akk and bkk give the k
    // offset of each lane's element in the stage (for switching off
    // negative k).
    //  * A, 16-byte form: instruction v covers sub-slab v / (BM/16), rows
    //    16 (v % (BM/16)) + lane/4; physical chunk lane % 4 holds logical
    //    chunk (lane % 4) ^ swz(row).
    //  * A, 4-byte form: instruction v covers sub-slab v / (BM/4), rows
    //    4 (v % (BM/4)) + lane/16; physical float lane % 16 of the row holds
    //    logical k 4 (((lane % 16) / 4) ^ swz(row)) + lane % 4.
    //  * B, 16-byte form: instruction v copies the 256 floats from float
    //    256 v of the stage's KST x BN block (one or more k rows); 4-byte
    //    form (B rows not 16-byte aligned, or N % 4 != 0): the 64 floats
    //    from float 64 v.
    // Rows past M read row M - 1, and columns (16-byte form: chunks) past N
    // the tile's first column.
    unsigned aoff[AQ], boff[BQ];
    int akk[AQ], bkk[BQ];
#pragma unroll
    for (int u = 0; u < AQ; ++u) {
        const int v = wave + 4 * u;
        int r, kk;
        if constexpr (AX4) {
            const int g = v / (BM / 16);
            r = 16 * (v % (BM / 16)) + (lane >> 2);
            kk = 16 * g + 4 * ((lane & 3) ^ swz_big(r));
        } else {
            const int g = v / (BM / 4);
            r = 4 * (v % (BM / 4)) + (lane >> 4);
            kk = 16 * g + 4 * (((lane & 15) >> 2) ^ swz_big(r)) + (lane & 3);
        }
        aoff[u] = 4u * ((unsigned)(min(m0 + r, M - 1) - m0) * (unsigned)p.lda + (unsigned)kk);
        akk[u] = kk;
    }
#pragma unroll
    for (int u = 0; u < BQ; ++u) {
        const int v = wave + 4 * u;
        const int e = BX4 ? 4 * (v * 64 + lane) : v * 64 + lane;   // float offset in the stage
        const int col = n0 + e % BN;
        boff[u] = 4u * ((unsigned)(e / BN) * (unsigned)p.ldb + (unsigned)(col < N ? col - n0 : 0));
        bkk[u] = e / BN;
    }
    const float* const a_tile = p.A + (long long)m0 * p.lda;
    const float* const b_tile = p.B + n0;
    // DMA d of the stage at k0 >= 0 into buffer buf
    auto issue_dma = [&](int d, int k0, int buf) {
        if (d < AQ) {
            const int v = wave + 4 * d;
            if constexpr (AX4)
                lds_dma16s(a_tile + k0, aoff[d], as_base + 4u * (unsigned)(buf * SA + v * 256));
            else
                lds_dma4s(a_tile + k0, aoff[d], as_base + 4u * (unsigned)(buf * SA + v * 64));
        } else {
            const int u = d - AQ, v = wave + 4 * u;
            if constexpr (BX4)
                lds_dma16s(b_tile + (long long)k0 * p.ldb, boff[u], bs_base + 4u * (unsigned)(buf * SB + v * 256));
            else
                lds_dma4s(b_tile + (long long)k0 * p.ldb, boff[u], bs_base + 4u * (unsigned)(buf * SB + v * 64));
        }
    };
    // A stage whose k may be negative (the prologue only): a lane with
    // k < 0 writes zeros to its own destination instead of copying; the
    // others fold k0 into their offset, which stays >= 0.  Every word of the
    // stage is the destination of exactly one lane, so the zeros need no
    // barrier of their own before the copies.
    auto zero_dst = [&](unsigned base, bool x4) {
        if (x4)
            *reinterpret_cast<__attribute__((address_space(3))) c_f4*>((size_t)(base + 16u * (unsigned)lane)) =
                c_f4{0.f, 0.f, 0.f, 0.f};
        else
            *reinterpret_cast<__attribute__((address_space(3))) float*>((size_t)(base + 4u * (unsigned)lane)) = 0.f;
    };
    auto issue_dma_masked = [&](int d, int k0, int buf) {
        if (d < AQ) {
            const int v = wave + 4 * d;
            const unsigned dst = as_base + 4u * (unsigned)(buf * SA + v * (AX4 ? 256 : 64));
            if (k0 + akk[d] < 0) {
                zero_dst(dst, AX4);
                return;
            }
            const unsigned off = aoff[d] + 4u * (unsigned)k0;
            if constexpr (AX4)
                lds_dma16s(a_tile, off, dst);
            else
                lds_dma4s(a_tile, off, dst);
        } else {
            const int u = d - AQ, v = wave + 4 * u;
            const unsigned dst = bs_base + 4u * (unsigned)(buf * SB + v * (BX4 ? 256 : 64));
            if (k0 + bkk[u] < 0) {
                zero_dst(dst, BX4);
                return;
            }
            const unsigned off = boff[u] + 4u * (unsigned)k0 * (unsigned)p.ldb;
            if constexpr (BX4)
                lds_dma16s(b_tile, off, dst);
            else
                lds_dma4s(b_tile, off, dst);
        }
    };
    auto barrier = [&](int inflight) {
        asm volatile("" ::: "memory");
        wait_vmcnt(inflight);
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };

    floatx4 acc[FBM][FBN];
#pragma unroll
    for (int i = 0; i < FBM; ++i)
#pragma unroll
        for (int j = 0; j < FBN; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
    // Zeroed accumulators -> first MFMA reads (SrcC): the empty statements
    // pin the zeroing before the pause (volatile asm keeps its order).
#pragma unroll
    for (int i = 0; i < FBM; ++i)
#pragma unroll
        for (int j = 0; j < FBN; ++j) asm volatile("" : "+a"(acc[i][j]));
    asm volatile("s_nop 7");

    // Operands.  Av[x][i] = A[wm + 16i + li][4q .. 4q+3] of the sub-slab
    // with global parity x; Bv[x][jb] = B[4q + s][wn + 64jb + 4li .. +3] of
    // the step with parity x, and for the float2 group (jb = NB4)
    // B[4q + s][wn + 64 NB4 + 2li .. +1] in its first two components.
    constexpr int NB4 = Cfg::NB4;
    float4 Av[2][FBM], Bv[2][NB];
    int a_off[FBM];
#pragma unroll
    for (int i = 0; i < FBM; ++i) {
        const int r = wm + 16 * i + li;
        a_off[i] = r * 16 + 4 * (q ^ swz_big(r));
    }
    const int b_off = 4 * q * BN + wn + 4 * li;
    // sub-slab g of buffer buf; step s (0..3) of that sub-slab
    auto read_a = [&](int buf, int g, int x, int i) {
        Av[x][i] = *reinterpret_cast<const float4*>(As + buf * SA + g * BM * 16 + a_off[i]);
    };
    auto read_b = [&](int buf, int g, int s, int jb) {
        if (jb < NB4) {
            Bv[s & 1][jb] = *reinterpret_cast<const float4*>(
                Bs + buf * SB + (16 * g + s) * BN + b_off + 64 * jb);
        } else {
            const float2 h2 = *reinterpret_cast<const float2*>(
                Bs + buf * SB + (16 * g + s) * BN + b_off - 2 * li + 64 * NB4);
            Bv[s & 1][jb].x = h2.x;
            Bv[s & 1][jb].y = h2.y;
        }
    };
    // The NMF MFMAs of one step (A parity xa, step s of its sub-slab),
    // op(n) issued before MFMA n, a fence after each.
    auto step_mma = [&](int xa, int s, auto&& op) {
        static_for<FBM>([&](auto I) {
            static_for<FBN>([&](auto J) {
                constexpr int i = decltype(I)::value, j = decltype(J)::value;
                op(FBN * i + j);
                const float4 a4 = Av[xa][i];
                const float av = s == 0 ? a4.x : s == 1 ? a4.y : s == 2 ? a4.z : a4.w;
                // block j < 4 NB4: component j % 4 of float4 group j / 4;
                // else component j - 4 NB4 of the float2 group
                constexpr int jb = j < 4 * NB4 ? j >> 2 : NB4;
                constexpr int e = j < 4 * NB4 ? j & 3 : j - 4 * NB4;
                const float4 b4 = Bv[s & 1][jb];
                const float bv = e == 0 ? b4.x : e == 1 ? b4.y : e == 2 ? b4.z : b4.w;
                asm volatile("v_mfma_f32_16x16x4_f32 %0, %1, %2, %0"
                             : "+a"(acc[i][j]) : "v"(av), "v"(bv));
                __builtin_amdgcn_sched_barrier(0);
            });
        });
    };

    // Stage t covers k = t KST - shift ..; nst is even.
    const int nst = (p.K + shift) / KST;

    // Fused form with beta != 0: the previous values of the lane's outputs
    // are loaded during the last stage (CPRE), one per MFMA of its first
    // step, so that their latency overlaps the stage's MFMAs instead of
    // following them.  Buffer loads address them from the tile's corner: a
    // per-lane byte offset fixed before the loop plus a scalar offset per
    // row and column group, so no vector instruction joins the MFMAs; a read
    // past the end of C returns zero and belongs to an output that is not
    // stored.  The 256 x 256 tile has no registers to spare and reads C at
    // the store.
    constexpr bool CPRE = EPI && CX4 && BM != 256 && Cfg::NB2 == 0;
    constexpr int NCP = CPRE ? FBM * 4 * NB : 1;
    static_assert(!CPRE || NCP <= NMF, "one prefetch per MFMA of a step");
    floatx4 cpre[NCP];
    bool do_cpre = false;
    unsigned coff = 0;
    long long cspan = 0;   // bytes from the tile's corner to the end of C's last row
    if constexpr (CPRE) {
        do_cpre = p.beta != 0.f && p.ldc < (1 << 22);
        if (do_cpre) {
            cspan = 4 * ((long long)(M - 1 - m0) * p.ldc + (N - n0));
            coff = 4u * ((unsigned)(4 * q) * (unsigned)p.ldc + (unsigned)(wn + 4 * li));
        }
    }
    // (a zero-range descriptor when there is nothing to prefetch)
    const __amdgpu_buffer_rsrc_t crsrc = __builtin_amdgcn_make_buffer_rsrc(
        p.C + (long long)m0 * p.ldc + n0, 0,
        (int)(cspan < 0xFFFFFFFFll ? cspan : 0xFFFFFFFFll), 0x00020000);
    // prefetch n of the lane: row block n / 4NB, register (n / NB) % 4,
    // column group n % NB
    auto issue_c = [&](int n) {
        if constexpr (CPRE) {
            if (!do_cpre) return;
            const int i = n / (4 * NB), r = (n / NB) % 4, jb = n % NB;
            const unsigned soff = 4u * ((unsigned)(wm + 16 * i + r) * (unsigned)p.ldc + 64u * jb);
            // (nontemporal: C is read once, and its lines should not push
            // the stage's A and B out of the L2; 1024^3 fused 17.97 against
            // 18.24 us)
            cpre[n] = __builtin_bit_cast(
                floatx4, __builtin_amdgcn_raw_buffer_load_b128(crsrc, (int)coff, (int)soff, 2));
        }
    };

    // Stage tt sits in buffer h = tt % 2.  `dma`: the stage issues the DMA of
    // stage tt + 1 (early: into buffer h ^ 1, which the barrier ending stage
    // tt - 1 freed) or of stage tt + 2 (late: into buffer h, after this
    // stage's own barrier); `more`: a stage follows.  Stages from 2 on start
    // at k >= 0.
    auto stage = [&](auto h_c, auto dma_c, auto more_c, int tt) {
        constexpr int h = decltype(h_c)::value;
        constexpr bool dma = decltype(dma_c)::value, more = decltype(more_c)::value;
        static_for<STEPS>([&](auto SG) {
            constexpr int sg = decltype(SG)::value;
            constexpr int g = sg >> 2, s = sg & 3;
            constexpr int xa = (SUBS * h + g) & 1;   // A parity of this sub-slab
            constexpr bool last = sg == STEPS - 1;
            if constexpr (!last) {
                step_mma(xa, s, [&](int n) {
                    // the last stage's first step: C's previous values
                    if (CPRE && !more && sg == 0 && n < NCP) issue_c(n);
                    if (!Cfg::LATE && dma && sg < Cfg::dsteps(AX4, BX4)) {
                        const int m = sg * NMF + n;
                        if (m % DGAP == 0 && m / DGAP < NDMA)
                            issue_dma(m / DGAP, (tt + 1) * KST - shift, h ^ 1);
                    }
                    // next step's B (same stage)
                    if (n >= RB && n < RB + NB) read_b(h, (sg + 1) >> 2, (sg + 1) & 3, n - RB);
                    // next sub-slab's A, in the last step of this one
                    if (s == 3 && n >= RB + NB && n < RB + NB + FBM) read_a(h, g + 1, xa ^ 1, n - RB - NB);
                });
            } else {
                // after the barrier, every OS-th MFMA: the next stage's first
                // B and A, then (late) the DMA of stage tt + 2
                step_mma(xa, s, [&](int n) {
                    if (more && n == PRE) barrier(0);   // only stage tt + 1 was in flight
                    const int m = n - PRE - 1;
                    if (m < 0 || m % OS) return;
                    const int x = m / OS;
                    if (more && x < NB) read_b(h ^ 1, 0, 0, x);
                    else if (more && x < NB + FBM) read_a(h ^ 1, 0, xa ^ 1, x - NB);
                    else if (Cfg::LATE && dma && x < NB + FBM + NDMA)
                        issue_dma(x - NB - FBM, (tt + 2) * KST - shift, h);
                });
            }
        });
    };
    using H0 = std::integral_constant<int, 0>;
    using H1 = std::integral_constant<int, 1>;
    using T = std::true_type;
    using F = std::false_type;
    if (nst > 0) {
        if (shift > 0) {
            // The first stages reach below k = 0: their lanes of negative k
            // write zeros, the others copy.  As without a shift, stage 0 is
            // waited for and stage 1's copy lands while stage 0 multiplies
            // (the barrier ending stage 0 waits for it).  A copy whose lanes
            // are all off is not issued at all, so the wait allows NDMA in
            // flight: when stage 0 holds real k (shift < KST) stage 1 issues
            // all NDMA and stage 0 has landed; when it lies wholly below
            // k = 0 it is all zeros and nothing of it is waited for.
#pragma unroll
            for (int d = 0; d < NDMA; ++d) issue_dma_masked(d, -shift, 0);
#pragma unroll
            for (int d = 0; d < NDMA; ++d) issue_dma_masked(d, KST - shift, 1);
            barrier(NDMA);
        } else {
#pragma unroll
            for (int d = 0; d < NDMA; ++d) issue_dma(d, 0, 0);
#pragma unroll
            for (int d = 0; d < NDMA; ++d) issue_dma(d, KST, 1);
            barrier(NDMA);
        }
#pragma unroll
        for (int jb = 0; jb < NB; ++jb) read_b(0, 0, 0, jb);
#pragma unroll
        for (int i = 0; i < FBM; ++i) read_a(0, 0, 0, i);
        if constexpr (Cfg::LATE) {
            // stage t issues stage t + 2's DMA: every pair but the last
            int t = 0;
            for (; t + 2 < nst; t += 2) {
                stage(H0{}, T{}, T{}, t);
                stage(H1{}, T{}, T{}, t + 1);
            }
            stage(H0{}, F{}, T{}, t);
            stage(H1{}, F{}, F{}, t + 1);
        } else {
            // stage t issues stage t + 1's DMA (stage 1's came with stage 0's);
            // an odd stage count (ODD, an instance of its own) ends with one
            // more stage, in buffer 0
            stage(H0{}, F{}, T{}, 0);
            int t = 1;
            for (; t + 2 < nst; t += 2) {
                stage(H1{}, T{}, T{}, t);
                stage(H0{}, T{}, T{}, t + 1);
            }
            if constexpr (ODD) {
                stage(H1{}, T{}, T{}, t);
                stage(H0{}, F{}, F{}, t + 1);
            } else {
                stage(H1{}, F{}, F{}, t);
            }
        }
    }
    // Last MFMAs -> accumulator reads: 24 wait states (an 8-pass MFMA's
    // result needs 11); each accumulator is read only after the pause.
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");
#pragma unroll
    for (int i = 0; i < FBM; ++i)
#pragma unroll
        for (int j = 0; j < FBN; ++j) asm volatile("" : "+a"(acc[i][j]));

    // Store: block (i, j) register r of lane (q, li) is C row
    // wm + 16i + 4q + r; for j < 4 NB4 column wn + 64(j/4) + 4li + j%4 --
    // four consecutive columns per column group jb = j/4 -- and for the
    // float2 group (jb = NB4) column wn + 64 NB4 + 2li + (j - 4 NB4).  A
    // group's columns are stored as one float4 (float2) where C's rows are
    // 16-byte aligned and N % 4 == 0 (the group is then inside C or wholly
    // outside it), else one by one, each guarded by col < N.
    // CX4: C's rows 16-byte aligned and N % 4 == 0 (the launcher checks)
    const bool whole = m0 + BM <= M && n0 + BN <= N;
    constexpr bool cvec = CX4;
    // group jb: its first column, its width and the accumulator block of
    // its first column
    auto gcol = [&](int jb) { return n0 + wn + 64 * jb + (jb < NB4 ? 4 : 2) * li; };
    auto gwidth = [&](int jb) { return jb < NB4 ? 4 : 2; };
    auto gblock = [&](int jb) { return 4 * jb; };
    // Fused form: the bias of the lane's columns is loaded once, and C's
    // previous values (beta != 0) for CG row blocks at a time are all
    // loaded before any of those outputs is stored, so the loads' latencies
    // overlap instead of following one another (C stores and loads go
    // through one pointer, so their program order is kept).  CG keeps the
    // group's values within 16 float4 registers.  The 256 x 256 tile, whose
    // registers are nearly all in use, keeps a plain guarded store per
    // float4 and, fused, reads each float4 of C just before its store (a
    // longer live range there moved a register copy into its main loop).
    if constexpr (BM == 256) {
        static_assert(Cfg::NB2 == 0, "float4 column groups only");
#pragma unroll
        for (int i = 0; i < FBM; ++i) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int jb = 0; jb < NB; ++jb) {
                    const int row = m0 + wm + 16 * i + 4 * q + r;
                    const int col = n0 + wn + 64 * jb + 4 * li;
                    if (!whole && (row >= M || col >= N)) continue;
                    float* cp = p.C + (long long)row * p.ldc + col;
                    float v[4] = {acc[i][4 * jb][r], acc[i][4 * jb + 1][r],
                                  acc[i][4 * jb + 2][r], acc[i][4 * jb + 3][r]};
                    const int ne = whole || col + 4 <= N ? 4 : N - col;
                    if constexpr (EPI) {
                        float c_in[4] = {0.f, 0.f, 0.f, 0.f}, bias[4] = {0.f, 0.f, 0.f, 0.f};
                        if (p.beta != 0.f) {
                            if constexpr (cvec) {
                                const float4 c4 = *reinterpret_cast<const float4*>(cp);
                                c_in[0] = c4.x; c_in[1] = c4.y; c_in[2] = c4.z; c_in[3] = c4.w;
                            } else {
#pragma unroll
                                for (int e = 0; e < 4; ++e)
                                    if (e < ne) c_in[e] = cp[e];
                            }
                        }
                        if (p.bias) {
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                if (e < ne) bias[e] = p.bias[col + e];
                        }
#pragma unroll
                        for (int e = 0; e < 4; ++e) v[e] = fused_out(p, v[e], c_in[e], bias[e]);
                    }
                    if constexpr (cvec) {
                        store_c4(cp, v[0], v[1], v[2], v[3]);
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (e < ne) store_c(cp + e, v[e]);
                    }
                }
            __builtin_amdgcn_sched_barrier(0);
        }
        return;
    }
    constexpr int CG = !EPI ? FBM : (4 * NB * FBM <= 16 ? FBM : (16 / (4 * NB) > 0 ? 16 / (4 * NB) : 1));
    static_assert(FBM % CG == 0, "whole groups of row blocks");
    // Addresses: the row m0 + wm + 16 i + r is wave-uniform (scalar), and
    // each lane adds its own offset of 4q rows and its group's columns,
    // fixed for the whole store.
    long long loff[NB];
#pragma unroll
    for (int jb = 0; jb < NB; ++jb) loff[jb] = (long long)(4 * q) * p.ldc + (gcol(jb) - n0);
    auto optr = [&](int i, int r, int jb) {
        return p.C + ((long long)(m0 + wm + 16 * i + r) * p.ldc + n0) + loff[jb];
    };
    // The fused form without branches: x = fma(beta', c, alpha s) + b, then
    // x < t ? 0 : x.  An absent term adds -0.0, which leaves every value
    // unchanged (-0.0 and NaN included): when beta == 0, C is not read,
    // c = +0 and beta' = -0.0, so the product term is -0.0; without a bias,
    // b = -0.0.  ReLU compares with t = 0 (-0.0 < 0 is false, NaN passes),
    // the identity with t = -Inf (never true).
    const float alpha = p.alpha, beta_e = p.beta != 0.f ? p.beta : -0.f;
    const bool read_c = EPI && p.beta != 0.f;
    const float relu_t = EPI && p.act == 1 ? 0.f : -__builtin_inff();
    float bias[NB][4];
#pragma unroll
    for (int jb = 0; jb < NB; ++jb)
#pragma unroll
        for (int e = 0; e < 4; ++e) bias[jb][e] = -0.f;
    if constexpr (EPI) {
        if (p.bias) {
#pragma unroll
            for (int jb = 0; jb < NB; ++jb)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int col = gcol(jb) + e;
                    if (e < gwidth(jb) && col < N) bias[jb][e] = p.bias[col];
                }
        }
    }
    // WHOLE_c: the tile lies inside C (no guards); else each output is
    // guarded by row < M and col < N.
    auto store_groups = [&](auto WHOLE_c) {
        constexpr bool WH = decltype(WHOLE_c)::value;
        static_for<FBM / CG>([&](auto G_c) {
            constexpr int i0 = decltype(G_c)::value * CG;
            constexpr int CGI = CPRE ? 1 : CG;   // c_in unused with the prefetch
            float c_in[CGI][4][NB][4];
#pragma unroll
            for (int ii = 0; ii < CGI; ++ii)
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int jb = 0; jb < NB; ++jb)
#pragma unroll
                        for (int e = 0; e < 4; ++e) c_in[ii][r][jb][e] = 0.f;
            if (!CPRE && read_c) {
#pragma unroll
                for (int ii = 0; ii < CG; ++ii)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
#pragma unroll
                        for (int jb = 0; jb < NB; ++jb) {
                            const int row = m0 + wm + 16 * (i0 + ii) + 4 * q + r;
                            const int col = gcol(jb), w = gwidth(jb);
                            if (!WH && (row >= M || col >= N)) continue;
                            const float* cp = optr(i0 + ii, r, jb);
                            if (cvec && w == 4) {
                                const floatx4 c4 = *reinterpret_cast<const floatx4*>(cp);
                                c_in[ii][r][jb][0] = c4[0]; c_in[ii][r][jb][1] = c4[1];
                                c_in[ii][r][jb][2] = c4[2]; c_in[ii][r][jb][3] = c4[3];
                            } else if (cvec) {
                                const float2 c2 = *reinterpret_cast<const float2*>(cp);
                                c_in[ii][r][jb][0] = c2.x; c_in[ii][r][jb][1] = c2.y;
                            } else {
                                const int ne = WH || col + w <= N ? w : N - col;
#pragma unroll
                                for (int e = 0; e < 4; ++e)
                                    if (e < ne) c_in[ii][r][jb][e] = cp[e];
                            }
                        }
            }
#pragma unroll
            for (int ii = 0; ii < CG; ++ii) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int jb = 0; jb < NB; ++jb) {
                        const int i = i0 + ii;
                        const int row = m0 + wm + 16 * i + 4 * q + r;
                        const int col = gcol(jb), w = gwidth(jb), j0 = gblock(jb);
                        if (!WH && (row >= M || col >= N)) continue;
                        float* cp = optr(i, r, jb);
                        float v[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) v[e] = e < w ? acc[i][j0 + e][r] : 0.f;
                        if constexpr (EPI) {
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                const float cv = CPRE ? cpre[CPRE ? ((i0 + ii) * 4 + r) * NB + jb : 0][e]
                                                      : c_in[CPRE ? 0 : ii][r][jb][e];
                                float x = __builtin_fmaf(beta_e, cv, alpha * v[e]);
                                x = x + bias[jb][e];
                                v[e] = x < relu_t ? 0.f : x;
                            }
                        }
                        // columns col .. col + ne - 1 are inside C
                        const int ne = WH || col + w <= N ? w : N - col;
                        if (cvec && w == 4) {
                            store_c4(cp, v[0], v[1], v[2], v[3]);
                        } else if (cvec) {
                            store_c2(cp, v[0], v[1]);
                        } else {
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                if (e < ne) store_c(cp + e, v[e]);
                        }
                    }
            }
            // one group at a time, so the fused form does not hold all of
            // C's previous values in registers at once
            __builtin_amdgcn_sched_barrier(0);
        });
    };
    // C's previous values: with the prefetch (CPRE) they stay in cpre --
    // loaded during the last stage, or here when the prefetch could not
    // address them, or +0 when C is not read -- so that no second copy is
    // live; else the groups load them into c_in.
    if constexpr (CPRE) {
        if (!read_c) {
#pragma unroll
            for (int n = 0; n < NCP; ++n) cpre[n] = floatx4{0.f, 0.f, 0.f, 0.f};
        } else if (!do_cpre) {
#pragma unroll
            for (int i = 0; i < FBM; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int jb = 0; jb < NB; ++jb) {
                        const int row = m0 + wm + 16 * i + 4 * q + r;
                        const int n = (i * 4 + r) * NB + jb;
                        cpre[n] = floatx4{0.f, 0.f, 0.f, 0.f};
                        if (!whole && (row >= M || gcol(jb) >= N)) continue;
                        cpre[n] = *reinterpret_cast<const floatx4*>(optr(i, r, jb));
                    }
        }
    }
    if (whole)
        store_groups(std::true_type{});
    else
        store_groups(std::false_type{});
}

// Rows of B and C 16-byte aligned, N a multiple of 4 (whole float4 columns).
// Leading dimensions below 2^22 keep a lane's byte offset from its tile's
// base (at most 256 rows of A, 64 rows of B) within 32 bits.  Any
// alignment and any N: 16-byte rows take the 16-byte DMA form, others the
// 4-byte form, and C is stored by float4 or one by one.
bool big_fits(const GemmArgs& a) {
    return a.lda < (1 << 22) && a.ldb < (1 << 22);
}
// The k shift: the stages start at k = -shift and end exactly at K, in
// whole pairs, or in configurations built for odd counts any count of at
// least two (the shift then stays below one stage).
template <class Cfg>
int big_shift(int K) {
    const int pair = (2 * Cfg::KST - K % (2 * Cfg::KST)) % (2 * Cfg::KST);
    if constexpr (Cfg::ODD) {
        const int one = (Cfg::KST - K % Cfg::KST) % Cfg::KST;
        if ((K + one) / Cfg::KST >= 2) return one;
    }
    return pair;
}
// Share of the MFMA work that is real k (the zeroed k below 0 are work too).
template <class Cfg>
double big_k_eff(const GemmArgs& a) {
    if (a.K <= 0) return 0.0;
    return (double)a.K / (double)(a.K + big_shift<Cfg>(a.K));
}
// A by the 16-byte DMA: rows aligned and k chunks never straddling k = 0.
bool big_a_x4(const GemmArgs& a) {
    return (a.lda % 4 == 0) && ((reinterpret_cast<uintptr_t>(a.A) & 15) == 0) && a.K % 4 == 0;
}
// B by the 16-byte DMA: rows aligned and N % 4 == 0, so no chunk reaches
// past column N - 1 (the last row of B may end there).
bool big_b_x4(const GemmArgs& a) {
    return (a.ldb % 4 == 0) && ((reinterpret_cast<uintptr_t>(a.B) & 15) == 0) && a.N % 4 == 0;
}
// The instance for the shape's DMA forms is built.
template <class Cfg>
bool big_forms_ok(const GemmArgs& a) {
    return Cfg::fits(big_a_x4(a), big_b_x4(a));
}

template <class Cfg, bool AX4, bool BX4, bool CX4, bool ODD>
hipError_t launch_big_odd(const GemmArgs& a, dim3 grid, dim3 block, int tiles_m, int tiles_n,
                          int shift, hipStream_t stream) {
    // The 64 x 96 tile's two stages take 40 KB of LDS, which lets four
    // workgroups share a CU, against the two waves per SIMD its registers
    // are budgeted for.  From K = 2048 the launch reserves unused dynamic
    // LDS up to 80 KB a workgroup, so that at most two do: 3072^3 130 ->
    // 146 TFLOP/s, 3072 x 3072 x 4096 131 -> 150, 3072 x 3072 x 2048 144 ->
    // 148.  At shorter K the extra workgroups overlap one another's prologue
    // and store and stay (5000 x 5000 x 1000: 137 against 132 capped,
    // 2000 x 2000 x 600 127 against 122), and the 64 x 64 tile (32 KB)
    // loses a little capped (2560^3 133 against 132).
    constexpr size_t kStatic = 2 * (Cfg::SA + Cfg::SB) * sizeof(float);
    constexpr bool kCap = Cfg::BM == 64 && Cfg::BN == 96 && kStatic < 80 * 1024;
    const size_t extra = (kCap && a.K >= 2048) ? 80 * 1024 - kStatic : 0;
    if (a.epi)
        hipLaunchKernelGGL((sgemm_mfma_big_kernel<Cfg, AX4, BX4, CX4, true, ODD>), grid, block, extra, stream, a,
                           tiles_m, tiles_n, shift);
    else
        hipLaunchKernelGGL((sgemm_mfma_big_kernel<Cfg, AX4, BX4, CX4, false, ODD>), grid, block, extra, stream, a,
                           tiles_m, tiles_n, shift);
    return hipGetLastError();
}

template <class Cfg, bool AX4, bool BX4, bool CX4>
hipError_t launch_big_forms(const GemmArgs& a, dim3 grid, dim3 block, int tiles_m, int tiles_n,
                            int shift, hipStream_t stream) {
    if constexpr (!Cfg::fits(AX4, BX4)) {
        return hipErrorInvalidValue;
    } else {
        if constexpr (Cfg::ODD) {
            if ((a.K + shift) / Cfg::KST % 2 == 1)
                return launch_big_odd<Cfg, AX4, BX4, CX4, true>(a, grid, block, tiles_m, tiles_n, shift, stream);
        }
        return launch_big_odd<Cfg, AX4, BX4, CX4, false>(a, grid, block, tiles_m, tiles_n, shift, stream);
    }
}

template <class Cfg>
hipError_t launch_big_cfg(const GemmArgs& a, hipStream_t stream) {
    if (!big_fits(a) || !big_forms_ok<Cfg>(a) || a.K <= 0) return hipErrorInvalidValue;
    const int tiles_m = (a.M + Cfg::BM - 1) / Cfg::BM, tiles_n = (a.N + Cfg::BN - 1) / Cfg::BN;
    const int shift = big_shift<Cfg>(a.K);
    const dim3 grid((unsigned)(tiles_m * tiles_n)), block(Cfg::NT);
    // float4 stores of C where its rows are aligned and N % 4 == 0 (B's
    // 16-byte form implies the latter); the 4-byte B form stores one by one
    const bool ax4 = big_a_x4(a), bx4 = big_b_x4(a);
    const bool cx4 = (a.ldc % 4 == 0) && ((reinterpret_cast<uintptr_t>(a.C) & 15) == 0) && a.N % 4 == 0;
    if (ax4 && bx4 && cx4) return launch_big_forms<Cfg, true, true, true>(a, grid, block, tiles_m, tiles_n, shift, stream);
    if (ax4 && bx4) return launch_big_forms<Cfg, true, true, false>(a, grid, block, tiles_m, tiles_n, shift, stream);
    if (ax4) return launch_big_forms<Cfg, true, false, false>(a, grid, block, tiles_m, tiles_n, shift, stream);
    if (bx4 && cx4) return launch_big_forms<Cfg, false, true, true>(a, grid, block, tiles_m, tiles_n, shift, stream);
    if (bx4) return launch_big_forms<Cfg, false, true, false>(a, grid, block, tiles_m, tiles_n, shift, stream);
    return launch_big_forms<Cfg, false, false, false>(a, grid, block, tiles_m, tiles_n, shift, stream);
}

template <class Cfg, bool EPI>
hipError_t launch_variant(const GemmArgs& a, bool va, bool vb, dim3 grid, dim3 block,
                          int tiles_m, int tiles_n, hipStream_t stream) {
    if (va && vb)
        hipLaunchKernelGGL((sgemm_mfma_kernel<Cfg, true, true, EPI>), grid, block, 0, stream, a, tiles_m, tiles_n);
    else if (va)
        hipLaunchKernelGGL((sgemm_mfma_kernel<Cfg, true, false, EPI>), grid, block, 0, stream, a, tiles_m, tiles_n);
    else if (vb)
        hipLaunchKernelGGL((sgemm_mfma_kernel<Cfg, false, true, EPI>), grid, block, 0, stream, a, tiles_m, tiles_n);
    else
        hipLaunchKernelGGL((sgemm_mfma_kernel<Cfg, false, false, EPI>), grid, block, 0, stream, a, tiles_m, tiles_n);
    return hipGetLastError();
}

template <class Cfg>
hipError_t launch_cfg(const GemmArgs& a, hipStream_t stream) {
    constexpr int BM = Cfg::BM, BN = Cfg::BN;
    const int tiles_m = (a.M + BM - 1) / BM;
    const int tiles_n = (a.N + BN - 1) / BN;
    const dim3 grid((unsigned)(tiles_m * tiles_n)), block(Cfg::NT);
    const bool va = (a.lda % 4 == 0) && ((reinterpret_cast<uintptr_t>(a.A) & 15) == 0);
    const bool vb = (a.ldb % 4 == 0) && ((reinterpret_cast<uintptr_t>(a.B) & 15) == 0);
    if (a.epi) return launch_variant<Cfg, true>(a, va, vb, grid, block, tiles_m, tiles_n, stream);
    return launch_variant<Cfg, false>(a, va, vb, grid, block, tiles_m, tiles_n, stream);
}

}  // namespace

// Tile table, chosen by interleaved timing on MI355X (256 CUs).  A grid of
// T tiles runs in rounds of about one tile per CU; a last round that is
// mostly empty wastes the largest tiles most.  So:
//  * the large wave-tile kernel (4 waves, 16x16x4 MFMAs, direct-to-LDS)
//    whenever its zeroed share of k is small enough (any alignment and any
//    N: rows that are not 16-byte aligned take the 4-byte DMA form, and C
//    is then stored one float at a time): of its 128x128, 256x256, 64x96
//    and 64x64 tiles the one with the best product of relative rate (1,
//    0.995, 0.97, 0.96), round fill and share of real k.  8192^3 153
//    TFLOP/s, 4096^3 151, 2048^3 144-146 and 6144^3 152 by 128x128; 1024^3
//    118-122, 3584^3 142, 5120^3 152, 3072^3 150 by 64x64; the ragged
//    1000x1500x777 105 by 64x96 (4-byte A DMA);
//  * otherwise (short K that is not a multiple of two stages, leading
//    dimensions of 2^22 or more):
//    256x256 register-staged tiles when their last round is at least 3/4
//    full; 64x64 register tiles when their grid fills its rounds so much
//    better than a 128x128 grid that it outweighs their lower efficiency
//    (0.85 of a 128x128 register tile's): 2000x3000x777 98.7 against 86.5;
//    else 128x128 tiles: register-staged (8 waves of 32x64, two workgroups
//    per CU) from 1.5 tiles per CU, 128x64 direct-to-LDS tiles between 1 and
//    1.5 per CU when whole and aligned, the direct-to-LDS 128x128 kernel at
//    3/4 to 1 per CU when whole and aligned;
//  * small grids: 64x64 tiles of 4 waves of 32x32, by DMA when A's and B's
//    rows are 16-byte aligned and M, N are whole tiles, split four ways in
//    K inside the workgroup (16 waves) when at most one tile per CU and
//    K >= 512 (+12-19 % over the unsplit kernel at 1024^3, 2048x512x2048,
//    4096x256x4096, 1024x1024x4096 before the large wave-tile kernel took
//    those shapes).  The split class runs the mid-stage barrier with four
//    stages; the 4-wave 64x64 and 8-wave 128x128 direct-to-LDS tiles keep
//    the end-of-stage barrier and separate interior and edge loops.
//    The register-staged fallback takes 64x96 tiles (6 waves) instead when
//    they fill their rounds better by more than 0.1 (1000x1500x777 with an
//    unaligned C, 700x2000x500, 1200^3: +2-4.5 %).
// Register-staged edge tiles cost no more than interior ones.
using MfmaLarge = MfmaCfg<256, 256, 16, 64, 64, 1>;
using MfmaMid = MfmaCfg<128, 128, 16, 32, 64, 2>;
using MfmaSmall = MfmaCfg<64, 64, 16, 32, 32, 2>;
using MfmaSmallWide = MfmaCfg<64, 96, 16, 32, 32, 2>;
using DmaMid = DmaCfg<128, 128, 32, 64, 2>;
using DmaMidHalf = DmaCfg<128, 64, 32, 32, 2>;
using DmaSmall = DmaCfg<64, 64, 32, 32, 2>;
using DmaSmallSplitK = DmaCfg<64, 64, 32, 32, 1, 4, 4, true>;
using BigLarge = BigCfg<256, 1, true>;
// 128x128 and 64x64 tiles: the early DMA over the first quarter of a
// stage (64x64: 1-10 % faster than over the first half, most at one tile
// per CU; 128x128: within 0.3 %)
using BigMid = BigCfg<128, 2, false, 4, 4, 4>;   // groups of 4 tile rows: +0.2-0.5 % at 2048^3 .. 8192^3
using BigSmall = BigCfg<64, 2, false, 1, 8, 4, 64, true>;
using BigSmallDeep = BigCfg<64, 4, false, 1, 8, 4>;
// 64 x 96 tiles (4 waves of 16 x 96, six blocks per step): where a grid of
// them fills its rounds better than 64 x 64 tiles (1000 x 1500: 256 tiles,
// one round, against 384)
using BigSmallWide = BigCfg<64, 2, false, 1, 8, 4, 96, true>;

static long long tiles_of(const GemmArgs& a, int bm, int bn) {
    return ((long long)a.M + bm - 1) / bm * (((long long)a.N + bn - 1) / bn);
}

// Share of the CU slots that a grid of t tiles keeps busy, one tile per CU
// per round: 1 when t is a multiple of the CU count, 0.75 for one and a half
// rounds.
static double fill_of(long long t, long long cus) {
    const long long rounds = (t + cus - 1) / cus;
    return (double)t / (double)(rounds * cus);
}

hipError_t launch_mfma(const GemmArgs& a, hipStream_t stream) {
    // the device's compute units (256 on a whole MI355X)
    const long long CUS = a.cus > 0 ? a.cus : 256;
    auto fill = [&](long long t) { return fill_of(t, CUS); };
    const bool aligned = rows_16b_aligned(a);
    const long long t256 = tiles_of(a, 256, 256), t128 = tiles_of(a, 128, 128);
    const long long t64 = tiles_of(a, 64, 64);
    // The large wave-tile kernel: of its 128x128, 256x256, 64x96 and 64x64
    // tiles the one whose grid keeps the CUs busiest, each weighed by its
    // rate when its rounds are full (1, 0.995, 0.97 and 0.96 of the 128
    // tile's, measured at 4096^3 .. 8192^3) and by its share of real k (the
    // k shifted below 0 are zeroed work; at least 3/4).  The register-staged kernels
    // below zero only the tail of their last slab; at short K they beat the
    // best large wave tile scoring under 0.65 of their own 128x128 grid's
    // fill (6000x6000x77: 79.5 TFLOP/s against 60.4 by 256x256 tiles;
    // 4096x4096x33: 42.5 against 39.6).  64x64 tiles take 64-k stages at
    // long K and, from K = 1024, on grids of at most one tile per CU, where
    // no second workgroup on the CU covers the DMA latency.
    auto score = [&](auto cfg, double rate, long long tiles) {
        using Cfg = decltype(cfg);
        if (!big_forms_ok<Cfg>(a)) return -1.0;
        const double eff = big_k_eff<Cfg>(a);
        return eff < 0.75 ? -1.0 : rate * fill(tiles) * eff;
    };
    const double s128 = score(BigMid{}, 1.0, t128);
    const double s256 = score(BigLarge{}, 0.995, t256);
    const double s64 = score(BigSmall{}, 0.96, t64);
    const double s96 = score(BigSmallWide{}, 0.97, tiles_of(a, 64, 96));
    const double sbest = std::max(std::max(s128, s256), std::max(s64, s96));
    if (big_fits(a) && sbest >= 0.65 * fill(t128)) {
        if (s128 > 0 && s128 >= sbest) return launch_big_cfg<BigMid>(a, stream);
        if (s256 > 0 && s256 >= sbest) return launch_big_cfg<BigLarge>(a, stream);
        if (s96 > 0 && s96 > s64) return launch_big_cfg<BigSmallWide>(a, stream);
        if (s64 > 0) {
            if (a.K >= 3072 || (t64 <= CUS && a.K >= 1024)) return launch_big_cfg<BigSmallDeep>(a, stream);
            return launch_big_cfg<BigSmall>(a, stream);
        }
    }
    const long long last_round = t256 % CUS;
    if (t256 >= 3 * CUS / 4 && (last_round == 0 || last_round >= 3 * CUS / 4))
        return launch_cfg<MfmaLarge>(a, stream);
    // 64x64 register tiles when they fill their rounds so much better that
    // it outweighs their lower per-tile efficiency (about 0.85 of a 128x128
    // register tile's: at 2560^3 the two tie at fills 0.78 and 0.89)
    const bool small_fills_better = 0.85 * fill(t64) > fill(t128);
    auto register_mid = [&] {
        if (small_fills_better) return launch_cfg<MfmaSmall>(a, stream);
        return launch_cfg<MfmaMid>(a, stream);
    };
    if (t128 >= 3 * CUS / 2) return register_mid();
    if (t128 > CUS) {
        if (aligned && a.M % 128 == 0 && a.N % 64 == 0) return launch_dma_cfg<DmaMidHalf>(a, stream);
        return register_mid();
    }
    if (t128 >= 3 * CUS / 4) {
        if (aligned && a.M % 128 == 0 && a.N % 128 == 0) return launch_dma_cfg<DmaMid>(a, stream);
        return register_mid();
    }
    if (aligned && a.M % 64 == 0 && a.N % 64 == 0) {
        if (t64 <= CUS && a.K >= 512) return launch_dma_cfg<DmaSmallSplitK>(a, stream);
        return launch_dma_cfg<DmaSmall>(a, stream);
    }
    if (fill(tiles_of(a, 64, 96)) > fill(t64) + 0.1) return launch_cfg<MfmaSmallWide>(a, stream);
    return launch_cfg<MfmaSmall>(a, stream);
}

}  // namespace sgemm
