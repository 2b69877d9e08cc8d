// sgemm_lowp.hip -- C = A.B with 16-bit floating-point A and B (bf16 or
// fp16) and fp32 accumulation and output, on the CDNA4 matrix cores.
//
// The pages tie the register/LDS tiling to tensor-core style matrix
// instructions and to half-precision inputs ("Register/Shared Memory
// Tiling", ryotta.opik.net: advantages item 3 and related technologies);
// this is that path on gfx950.  The tiling is the same as the fp32
// direct-to-LDS kernel: a workgroup owns a BM x BN tile of C, walks K in
// 32-deep stages streamed into LDS by global_load_lds_dwordx4 three stages
// deep, and each wave keeps a WM x WN sub-tile of fp32 accumulators.  The
// inner step is v_mfma_f32_32x32x16_{bf16,f16}: a rank-16 update of a 32x32
// block (16384 multiply-adds), fp32 accumulate.  Each product of two 16-bit
// values is exact in fp32, so results differ from the exact sum of the
// stored inputs only by fp32 rounding of the sums, as on the fp32 path.
//
// Operand layouts of v_mfma_f32_32x32x16_{bf16,f16} (wave64, four VGPRs of
// eight 16-bit values per operand):
//   A (32 x 16): lane l holds A[l % 32][8*(l/32) + e], e = 0..7
//   B (16 x 32): lane l holds B[8*(l/32) + e][l % 32]
//   D (32 x 32): as for v_mfma_f32_32x32x2_f32
// Stage s of 32 k is two MFMA steps; step t covers k = 16t .. 16t + 15.
//
// LDS, one array, A stages then B stages, 16-byte chunks XOR-swizzled:
//   A (BM x 32, rows of 64 bytes): chunk c of row r at c ^ (((r>>1)^(r>>3))&3).
//     A lane's operand is one chunk (8 consecutive k): one ds_read_b128;
//     eight consecutive rows of one chunk fall in distinct banks.
//   B (32 x BN, rows of 2*BN bytes): chunk c of row k at c ^ (4 * ((k>>3)&1)).
//     A lane's operand is 8 values down one column: eight ds_read_u16.  The
//     two lane halves read rows k and k + 8, which the swizzle places 64
//     bytes apart, so the 64 lanes of one read hit distinct banks.
// Tiles that cross the matrix edge, the K tail, and matrices whose rows are
// not 16-byte aligned take a register loader that zero-fills and writes the
// same layout.
#include "tiles.h"

namespace sgemm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));

template <int BM_, int BN_, int WM_, int WN_, int MINW_ = 1, int GROUP_M_ = 8>
struct LowpCfg {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, BK = 32;
    static constexpr int MINW = MINW_, GROUP_M = GROUP_M_;
    static constexpr int STAGES = 3;
    static constexpr bool XCD = true;
    static constexpr int WAVES_N = BN / WN;
    static constexpr int NW = (BM / WM) * (BN / WN);
    static constexpr int NT = NW * 64;
    static constexpr int FM = WM / 32, FN = WN / 32;
    static constexpr int CA = BK / 8;                  // 16-byte chunks per A row
    static constexpr int CB = BN / 8;                  // 16-byte chunks per B row
    static constexpr int A_INS = BM * CA / 64;         // DMA instructions per stage
    static constexpr int B_INS = BK * CB / 64;
    static constexpr int SA = BM * BK, SB = BK * BN;   // 16-bit elements per stage
    static_assert(BM % WM == 0 && BN % WN == 0 && WM % 32 == 0 && WN % 32 == 0, "tiles");
    static_assert((BM * CA) % 64 == 0 && (BK * CB) % 64 == 0, "whole DMA instructions");
    static_assert(BN % 64 == 0, "B swizzle flips chunk bit 2 inside 8-chunk groups");
    static_assert(STAGES * (SA + SB) * 2 <= 160 * 1024, "LDS budget of one CU");
    static_assert(NT <= 1024, "workgroup size");
};

__device__ __forceinline__ int swz_a(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }

// Same wave-wide DMA as the fp32 kernel: lane i copies 16 bytes from g into
// LDS at byte offset lds_base + 16 * i; M0 carries the base.
__device__ __forceinline__ void lds_dma16(const void* g, unsigned lds_base) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                 :: "v"(g), "s"(lds_base) : "memory", "m0");
}
__device__ __forceinline__ unsigned lds_addr(const void* p) {
    return (unsigned)(size_t)(__attribute__((address_space(3))) const void*)p;
}
__device__ __forceinline__ void wait_vmcnt(int n) {
    switch (n) {
        case 0: __builtin_amdgcn_s_waitcnt(0x0F70); break;
        case 1: __builtin_amdgcn_s_waitcnt(0x0F71); break;
        case 2: __builtin_amdgcn_s_waitcnt(0x0F72); break;
        case 3: __builtin_amdgcn_s_waitcnt(0x0F73); break;
        case 4: __builtin_amdgcn_s_waitcnt(0x0F74); break;
        case 5: __builtin_amdgcn_s_waitcnt(0x0F75); break;
        case 6: __builtin_amdgcn_s_waitcnt(0x0F76); break;
        case 7: __builtin_amdgcn_s_waitcnt(0x0F77); break;
        case 8: __builtin_amdgcn_s_waitcnt(0x0F78); break;
        default: __builtin_amdgcn_s_waitcnt(0x0F70); break;
    }
}

template <Lowp T>
__device__ __forceinline__ floatx16 mfma16(uint4 a, uint4 b, floatx16 c) {
    if constexpr (T == Lowp::bf16)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(halfx8, a),
                                                      __builtin_bit_cast(halfx8, b), c, 0, 0, 0);
}

// DMA: A's and B's rows are 16-byte aligned, so interior tiles stream by
// DMA; otherwise every stage goes through the register loader.
template <class Cfg, Lowp T, bool DMA>
__global__ __launch_bounds__(Cfg::NT, Cfg::MINW)
void gemm_lowp_kernel(LowpArgs p, int tiles_m, int tiles_n) {
    constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK, WM = Cfg::WM, WN = Cfg::WN;
    constexpr int NW = Cfg::NW, FM = Cfg::FM, FN = Cfg::FN, CA = Cfg::CA, CB = Cfg::CB;
    constexpr int SA = Cfg::SA, SB = Cfg::SB, STAGES = Cfg::STAGES;
    __shared__ __attribute__((aligned(16))) unsigned short lds[STAGES * (SA + SB)];
    unsigned short* const As = lds;
    unsigned short* const Bs = lds + STAGES * SA;

    int tm, tn;
    tile_coords(blockIdx.x, tiles_m, tiles_n, Cfg::GROUP_M, Cfg::XCD, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int M = p.M, N = p.N, K = p.K;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = (wave / Cfg::WAVES_N) * WM;
    const int wn = (wave % Cfg::WAVES_N) * WN;
    const int li = lane & 31, lh = lane >> 5;
    const unsigned short* __restrict__ Ablk = p.A + (long long)m0 * p.lda;
    const unsigned short* __restrict__ Bblk = p.B + n0;
    const int mrem = M - m0, nrem = N - n0;
    const bool mn_full = DMA && mrem >= BM && nrem >= BN;
    const int n_dma = (Cfg::A_INS % NW == 0 && Cfg::B_INS % NW == 0)
        ? Cfg::A_INS / NW + Cfg::B_INS / NW
        : (wave < Cfg::A_INS ? (Cfg::A_INS - wave + NW - 1) / NW : 0) +
          (wave < Cfg::B_INS ? (Cfg::B_INS - wave + NW - 1) / NW : 0);
    const unsigned as_base = lds_addr(As), bs_base = lds_addr(Bs);

    // Instruction q of a stage, lane l: chunk P = 64q + l of the operand,
    // written at byte 1024q + 16l of the stage.
    auto issue_full = [&](int k0, int st) {
        for (int q = wave; q < Cfg::A_INS; q += NW) {
            const int P = q * 64 + lane;
            const int r = P / CA, c = (P % CA) ^ swz_a(P / CA);
            lds_dma16(Ablk + (long long)r * p.lda + k0 + 8 * c,
                      __builtin_amdgcn_readfirstlane(as_base + 2u * (unsigned)(st * SA) + 1024u * q));
        }
        for (int q = wave; q < Cfg::B_INS; q += NW) {
            const int P = q * 64 + lane;
            const int k = P / CB, c = (P % CB) ^ (((k >> 3) & 1) << 2);
            lds_dma16(Bblk + (long long)(k0 + k) * p.ldb + 8 * c,
                      __builtin_amdgcn_readfirstlane(bs_base + 2u * (unsigned)(st * SB) + 1024u * q));
        }
    };
    // Register loader with zero fill for any stage; same placement.  Branch
    // free: an element outside the matrix is loaded from the matrix's first
    // element instead (always valid when there is a stage to load) and
    // replaced by zero.
    auto pack8 = [](const unsigned short (&v)[8]) {
        uint4 w;
        w.x = v[0] | ((unsigned)v[1] << 16); w.y = v[2] | ((unsigned)v[3] << 16);
        w.z = v[4] | ((unsigned)v[5] << 16); w.w = v[6] | ((unsigned)v[7] << 16);
        return w;
    };
    auto issue_edge = [&](int k0, int st) {
        for (int q = wave; q < Cfg::A_INS; q += NW) {
            const int P = q * 64 + lane;
            const int r = P / CA, c = (P % CA) ^ swz_a(P / CA);
            const int kg = k0 + 8 * c;
            const long long row = (long long)r * p.lda + kg;
            unsigned short v[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const bool in = r < mrem && kg + e < K;
                const unsigned short x = Ablk[in ? row + e : -(long long)m0 * p.lda];
                v[e] = in ? x : (unsigned short)0;
            }
            *reinterpret_cast<uint4*>(&As[st * SA + q * 512 + lane * 8]) = pack8(v);
        }
        for (int q = wave; q < Cfg::B_INS; q += NW) {
            const int P = q * 64 + lane;
            const int k = P / CB, c = (P % CB) ^ (((k >> 3) & 1) << 2);
            const int kg = k0 + k;
            const long long row = (long long)kg * p.ldb + 8 * c;
            unsigned short v[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const bool in = kg < K && 8 * c + e < nrem;
                const unsigned short x = Bblk[in ? row + e : -(long long)n0];
                v[e] = in ? x : (unsigned short)0;
            }
            *reinterpret_cast<uint4*>(&Bs[st * SB + q * 512 + lane * 8]) = pack8(v);
        }
    };
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

    // Operand addresses inside a stage (16-bit elements).  A: row
    // wm + 32i + li, chunk 2t + lh of step t.  B: rows 16t + 8lh + e of
    // column wn + 32j + li, whose chunk sits at (col >> 3) ^ (4 * lh).
    int a_row[FM], a_swz[FM], b_off[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        a_row[i] = (wm + i * 32 + li) * BK;
        a_swz[i] = swz_a(wm + i * 32 + li);
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int col = wn + j * 32 + li;
        b_off[j] = 8 * lh * BN + ((((col >> 3) ^ (lh << 2)) << 3) | (col & 7));
    }
    // One stage: two MFMA steps, each reading its operands just before it
    // multiplies (fewer live registers than reading both up front); later
    // stages are requested between the first step's reads and its MFMAs.
    auto compute = [&](int st, auto&& between) {
        const unsigned short* as = &As[st * SA];
        const unsigned short* bs = &Bs[st * SB];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            uint4 fa[FM], fb[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i)
                fa[i] = *reinterpret_cast<const uint4*>(&as[a_row[i] + 8 * ((2 * t + lh) ^ a_swz[i])]);
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const unsigned short* b = bs + b_off[j] + 16 * t * BN;
                fb[j].x = b[0 * BN] | ((unsigned)b[1 * BN] << 16);
                fb[j].y = b[2 * BN] | ((unsigned)b[3 * BN] << 16);
                fb[j].z = b[4 * BN] | ((unsigned)b[5 * BN] << 16);
                fb[j].w = b[6 * BN] | ((unsigned)b[7 * BN] << 16);
            }
            if (t == 0) between();
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] = mfma16<T>(fa[i], fb[j], acc[i][j]);
        }
    };

    if (mn_full) {
        // Interior tile: three stages by DMA, stage t + 2 requested while
        // stage t multiplies (as in the fp32 kernel).
        const int nfull = K / BK;
        if (nfull > 0) issue_full(0, 0);
        if (nfull > 1) issue_full(BK, 1);
        lds_barrier(nfull > 1 ? n_dma : 0);
        int st = 0;
        for (int t = 0; t < nfull; ++t) {
            const int st2 = st == 0 ? 2 : st - 1;
            const bool more = t + 2 < nfull;
            compute(st, [&] { if (more) issue_full((t + 2) * BK, st2); });
            lds_barrier(more ? n_dma : 0);
            st = st == 2 ? 0 : st + 1;
        }
        if (K % BK) {
            issue_edge(nfull * BK, 0);
            lds_barrier(0);
            compute(0, [] {});
        }
    } else {
        const int nstage = (K + BK - 1) / BK;
        for (int t = 0; t < nstage; ++t) {
            issue_edge(t * BK, 0);
            lds_barrier(0);
            compute(0, [] {});
            lds_barrier(0);
        }
    }
    store_tile<false, FM, FN>(p, acc, m0 + wm, n0 + wn, li, lh);
}

template <class Cfg, Lowp T>
hipError_t launch_lowp_cfg(const LowpArgs& a, hipStream_t stream) {
    const int tiles_m = (a.M + Cfg::BM - 1) / Cfg::BM;
    const int tiles_n = (a.N + Cfg::BN - 1) / Cfg::BN;
    const dim3 grid((unsigned)(tiles_m * tiles_n)), block(Cfg::NT);
    const bool dma = (a.lda % 8 == 0) && (a.ldb % 8 == 0) &&
                     ((reinterpret_cast<uintptr_t>(a.A) & 15) == 0) &&
                     ((reinterpret_cast<uintptr_t>(a.B) & 15) == 0);
    if (dma)
        hipLaunchKernelGGL((gemm_lowp_kernel<Cfg, T, true>), grid, block, 0, stream, a, tiles_m, tiles_n);
    else
        hipLaunchKernelGGL((gemm_lowp_kernel<Cfg, T, false>), grid, block, 0, stream, a, tiles_m, tiles_n);
    return hipGetLastError();
}

// Tile table, from interleaved timing of bf16 products on MI355X: 256x256
// tiles of 8 waves of 128x64 once the grid holds >= 256 of them (869
// TFLOP/s at 8192^3, 833 at 4096^3; 64x128 waves and 128x256 or 256x128
// tiles 5-15 % slower), else 128x128 tiles of 8 waves of 32x64, the most
// waves per CU for mid-size grids (488 TFLOP/s at 2048^3 against 370 for
// 4 waves of 64x64).
using LowpLarge = LowpCfg<256, 256, 128, 64, 1>;
using LowpMid = LowpCfg<128, 128, 32, 64, 2>;

template <Lowp T>
hipError_t launch_lowp_t(const LowpArgs& a, hipStream_t stream) {
    const long long tiles = ((long long)a.M + 255) / 256 * (((long long)a.N + 255) / 256);
    if (tiles >= 256) return launch_lowp_cfg<LowpLarge, T>(a, stream);
    return launch_lowp_cfg<LowpMid, T>(a, stream);
}

}  // namespace

hipError_t launch_lowp(const LowpArgs& a, Lowp type, hipStream_t stream) {
    return type == Lowp::bf16 ? launch_lowp_t<Lowp::bf16>(a, stream)
                              : launch_lowp_t<Lowp::f16>(a, stream);
}

}  // namespace sgemm
