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
// Stage s of 32 k is two MFMA steps.  The order of the k terms is free, so
// step t gives lane half h the k = 16h + 8t .. 16h + 8t + 7 of the stage
// (chunks t and t + 2 of an A row are read by the two halves together,
// which keeps their 16-byte reads in distinct banks).
//
// LDS, one array, A stages then B stages, 16-byte chunks XOR-swizzled:
//   A (BM x 32, rows of 64 bytes): chunk c of row r at c ^ (((r>>1)^(r>>3))&3).
//     A lane's operand is one chunk (8 consecutive k): one ds_read_b128;
//     eight consecutive rows of one chunk fall in distinct banks.
//   B (32 x BN, rows of 2*BN bytes): chunk c of row k at c ^ (4 * (k & 3)).
//     A lane's operand is 8 values down one column, gathered by two
//     ds_read_b64_tr_b16 (gfx950's transposing LDS read).  Within each group
//     of 16 lanes, result element e of lane i is element i % 4 of the 8
//     bytes addressed by lane 4e + i/4 of the group (checked on the GPU with
//     a one-wave probe).  So when lane 4e + j of group g addresses row
//     k + e, columns n + 4j .. n + 4j + 3, lane i of the group receives
//     B[k + e][n + i], e = 0..3: four k down its own column.  Groups 0-3 of
//     a read cover columns n, n + 16 and rows k, k + 16 (the two lane
//     halves).  Each half-wave of a read touches 4 rows (k .. k + 3), 64
//     bytes each; the swizzle puts them in the four 64-byte slots of the
//     256-byte bank window.  (A probe of the read alone on MI355X: no bank
//     conflicts this way, against 2-way with only k & 1 and 4-way with no
//     swizzle.)
// Tiles that cross the matrix edge, the K tail, and matrices whose rows are
// not 16-byte aligned take a register loader that zero-fills and writes the
// same layout.
#include "lds_dma.h"
#include "tiles.h"

namespace sgemm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;

// Four dwords read from a 4-byte aligned address.
typedef unsigned u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));

template <int BM_, int BN_, int WM_, int WN_, int MINW_ = 1, int STAGES_ = 3, int GROUP_M_ = 8>
struct LowpCfg {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, BK = 32;
    static constexpr int MINW = MINW_, GROUP_M = GROUP_M_;
    // LDS buffers; stage t + STAGES - 1 is requested while stage t multiplies.
    static constexpr int STAGES = STAGES_;
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
    static_assert(BN % 128 == 0, "B swizzle flips chunk bits 2-3 inside 16-chunk groups");
    static_assert(WN % 32 == 0, "B operand reads cover 32 columns");
    static_assert(STAGES * (SA + SB) * 2 <= 160 * 1024, "LDS budget of one CU");
    static_assert(NT <= 1024, "workgroup size");
    static_assert(STAGES >= 3, "the schedule keeps two stages ahead of the one being read");
};

__device__ __forceinline__ int swz_a(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }
// B rows k: chunk c sits at c ^ (4 * bswz(k)).
__device__ __forceinline__ int bswz(int k) { return k & 3; }


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
    tile_coords(blockIdx.x, tiles_m, tiles_n, Cfg::GROUP_M, Cfg::XCD ? p.xcds : 1, tm, tn);
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
    constexpr int n_dma = Cfg::A_INS / NW + Cfg::B_INS / NW;   // per wave per stage
    const unsigned as_base = lds_addr(As), bs_base = lds_addr(Bs);

    // Instruction q of a stage, lane l: chunk P = 64q + l of the operand,
    // written at byte 1024q + 16l of the stage.
    auto issue_full = [&](int k0, int st) {
        static_assert(Cfg::A_INS % NW == 0 && Cfg::B_INS % NW == 0, "whole DMA rounds");
#pragma unroll
        for (int u = 0; u < Cfg::A_INS / NW; ++u) {
            const int q = wave + u * NW;
            const int P = q * 64 + lane;
            const int r = P / CA, c = (P % CA) ^ swz_a(P / CA);
            lds_dma16(Ablk + (long long)r * p.lda + k0 + 8 * c,
                      __builtin_amdgcn_readfirstlane(as_base + 2u * (unsigned)(st * SA) + 1024u * q));
        }
#pragma unroll
        for (int u = 0; u < Cfg::B_INS / NW; ++u) {
            const int q = wave + u * NW;
            const int P = q * 64 + lane;
            const int k = P / CB, c = (P % CB) ^ (4 * bswz(k));
            lds_dma16(Bblk + (long long)(k0 + k) * p.ldb + 8 * c,
                      __builtin_amdgcn_readfirstlane(bs_base + 2u * (unsigned)(st * SB) + 1024u * q));
        }
    };
    // Register loader with zero fill for any stage; same placement.  Branch
    // free: an element outside the matrix is loaded from the matrix's first
    // element instead (always valid when there is a stage to load) and
    // replaced by zero when written to LDS.  load_* fill ea/eb, store_*
    // zero-fill and write one chunk.
    auto pack8 = [](const unsigned short (&v)[8]) {
        uint4 w;
        w.x = v[0] | ((unsigned)v[1] << 16); w.y = v[2] | ((unsigned)v[3] << 16);
        w.z = v[4] | ((unsigned)v[5] << 16); w.w = v[6] | ((unsigned)v[7] << 16);
        return w;
    };
    static_assert(Cfg::A_INS % NW == 0 && Cfg::B_INS % NW == 0, "whole loader rounds");
    constexpr int AE = Cfg::A_INS / NW, BE = Cfg::B_INS / NW;
    unsigned short ea[AE][8], eb[BE][8];
    auto a_chunk = [&](int u, int& r, int& c) {
        const int P = (wave + u * NW) * 64 + lane;
        r = P / CA;
        c = (P % CA) ^ swz_a(P / CA);
    };
    auto b_chunk = [&](int u, int& k, int& c) {
        const int P = (wave + u * NW) * 64 + lane;
        k = P / CB;
        c = (P % CB) ^ (4 * bswz(k));
    };
    auto load_a = [&](int u, int k0) {
        int r, c;
        a_chunk(u, r, c);
        const int kg = k0 + 8 * c;
        const long long row = (long long)r * p.lda + kg;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const bool in = r < mrem && kg + e < K;
            ea[u][e] = Ablk[in ? row + e : -(long long)m0 * p.lda];
        }
    };
    auto store_a = [&](int u, int k0, int st) {
        int r, c;
        a_chunk(u, r, c);
        unsigned short v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = r < mrem && k0 + 8 * c + e < K ? ea[u][e] : (unsigned short)0;
        *reinterpret_cast<uint4*>(&As[st * SA + (wave + u * NW) * 512 + lane * 8]) = pack8(v);
    };
    auto load_b = [&](int u, int k0) {
        int k, c;
        b_chunk(u, k, c);
        const int kg = k0 + k;
        const long long row = (long long)kg * p.ldb + 8 * c;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const bool in = kg < K && 8 * c + e < nrem;
            eb[u][e] = Bblk[in ? row + e : -(long long)n0];
        }
    };
    auto store_b = [&](int u, int k0, int st) {
        int k, c;
        b_chunk(u, k, c);
        unsigned short v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = k0 + k < K && 8 * c + e < nrem ? eb[u][e] : (unsigned short)0;
        *reinterpret_cast<uint4*>(&Bs[st * SB + (wave + u * NW) * 512 + lane * 8]) = pack8(v);
    };
    // A whole stage, chunk by chunk.
    auto issue_edge = [&](int k0, int st) {
#pragma unroll
        for (int u = 0; u < AE; ++u) { load_a(u, k0); store_a(u, k0, st); }
#pragma unroll
        for (int u = 0; u < BE; ++u) { load_b(u, k0); store_b(u, k0, st); }
    };
    // Unaligned rows, whole stages (k0 + BK <= K): a chunk's 16 bytes start
    // on a 2-byte boundary, so the loader reads the five dwords around them
    // (4-byte aligned) and shifts the chunk out with alignbit when it is
    // written.  Offsets are bytes from the operand's base rounded down to 4
    // bytes (32-bit: the loader needs lda, ldb < 2^22); a stage adds 2 k0
    // bytes to A's base and 2 k0 ldb to B's, both multiples of 4.  No read
    // leaves the matrix:
    //  * A rows past M read row M - 1 (they only reach rows of C past M);
    //  * a B chunk past N reads the tile's first chunk; in a tile that
    //    crosses N each of the five dwords is read only if it holds a byte
    //    of the chunk's columns below N, else the first dword again (the
    //    values past N only reach columns of C past N);
    //  * in a whole chunk every dword holds a byte of the chunk: one
    //    dwordx4 and the fifth dword only when the chunk starts mid-dword.
    const char* const a_al = reinterpret_cast<const char*>(Ablk) - (reinterpret_cast<uintptr_t>(Ablk) & 3);
    const char* const b_al = reinterpret_cast<const char*>(Bblk) - (reinterpret_cast<uintptr_t>(Bblk) & 3);
    unsigned fa_off[AE], fb_off[BE];   // chunk start, bytes from a_al / b_al
    unsigned fa[AE][5], fb[BE][5];     // the dwords in flight
#pragma unroll
    for (int u = 0; u < AE; ++u) {
        int r, c;
        a_chunk(u, r, c);
        r = min(r, mrem - 1);
        fa_off[u] = (unsigned)(reinterpret_cast<uintptr_t>(Ablk) & 3) + 2u * ((unsigned)r * (unsigned)p.lda + 8u * (unsigned)c);
    }
    // bytes of B chunk u below column N (16 in a whole chunk)
    auto b_valid = [&](int u) {
        int k, c;
        b_chunk(u, k, c);
        if (8 * c >= nrem) c = 0;
        return (unsigned)min(16, 2 * (nrem - 8 * c));
    };
#pragma unroll
    for (int u = 0; u < BE; ++u) {
        int k, c;
        b_chunk(u, k, c);
        if (8 * c >= nrem) c = 0;
        fb_off[u] = (unsigned)(reinterpret_cast<uintptr_t>(Bblk) & 3) + 2u * ((unsigned)k * (unsigned)p.ldb + 8u * (unsigned)c);
    }
    auto load_window = [](const char* base, unsigned off, unsigned (&w)[5]) {
        const unsigned lo = off & ~3u;
        const u32x4_a4 v = *reinterpret_cast<const u32x4_a4*>(base + lo);
        w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
        w[4] = *reinterpret_cast<const unsigned*>(base + lo + ((off & 2) ? 16u : 12u));
    };
    auto load_window_part = [](const char* base, unsigned off, unsigned valid, unsigned (&w)[5]) {
        const unsigned lo = off & ~3u;
#pragma unroll
        for (int i = 0; i < 5; ++i) {
            const unsigned at = lo + 4u * i < off + valid ? lo + 4u * i : lo;
            w[i] = *reinterpret_cast<const unsigned*>(base + at);
        }
    };
    auto window_chunk = [](unsigned off, const unsigned (&w)[5]) {
        const unsigned sh = (off & 2) * 8;
        return make_uint4(__builtin_amdgcn_alignbit(w[1], w[0], sh), __builtin_amdgcn_alignbit(w[2], w[1], sh),
                          __builtin_amdgcn_alignbit(w[3], w[2], sh), __builtin_amdgcn_alignbit(w[4], w[3], sh));
    };
    auto load_fast = [&](int k0) {
#pragma unroll
        for (int u = 0; u < AE; ++u) load_window(a_al + 2 * (long long)k0, fa_off[u], fa[u]);
        const char* const bk = b_al + 2 * (long long)k0 * p.ldb;
        if (nrem >= BN) {
#pragma unroll
            for (int u = 0; u < BE; ++u) load_window(bk, fb_off[u], fb[u]);
        } else {
#pragma unroll
            for (int u = 0; u < BE; ++u) load_window_part(bk, fb_off[u], b_valid(u), fb[u]);
        }
    };
    auto store_fast = [&](int st) {
#pragma unroll
        for (int u = 0; u < AE; ++u)
            *reinterpret_cast<uint4*>(&As[st * SA + (wave + u * NW) * 512 + lane * 8]) = window_chunk(fa_off[u], fa[u]);
#pragma unroll
        for (int u = 0; u < BE; ++u)
            *reinterpret_cast<uint4*>(&Bs[st * SB + (wave + u * NW) * 512 + lane * 8]) = window_chunk(fb_off[u], fb[u]);
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
    // wm + 32i + li, chunk 2lh + t of step t.  B: this lane is lane
    // 4e + j of group g = lane / 16 of a transposing read; it addresses row
    // 16(g / 2) + 8t + 4r + e (read r = 0, 1 of step t) at columns
    // wn + 32jb + 16(g % 2) + 4j .. + 3, whose chunk sits at
    // (col / 8) ^ (4 * bswz(row)), and bswz(row) = e.
    int a_row[FM], a_swz[FM], b_off[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        a_row[i] = (wm + i * 32 + li) * BK;
        a_swz[i] = swz_a(wm + i * 32 + li);
    }
    {
        const int g = lane >> 4, e = (lane >> 2) & 3, j = lane & 3;
        const int krow = 16 * (g >> 1) + e;
#pragma unroll
        for (int jb = 0; jb < FN; ++jb) {
            const int col = wn + 32 * jb + 16 * (g & 1) + 4 * j;
            b_off[jb] = krow * BN + ((((col >> 3) ^ (4 * bswz(krow))) << 3) | (col & 7));
        }
    }
    struct Frag {
        uint4 a[FM], b[FN];
    };
    auto read_frags = [&](const unsigned short* as, const unsigned short* bs, int t, Frag& f) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
            f.a[i] = *reinterpret_cast<const uint4*>(&as[a_row[i] + 8 * ((2 * lh + t) ^ a_swz[i])]);
#pragma unroll
        for (int jb = 0; jb < FN; ++jb) {
            const unsigned short* b = bs + b_off[jb] + 8 * t * BN;
            const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_shortx4*)(__attribute__((address_space(3))) const unsigned short*)b);
            const shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_shortx4*)(__attribute__((address_space(3))) const unsigned short*)(b + 4 * BN));
            const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
            f.b[jb] = make_uint4(l2.x, l2.y, h2.x, h2.y);
        }
    };
    auto mma = [&](const Frag& f) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int jb = 0; jb < FN; ++jb) acc[i][jb] = mfma16<T>(f.a[i], f.b[jb], acc[i][jb]);
    };
    // One pipeline for every tile, S = STAGES LDS buffers, D = S - 1 stages
    // requested ahead, one barrier per stage placed between the stage's two
    // MFMA steps.  Iteration t (stage t in buffer t % S; its step-0 operands
    // f0 already in registers):
    //   1. read step 1's operands f1 of stage t;
    //   2. request stage t + D into the buffer stage t - 1 used -- every
    //      wave finished reading stage t - 1 before the previous barrier;
    //   3. multiply step 0 (f0);
    //   4. wait until stage t + 1 has landed (stages t + 2 .. t + D may stay
    //      in flight), barrier, read its step-0 operands into f0 -- their
    //      latency hides behind
    //   5. multiply step 1 (f1).
    // Whole stages of interior tiles come by DMA and may stay in flight;
    // stages that cross an edge of the matrix (and every stage when rows are
    // unaligned) come through the register loader, which orders its LDS
    // writes by the next barrier; with unaligned rows the loop issues its
    // loads before step 0's MFMAs and writes them after.  A single multiply site per
    // step keeps the accumulators in one register class.
    constexpr int S = Cfg::STAGES, D = S - 1;
    const int nstage = (K + BK - 1) / BK;
    const int nfull = mn_full ? K / BK : 0;       // stages 0 .. nfull-1 by DMA
    // unaligned rows: the whole stages 0 .. nfast-1 by the dword-window loader
    // (elements on 2-byte boundaries: the window shifts by 0 or 16 bits)
    const bool fast_tile = !DMA && p.lda < (1 << 22) && p.ldb < (1 << 22) &&
                           ((reinterpret_cast<uintptr_t>(p.A) | reinterpret_cast<uintptr_t>(p.B)) & 1) == 0;
    const int nfast = fast_tile ? K / BK : 0;
    // debug build: the chunks of buffer st the register loaders write (the
    // DMA helpers poison their own destinations)
    auto poison_stage = [&](int st) {
#pragma unroll
        for (int u = 0; u < AE; ++u) lds_poison_f4(&As[st * SA + (wave + u * NW) * 512 + lane * 8]);
#pragma unroll
        for (int u = 0; u < BE; ++u) lds_poison_f4(&Bs[st * SB + (wave + u * NW) * 512 + lane * 8]);
    };
    auto issue = [&](int t, int st) {
        if (t < nfull) {
            issue_full(t * BK, st);
        } else if (t < nfast) {
            load_fast(t * BK);
            store_fast(st);
        } else {
            issue_edge(t * BK, st);
        }
    };
    // DMA instructions of this wave still allowed in flight once stage u has
    // landed: those of the DMA stages u + 1 .. min(last requested, nfull - 1).
    auto inflight_after = [&](int u, int last) {
        const int hi = min(last, nfull - 1);
        return hi > u ? (hi - u) * n_dma : 0;
    };
    Frag f0, f1;
#pragma unroll
    for (int u = 0; u < D; ++u)
        if (u < nstage) issue(u, u);
    lds_barrier(inflight_after(0, D - 1));
    if (nstage > 0) read_frags(As, Bs, 0, f0);
    int st = 0, st_req = D;   // buffer of stage t; buffer for stage t + D
    for (int t = 0; t < nstage; ++t) {
        const int st1 = st + 1 == S ? 0 : st + 1;
        read_frags(&As[st * SA], &Bs[st * SB], 1, f1);
        // Unaligned rows, interior stages: the dword-window loader, split
        // around the MFMAs.  Every other stage (DMA, edges) is issued whole
        // here: the element loader's registers would not fit beside the
        // accumulators across the MFMAs.
        const int st_fast = st_req;
        const bool fast = t + D < nfast;
        if (kLdsPoison && t + D < nstage && t + D >= nfull) poison_stage(st_req);
        if (fast) load_fast((t + D) * BK);
        else if (t + D < nstage) issue(t + D, st_req);
        st_req = st_req + 1 == S ? 0 : st_req + 1;
        __builtin_amdgcn_sched_barrier(0);
        mma(f0);
        if (fast) store_fast(st_fast);
        if (t + 1 < nstage) {
            lds_barrier(inflight_after(t + 1, t + D));
            read_frags(&As[st1 * SA], &Bs[st1 * SB], 0, f0);
        }
        __builtin_amdgcn_sched_barrier(0);
        mma(f1);
        st = st1;
    }
    store_tile<false, FM, FN>(p, acc, acc, m0 + wm, n0 + wn, li, lh);
}

template <class Cfg, Lowp T, bool DMA>
hipError_t launch_lowp_cfg(const LowpArgs& a, hipStream_t stream) {
    const int tiles_m = (a.M + Cfg::BM - 1) / Cfg::BM;
    const int tiles_n = (a.N + Cfg::BN - 1) / Cfg::BN;
    const dim3 grid((unsigned)(tiles_m * tiles_n)), block(Cfg::NT);
    hipLaunchKernelGGL((gemm_lowp_kernel<Cfg, T, DMA>), grid, block, 0, stream, a, tiles_m, tiles_n);
    return hipGetLastError();
}

// A's and B's rows 16-byte aligned: whole stages by DMA.
bool lowp_dma_ok(const LowpArgs& a) {
    return (a.lda % 8 == 0) && (a.ldb % 8 == 0) && ((reinterpret_cast<uintptr_t>(a.A) & 15) == 0) &&
           ((reinterpret_cast<uintptr_t>(a.B) & 15) == 0);
}

// ---------------------------------------------------------------------------
// Large wave tiles for 16-bit inputs.  The same plan as the fp32 large
// wave-tile kernel, with the operand layouts above: a 256 x 256 tile of 4
// waves, one per SIMD, each holding 128 x 128 of C as 4 x 4 accumulator
// blocks of v_mfma_f32_32x32x16_{bf16,f16} in AGPRs (256 registers).
//  * A stage is 32 k (two MFMA steps of 16); four LDS buffers, each
//    [A (256 x 32) | B (32 x 256)], swizzled as above.  Stage t's DMA of
//    stage t + 3 goes, one instruction every other MFMA of its first step,
//    into the buffer stage t - 1 used; the loop runs four stages per
//    iteration, so every buffer index is a compile-time constant.  In the
//    last iteration the DMAs past the last stage reload the last stage into
//    buffers nobody reads again, which keeps the loop free of branches.
//  * Each step's operands (4 A reads of 16 bytes, 8 transposing B reads of
//    8 bytes) are read one per MFMA during the previous step, into the
//    other half of a double-buffered register set.  One barrier per stage,
//    PRE MFMAs into its second step, after which the next stage's first
//    operands are read.
//  * Every address in the loop is a fixed per-lane register plus an
//    immediate: the DMA uses a scalar base per stage and a 32-bit lane
//    offset, and each (buffer, operand) pair has its own LDS base register,
//    so the loop holds no vector ALU instruction.
//  * The MFMA is inline assembly on AGPR accumulators; the kernel keeps the
//    wait states after zeroing and before the store itself.
//  * K % 128 != 0: the stages start at k = -shift so that whole groups of
//    four end at K; the buffers start zeroed and the copies below k = 0
//    leave lanes off (lane masks in SGPRs, see the kernel).
// Whole 16-byte chunks: A and B rows 16-byte aligned, N % 8 == 0, K % 8 ==
// 0.  Ragged M and N: DMA rows past M read row M - 1 and chunks past N the
// tile's first chunk; the store is guarded.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

template <int BM_ = 256, int PRE_ = 2, int GROUP_M_ = 8>
struct LowpBigCfg {
    static constexpr int BM = BM_, BN = BM_, NW = 4, NT = 256;
    static constexpr int WM = BM / 2, WN = BN / 2, WAVES_N = 2;
    static constexpr int FBM = WM / 32, FBN = WN / 32;      // 32 x 32 blocks per wave
    static constexpr int KST = 32;                          // k per stage: two 16-k steps
    static constexpr int NBUF = 4, PRE = PRE_, GROUP_M = GROUP_M_;
    static constexpr int SA = BM * KST, SB = KST * BN;      // 16-bit elements per stage
    static constexpr int SBUF = 2 * (SA + SB);              // bytes per stage buffer
    static constexpr int AQ = BM * KST / 512 / NW;          // 512 elements per DMA instruction
    static constexpr int BQ = KST * BN / 512 / NW;
    static constexpr int NDMA = AQ + BQ;                    // DMA per wave per stage
    static constexpr int CB = BN / 8;                       // 16-byte chunks per B row
    static constexpr int NMF = FBM * FBN;                   // MFMAs per step
    static constexpr int NRD = FBM + 2 * FBN;               // LDS reads per step
    // Step 0 spreads its NDMA DMAs over its MFMAs from the first and its NRD
    // reads from MFMA RB; step 1 takes the barrier before MFMA PRE and
    // spreads the next stage's reads from the MFMA after.  Operations that
    // share a slot go out together before that MFMA.
    static constexpr int RB = NMF >= 16 ? 4 : 1;
    static constexpr int slot(int j, int n_ops, int first) { return first + j * (NMF - first) / n_ops; }
    static_assert(BM == 256 || BM == 128, "tile");
    static_assert(RB < NMF && PRE + 1 < NMF, "every step has slots for its reads");
    static_assert(BN % 128 == 0, "B swizzle flips chunk bits 2-3 inside 16-chunk groups");
    static_assert(NBUF * SBUF <= 160 * 1024, "LDS");
    // waves per SIMD the kernel can run at (its LDS decides)
    static constexpr int MAXW = NBUF * SBUF > 80 * 1024 ? 1 : 2;
    static_assert((NBUF - 2) * NDMA <= 16, "vmcnt range of wait_vmcnt");
    static_assert(AQ * NW * 512 == SA && BQ * NW * 512 == SB, "whole DMA instructions");
};

template <Lowp T>
__device__ __forceinline__ void mfma16_asm(floatx16& acc, u32x4 a, u32x4 b) {
    if constexpr (T == Lowp::bf16)
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
    else
        asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// LANES: the k shift passes 96, so the DMA of stage 3, issued inside the
// main loop, reaches below k = 0 (a kernel of its own, so the common case
// keeps a loop without lane masks).
template <class Cfg, Lowp T, bool LANES>
__global__ __launch_bounds__(256, 1) __attribute__((amdgpu_waves_per_eu(1, Cfg::MAXW)))
void gemm_lowp_big_kernel(LowpArgs p, int tiles_m, int tiles_n, int shift) {
    constexpr int BM = Cfg::BM, BN = Cfg::BN, KST = Cfg::KST, NBUF = Cfg::NBUF;
    constexpr int FBM = Cfg::FBM, FBN = Cfg::FBN, SA = Cfg::SA, SBUF = Cfg::SBUF;
    constexpr int AQ = Cfg::AQ, BQ = Cfg::BQ, NDMA = Cfg::NDMA;
    constexpr int PRE = Cfg::PRE, RB = Cfg::RB, NRD = Cfg::NRD, CB = Cfg::CB;
    __shared__ __attribute__((aligned(16))) unsigned short lds[NBUF * (SA + Cfg::SB)];

    int tm, tn;
    tile_coords(blockIdx.x, tiles_m, tiles_n, Cfg::GROUP_M, p.xcds, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int M = p.M, N = p.N;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = (wave / Cfg::WAVES_N) * Cfg::WM, wn = (wave % Cfg::WAVES_N) * Cfg::WN;
    const int li = lane & 31, lh = lane >> 5;
    const unsigned lds0 = __builtin_amdgcn_readfirstlane(lds_addr(lds));

    // DMA: instruction v of a stage writes bytes 1024 v + 16 lane of the
    // operand's part of the buffer.  A: row 16 v + lane / 4, physical chunk
    // lane % 4 holding logical chunk (lane % 4) ^ swz_a(row).  B (CB chunks
    // a row): k row (64 / CB) v + lane / CB, physical chunk lane % CB holding
    // logical chunk (lane % CB) ^ 4 bswz(k).  Offsets in bytes from the
    // stage's base.
    // kk: the k offset of the lane's chunk within its stage.
    unsigned aoff[AQ], boff[BQ];
    int akk[AQ], bkk[BQ];
#pragma unroll
    for (int u = 0; u < AQ; ++u) {
        const int v = wave + Cfg::NW * u, row = 16 * v + (lane >> 2);
        const int c = (lane & 3) ^ swz_a(row);
        aoff[u] = 2u * ((unsigned)(min(m0 + row, M - 1) - m0) * (unsigned)p.lda + 8u * (unsigned)c);
        akk[u] = 8 * c;
    }
#pragma unroll
    for (int u = 0; u < BQ; ++u) {
        const int v = wave + Cfg::NW * u, k = (64 / CB) * v + lane / CB;
        const int c = (lane % CB) ^ (4 * bswz(k));
        const int col = n0 + 8 * c;
        boff[u] = 2u * ((unsigned)k * (unsigned)p.ldb + (unsigned)(col < N ? col - n0 : 0));
        bkk[u] = k;
    }
    const unsigned short* const a_tile = p.A + (long long)m0 * p.lda;
    const unsigned short* const b_tile = p.B + n0;
    auto issue_dma = [&](int d, int k0, int buf) {
        if (d < AQ) {
            const int v = wave + Cfg::NW * d;
            lds_dma16s(a_tile + k0, aoff[d], lds0 + (unsigned)(buf * SBUF + 1024 * v));
        } else {
            const int v = wave + Cfg::NW * (d - AQ);
            lds_dma16s(b_tile + (long long)k0 * p.ldb, boff[d - AQ],
                       lds0 + (unsigned)(buf * SBUF + 2 * SA + 1024 * v));
        }
    };
    // A stage that reaches below k = 0 (only the first four when K is not a
    // multiple of four stages): the lanes of k >= 0 copy, from the same
    // scalar base a_tile + k0 (an address below the matrix that no lane
    // with k >= 0 reaches under), the others stay off.
    auto lanes_on = [&](int d, int k0) {
        return (unsigned long long)__ballot(k0 + (d < AQ ? akk[d] : bkk[d - AQ]) >= 0);
    };
    // Zeros for the lanes a masked copy leaves off, at their own destinations
    // (lane l of instruction d owns bytes 16 l of its 1024-byte block).
    auto zero_off = [&](int d, int buf, unsigned long long lanes) {
        if ((lanes >> lane) & 1ull) return;
        const unsigned blk = d < AQ ? lds0 + (unsigned)(buf * SBUF + 1024 * (wave + Cfg::NW * d))
                                    : lds0 + (unsigned)(buf * SBUF + 2 * SA + 1024 * (wave + Cfg::NW * (d - AQ)));
        *reinterpret_cast<__attribute__((address_space(3))) u32x4*>((size_t)(blk + 16u * (unsigned)lane)) =
            u32x4{0u, 0u, 0u, 0u};
    };
    auto issue_dma_lanes = [&](int d, int k0, int buf, unsigned long long lanes) {
        if (d < AQ) {
            const int v = wave + Cfg::NW * d;
            lds_dma16s_lanes(a_tile + k0, aoff[d], lds0 + (unsigned)(buf * SBUF + 1024 * v), lanes);
        } else {
            const int v = wave + Cfg::NW * (d - AQ);
            lds_dma16s_lanes(b_tile + (long long)k0 * p.ldb, boff[d - AQ],
                             lds0 + (unsigned)(buf * SBUF + 2 * SA + 1024 * v), lanes);
        }
    };
    auto barrier = [&](int inflight) {
        asm volatile("" ::: "memory");
        wait_vmcnt(inflight);
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };

    floatx16 acc[FBM][FBN];
#pragma unroll
    for (int i = 0; i < FBM; ++i)
#pragma unroll
        for (int j = 0; j < FBN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
#pragma unroll
    for (int i = 0; i < FBM; ++i)
#pragma unroll
        for (int j = 0; j < FBN; ++j) asm volatile("" : "+a"(acc[i][j]));
    asm volatile("s_nop 7");

    // LDS operand bases, one register per (buffer, operand), byte addresses.
    //  * A, step t: row wm + 32 i + li, logical chunk 2 lh + t (k = 16 lh +
    //    8 t + e); 32 rows down (block i) the swizzle repeats, so block i is
    //    the immediate 2048 i.
    //  * B, block jb: this lane is lane 4e + j of group g = lane / 16 of a
    //    transposing read; it addresses k row 16 (g / 2) + e (+ 8 t + 4 r as
    //    immediates: the swizzle depends on k % 4 = e only) at columns
    //    wn + 32 jb + 16 (g % 2) + 4 j .. + 3.
    unsigned a_base[NBUF][2], b_base[NBUF][FBN];
    {
        const int g = lane >> 4, e = (lane >> 2) & 3, j = lane & 3;
        const int krow = 16 * (g >> 1) + e;
#pragma unroll
        for (int b = 0; b < NBUF; ++b) {
            const unsigned buf = lds0 + (unsigned)(b * SBUF);
#pragma unroll
            for (int t = 0; t < 2; ++t)
                a_base[b][t] = buf + (unsigned)((wm + li) * 64 + 16 * ((2 * lh + t) ^ swz_a(li)));
#pragma unroll
            for (int jb = 0; jb < FBN; ++jb) {
                const int col = wn + 32 * jb + 16 * (g & 1) + 4 * j;
                const int el = krow * BN + ((((col >> 3) ^ (4 * bswz(krow))) << 3) | (col & 7));
                b_base[b][jb] = buf + (unsigned)(2 * SA + 2 * el);
            }
        }
    }
    // Operands: Av[x][i], Bv[x][jb] for step parity x.
    u32x4 Av[2][FBM], Bv[2][FBN];
    shortx4 Bh[2][FBN][2];
    auto read_op = [&](auto B_c, auto T_c, auto X_c, int r) {
        // read r (0 .. NRD - 1) of the step with parity X and k step T of
        // buffer B: order A0, B0 lo, B0 hi, .. B3 hi, A1, A2, A3
        constexpr int b = decltype(B_c)::value, t = decltype(T_c)::value, x = decltype(X_c)::value;
        auto rd_a = [&](int i) {
            Av[x][i] = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
                (size_t)(a_base[b][t] + 2048u * (unsigned)i));
        };
        auto rd_b = [&](int jb, int h) {
            Bh[x][jb][h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_shortx4*)(size_t)(b_base[b][jb] + (unsigned)((8 * t + 4 * h) * BN * 2)));
        };
        if (r == 0) rd_a(0);
        else if (r <= 2 * FBN) rd_b((r - 1) >> 1, (r - 1) & 1);
        else rd_a(r - 2 * FBN);
    };
    auto b_op = [&](int x, int jb) {
        const uint2 l2 = __builtin_bit_cast(uint2, Bh[x][jb][0]);
        const uint2 h2 = __builtin_bit_cast(uint2, Bh[x][jb][1]);
        return u32x4{l2.x, l2.y, h2.x, h2.y};
    };
    auto step_mma = [&](int x, auto&& op) {
        static_for<FBN>([&](auto JB) { Bv[x][JB] = b_op(x, JB); });
        static_for<FBM>([&](auto I) {
            static_for<FBN>([&](auto J) {
                constexpr int i = decltype(I)::value, j = decltype(J)::value;
                op(FBN * i + j);
                mfma16_asm<T>(acc[i][j], Av[x][i], Bv[x][j]);
                __builtin_amdgcn_sched_barrier(0);
            });
        });
    };

    // Stage t covers k = t KST - shift ..; nst is a multiple of NBUF.
    const int nst = (p.K + shift) / KST;
    const int k_last = (nst - 1) * KST - shift;
    // Stage tt in buffer H: step 0 issues stage tt + 3's DMA (clamped to
    // the last stage) into buffer H - 1 and reads step 1's operands; step 1
    // passes the barrier (stage tt + 1 landed; tt + 2 and tt + 3 may be in
    // flight) and reads stage tt + 1's step-0 operands from buffer H + 1.
    // With LANES, the DMA copies only the lanes in `lanes` (stage 3 when
    // shift > 96 reaches below k = 0).
    auto stage = [&](auto H_c, int tt, auto lanes_c, const unsigned long long* lanes) {
        constexpr int h = decltype(H_c)::value;
        constexpr bool with_lanes = decltype(lanes_c)::value;
        using HN = std::integral_constant<int, (h + 1) % NBUF>;
        using HC = std::integral_constant<int, h>;
        using T0 = std::integral_constant<int, 0>;
        using T1 = std::integral_constant<int, 1>;
        const int kd = min((tt + NBUF - 1) * KST - shift, k_last);
        step_mma(0, [&](int n) {
#pragma unroll
            for (int d = 0; d < NDMA; ++d) {
                if (Cfg::slot(d, NDMA, 0) != n) continue;
                if constexpr (with_lanes) issue_dma_lanes(d, kd, (h + NBUF - 1) % NBUF, lanes[d]);
                else issue_dma(d, kd, (h + NBUF - 1) % NBUF);
            }
#pragma unroll
            for (int r = 0; r < NRD; ++r)
                if (Cfg::slot(r, NRD, RB) == n) read_op(HC{}, T1{}, T1{}, r);
        });
        step_mma(1, [&](int n) {
            if (n == PRE) barrier((NBUF - 2) * NDMA);
#pragma unroll
            for (int r = 0; r < NRD; ++r)
                if (Cfg::slot(r, NRD, PRE + 1) == n) read_op(HN{}, T0{}, T0{}, r);
        });
    };
    // The main loop.  With lanes, stage 0 copies with lanes3: the lanes of
    // stage 3 that reach k >= 0 in the first pass, every lane after it (an
    // SALU move; no vector instruction joins the MFMA stream).
    auto main_loop = [&](auto lanes_c) {
        constexpr bool with_lanes = decltype(lanes_c)::value;
        using F = std::false_type;
        unsigned long long lanes3[NDMA];
#pragma unroll
        for (int d = 0; d < NDMA; ++d) lanes3[d] = with_lanes ? lanes_on(d, (NBUF - 1) * KST - shift) : ~0ull;
        for (int t = 0; t < nst; t += NBUF) {
            stage(std::integral_constant<int, 0>{}, t, lanes_c, lanes3);
            stage(std::integral_constant<int, 1>{}, t + 1, F{}, lanes3);
            stage(std::integral_constant<int, 2>{}, t + 2, F{}, lanes3);
            stage(std::integral_constant<int, 3>{}, t + 3, F{}, lanes3);
            if constexpr (with_lanes) {
#pragma unroll
                for (int d = 0; d < NDMA; ++d) lanes3[d] = ~0ull;
            }
        }
    };

    if (nst > 0) {
        if (shift > 0) {
            // The first stages reach below k = 0: their lanes of negative k
            // write zeros to their own destinations, the others copy (each
            // 16-byte chunk of a stage belongs to one lane, so the zeros
            // need no barrier before the copies).  With LANES the main
            // loop's first copy into buffer NBUF - 1 leaves lanes off too:
            // that buffer is zeroed whole here, before the barrier that
            // precedes the copy.  As without a shift, stage 0 is waited for
            // and the others stay in flight: a copy whose lanes are all off
            // only precedes stages with none on below it.
#pragma unroll
            for (int s = 0; s < NBUF - 1; ++s)
#pragma unroll
                for (int d = 0; d < NDMA; ++d) {
                    const unsigned long long on = lanes_on(d, s * KST - shift);
                    zero_off(d, s, on);
                    issue_dma_lanes(d, s * KST - shift, s, on);
                }
            if constexpr (LANES) {
                unsigned short* const last = lds + (NBUF - 1) * (SA + Cfg::SB);
                for (int e = 8 * (int)threadIdx.x; e < SA + Cfg::SB; e += 8 * Cfg::NT)
                    *reinterpret_cast<uint4*>(last + e) = make_uint4(0u, 0u, 0u, 0u);
            }
            barrier((NBUF - 2) * NDMA);
        } else {
#pragma unroll
            for (int s = 0; s < NBUF - 1; ++s)
#pragma unroll
                for (int d = 0; d < NDMA; ++d) issue_dma(d, min(s * KST, k_last), s);
            barrier((NBUF - 2) * NDMA);
        }
        using B0 = std::integral_constant<int, 0>;
        static_for<NRD>([&](auto R) { read_op(B0{}, B0{}, B0{}, R); });
        main_loop(std::integral_constant<bool, LANES>{});
        wait_vmcnt(0);   // the reloads past the last stage land before exit
    }
    // Last MFMAs -> accumulator reads: 24 wait states (an 8-pass MFMA's
    // result needs 11); each accumulator is read only after the pause.
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");
#pragma unroll
    for (int i = 0; i < FBM; ++i)
#pragma unroll
        for (int j = 0; j < FBN; ++j) asm volatile("" : "+a"(acc[i][j]));
    store_tile<false, FBM, FBN>(p, acc, acc, m0 + wm, n0 + wn, li, lh);
}

// Whole 16-byte chunks (K % 8 == 0: the k shift moves whole chunks), at
// most a quarter of the k zeroed by the shift to four stages, 32-bit DMA
// offsets.
int lowp_big_shift(const LowpArgs& a) { return (128 - a.K % 128) % 128; }
bool lowp_big_fits(const LowpArgs& a) {
    return (a.lda % 8 == 0) && (a.ldb % 8 == 0) && a.N % 8 == 0 && a.K % 8 == 0 && a.K > 0 &&
           3 * lowp_big_shift(a) <= a.K &&
           ((reinterpret_cast<uintptr_t>(a.A) & 15) == 0) &&
           ((reinterpret_cast<uintptr_t>(a.B) & 15) == 0) &&
           a.lda < (1 << 22) && a.ldb < (1 << 22);
}

template <class Cfg, Lowp T>
hipError_t launch_lowp_big_cfg(const LowpArgs& a, hipStream_t stream) {
    if (!lowp_big_fits(a)) return hipErrorInvalidValue;
    const int tiles_m = (a.M + Cfg::BM - 1) / Cfg::BM, tiles_n = (a.N + Cfg::BN - 1) / Cfg::BN;
    const int shift = lowp_big_shift(a);
    if (shift > (Cfg::NBUF - 1) * Cfg::KST)
        hipLaunchKernelGGL((gemm_lowp_big_kernel<Cfg, T, true>), dim3((unsigned)(tiles_m * tiles_n)),
                           dim3(Cfg::NT), 0, stream, a, tiles_m, tiles_n, shift);
    else
        hipLaunchKernelGGL((gemm_lowp_big_kernel<Cfg, T, false>), dim3((unsigned)(tiles_m * tiles_n)),
                           dim3(Cfg::NT), 0, stream, a, tiles_m, tiles_n, shift);
    return hipGetLastError();
}

// Tile table of the kernel above, for the shapes the large wave tiles do
// not take (rows not 16-byte aligned, N % 8 != 0, K % 8 != 0, a k shift
// above a third of K), from
// interleaved timing of bf16 products on MI355X:
//  * 256x256 tiles of 8 waves of 64x128, four LDS stages, from 128 tiles
//    (half the CUs busy): 1148-1167 TFLOP/s at 8192^3 (128x64 waves 1078,
//    4 waves of 128x128 with accumulators in AGPRs 1077, 128x256 tiles
//    887-1108; three stages 2 % slower), 821 at 4096x4096x1024, 698 at
//    3072^3 (144 tiles; 64x128 tiles 638);
//  * else 64x128 tiles of 4 waves of 32x64, three stages, the most
//    workgroups: 570 at 2048^3 (128x128 of 8 waves 547), 162 at 1024^3
//    (129).
// Unaligned rows (the dword-window loader, whose registers the 256x256
// tiles cannot hold beside their accumulators): 128x128 tiles of 4 waves
// of 64x64 beyond two per CU (8192x8192x8191 525 against 441 for 64x128,
// 4096x4096x4095 579 against 456), else 64x128 (2048x2048x2047 329
// against 276).
using LowpLarge = LowpCfg<256, 256, 64, 128, 1, 4>;
using LowpMid = LowpCfg<64, 128, 32, 64, 2, 3>;
using LowpUnaligned = LowpCfg<128, 128, 64, 64, 2, 3>;

// Large wave tiles where they fit: 128 x 128 tiles (4 waves of 64 x 64) up
// to two per CU -- 2048^3 774 TFLOP/s against 563 for the 64 x 128 tiles
// below, 1024^3 229 against 150, 2560^3 729 against 630 for 256 x 256 --
// and 256 x 256 tiles beyond (4096^3 1262 against 984, 8192^3 1343 against
// 847).  256 x 256 tiles use raster groups of 4 tile rows (+1.9 % at
// 8192^3 and +4 % at 8192 x 8192 x 2048 over groups of 8).
using LowpBig = LowpBigCfg<256, 2, 4>;
using LowpBigMid = LowpBigCfg<128, 1, 8>;

template <Lowp T>
hipError_t launch_lowp_t(const LowpArgs& a, hipStream_t stream) {
    const long long tiles = ((long long)a.M + 255) / 256 * (((long long)a.N + 255) / 256);
    const long long tiles128 = ((long long)a.M + 127) / 128 * (((long long)a.N + 127) / 128);
    if (lowp_big_fits(a)) {
        if (tiles128 <= 2LL * a.cus) return launch_lowp_big_cfg<LowpBigMid, T>(a, stream);
        return launch_lowp_big_cfg<LowpBig, T>(a, stream);
    }
    if (!lowp_dma_ok(a)) {
        if (tiles128 > 2LL * a.cus) return launch_lowp_cfg<LowpUnaligned, T, false>(a, stream);
        return launch_lowp_cfg<LowpMid, T, false>(a, stream);
    }
    if (tiles >= a.cus / 2) return launch_lowp_cfg<LowpLarge, T, true>(a, stream);
    return launch_lowp_cfg<LowpMid, T, true>(a, stream);
}

}  // namespace

hipError_t launch_lowp(const LowpArgs& a, Lowp type, hipStream_t stream) {
    return type == Lowp::bf16 ? launch_lowp_t<Lowp::bf16>(a, stream)
                              : launch_lowp_t<Lowp::f16>(a, stream);
}

}  // namespace sgemm
