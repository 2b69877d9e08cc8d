// tiles.h -- internal declarations shared by the HIP kernel translation units
// and the C-ABI front end of libsgemm_mi355x.so.  Not installed, not part of
// the ABI (that is include/sgemm.h).
#pragma once

#include <hip/hip_runtime.h>

#include "lds_poison.h"

namespace sgemm {

// Arguments of one call after validation.  Row-major, leading dimensions in
// elements, offsets formed in 64 bits on the device.  The plain product is
// C = A.B; the fused form is C = act(alpha * A.B + beta * C + bias[col]),
// selected by `epi` (false: alpha, beta, bias and act are not looked at).
struct GemmArgs {
    int M, N, K;
    const float* __restrict__ A;
    long long lda;
    const float* __restrict__ B;
    long long ldb;
    float* __restrict__ C;
    long long ldc;
    float alpha = 1.f, beta = 0.f;
    const float* __restrict__ bias = nullptr;   // N floats, or none
    int act = 0;                                // 0 identity, 1 ReLU
    bool epi = false;
    // The device the launch runs on: compute units (the tile tables size
    // grids in rounds of one tile per CU) and XCDs (each with its own L2;
    // tile_coords gives each a contiguous run of tiles).  Set by the ABI
    // layer from the device's attributes.
    int cus = 256, xcds = 8;
};

// One output of the fused form, in fp32: s is the accumulated dot product,
// c_in the output's previous value (used only when beta != 0), bias_j the
// column's bias (added only when there is a bias).  ReLU sends negatives to
// zero and lets NaN through; it is written as a compare and select because a
// max() would turn NaN into 0.
__device__ __forceinline__ float fused_out(const GemmArgs& p, float s, float c_in, float bias_j) {
    float v = p.alpha * s;
    if (p.beta != 0.f) v = __builtin_fmaf(p.beta, c_in, v);
    if (p.bias != nullptr) v += bias_j;
    if (p.act == 1 && v < 0.f) v = 0.f;
    return v;
}

typedef float floatx16 __attribute__((ext_vector_type(16)));

// The previous values of a wave's FM x FN blocks of C, in the accumulator
// layout, for the fused form with beta != 0 (with beta == 0 C is not read:
// it may hold anything).  A kernel may load them before its main loop, so
// that the reads overlap the multiplication instead of following it; C
// never overlaps A or B, and each lane reads only the outputs it will
// write.  Outputs outside M x N are not read.
template <int FM, int FN>
__device__ __forceinline__ void load_c_tile(const GemmArgs& p, floatx16 (&cin)[FM][FN],
                                            int r0, int c0, int li, int lh) {
    if (p.beta == 0.f) return;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = r0 + i * 32 + 8 * (r / 4) + 4 * lh + (r % 4);
            if (row >= p.M) continue;
            const float* crow = p.C + (long long)row * p.ldc + c0 + li;
#pragma unroll
            for (int j = 0; j < FN; ++j)
                if (c0 + j * 32 + li < p.N) cin[i][j][r] = crow[j * 32];
        }
    }
}

// Store of a wave's FM x FN accumulator blocks, whose top-left output is
// (r0, c0).  Register r of lane l of a block holds row 8(r/4) + 4(l/32) + r%4
// and column l%32, so each register is one 128-byte row segment across the
// 32 lanes of a half-wave.  Outputs outside M x N are skipped (ragged
// tiles).  EPI: the fused form act(alpha*acc + beta*C + bias[col]), with the
// column's bias loaded once per block; PRE: C's previous values are already
// in cin (load_c_tile), else they are read here.
// Stores of C carry the nontemporal hint: each output is written once, and
// streamed out this way the stores drain while other workgroups still
// compute instead of at the end of the launch (1024^3: 113 -> 117 TFLOP/s,
// 2048^3: 135.5 -> 138.9, interleaved on one box).
typedef float c_f4 __attribute__((ext_vector_type(4)));
typedef float c_f2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void store_c(float* p, float v) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ void store_c4(float* p, float a, float b, float c, float d) {
    __builtin_nontemporal_store(c_f4{a, b, c, d}, reinterpret_cast<c_f4*>(p));
}
__device__ __forceinline__ void store_c2(float* p, float a, float b) {
    __builtin_nontemporal_store(c_f2{a, b}, reinterpret_cast<c_f2*>(p));
}

template <bool EPI, int FM, int FN, bool PRE = false, class Args>
__device__ __forceinline__ void store_tile(const Args& p, const floatx16 (&acc)[FM][FN],
                                           const floatx16 (&cin)[FM][FN],
                                           int r0, int c0, int li, int lh) {
    float bias_j[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        bias_j[j] = 0.f;
        if constexpr (EPI) {
            const int col = c0 + j * 32 + li;
            if (p.bias != nullptr && col < p.N) bias_j[j] = p.bias[col];
        }
    }
    // One row address per (block row, register), shared by the FN blocks.
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = r0 + i * 32 + 8 * (r / 4) + 4 * lh + (r % 4);
            if (row >= p.M) continue;
            float* crow = p.C + (long long)row * p.ldc + c0 + li;
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                if (c0 + j * 32 + li >= p.N) continue;
                float* c = crow + j * 32;
                if constexpr (EPI) {
                    const float c_in = PRE ? cin[i][j][r] : (p.beta != 0.f ? *c : 0.f);
                    store_c(c, fused_out(p, acc[i][j][r], c_in, bias_j[j]));
                } else {
                    store_c(c, acc[i][j][r]);
                }
            }
        }
    }
}

// Launchers, one per kernel family.  Each picks the template instance for the
// shape/alignment, enqueues one launch on `stream` and returns the launch
// status (hipGetLastError).
hipError_t launch_mfma(const GemmArgs& a, hipStream_t stream);
hipError_t launch_valu(const GemmArgs& a, hipStream_t stream);
hipError_t launch_valu_page(const GemmArgs& a, hipStream_t stream);
// A with at most 16 rows and no fused epilogue: the B-streaming kernel.
bool skinny_m_fits(const GemmArgs& a);
hipError_t launch_skinny_m(const GemmArgs& a, hipStream_t stream);
// B with at most 16 columns (and A with more than 16 rows): the A-streaming kernels.
bool skinny_n_fits(const GemmArgs& a);
hipError_t launch_skinny_n(const GemmArgs& a, hipStream_t stream);
hipError_t launch_micro4x4(int K, const float* A, const float* B, float* C,
                           hipStream_t stream);

// 16-bit-input product (bf16 or fp16 A and B, fp32 C); A and B are passed
// as raw 16-bit storage.
enum class Lowp { bf16, f16 };
struct LowpArgs {
    int M, N, K;
    const unsigned short* __restrict__ A;
    long long lda;
    const unsigned short* __restrict__ B;
    long long ldb;
    float* __restrict__ C;
    long long ldc;
    int cus = 256, xcds = 8;   // as in GemmArgs
};
hipError_t launch_lowp(const LowpArgs& a, Lowp type, hipStream_t stream);

// The VALU path's built tile configurations (a table of block, wave and
// lane tiles; launch_valu picks among them by shape): how many there are,
// a readable description of one, and a launch at one of them.
int valu_tile_count();
const char* valu_tile_name(int tile);
hipError_t launch_valu_tile(const GemmArgs& a, int tile, hipStream_t stream);

// Workgroups of one dispatch are handed to the XCDs of an MI355X (8 on a
// whole device) in round-robin order of their linear id, and each XCD has
// its own L2.  This maps the linear workgroup id to a C tile so that (1) the
// workgroups that land on one XCD own a contiguous run of the tile raster
// and (2) the raster walks `group_m` tile-rows at a time, so that
// concurrently running tiles on an XCD share A row-panels and B
// column-panels in that XCD's L2.  xcds <= 1: no remap.
__device__ __forceinline__ void tile_coords(int wg, int tiles_m, int tiles_n,
                                            int group_m, int xcds, int& tm, int& tn) {
    const int T = tiles_m * tiles_n;
    int id = wg;
    if (xcds > 1) {
        const int q = T / xcds, r = T - q * xcds;
        const int j = wg / xcds, x = wg - j * xcds;
        // bijection [0,T) -> [0,T): XCD x owns ids [start_x, start_x + count_x)
        id = (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + j;
    }
    const int per_group = group_m * tiles_n;
    const int g = id / per_group;
    const int first_m = g * group_m;
    const int gsize = min(tiles_m - first_m, group_m);
    const int local = id - g * per_group;
    tm = first_m + local % gsize;
    tn = local / gsize;
}

// Load one float4 of a row-major matrix X (rows x cols valid, leading
// dimension ld) at (r, c..c+3); elements outside the valid range read as 0
// (the zero fill of ragged tiles).  full: the whole float4 is known to be in
// range.  VEC: X and ld allow a 16-byte aligned load.
template <bool VEC>
__device__ __forceinline__ float4 load4(const float* __restrict__ X, long long ld,
                                        int r, int c, int rows, int cols, bool full) {
    if (full && VEC) {
        return *reinterpret_cast<const float4*>(X + (long long)r * ld + c);
    }
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (r < rows) {
        const float* p = X + (long long)r * ld;
        if (full) {
            v.x = p[c]; v.y = p[c + 1]; v.z = p[c + 2]; v.w = p[c + 3];
        } else {
            if (c + 0 < cols) v.x = p[c + 0];
            if (c + 1 < cols) v.y = p[c + 1];
            if (c + 2 < cols) v.z = p[c + 2];
            if (c + 3 < cols) v.w = p[c + 3];
        }
    }
    return v;
}

}  // namespace sgemm
