// lds_dma.h -- device helpers shared by the matrix-core kernels: the
// direct-to-LDS DMA (gfx950 global_load_lds), its completion wait, and
// compile-time unrolling.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>
#include <utility>

#include "lds_poison.h"

namespace sgemm {

// Byte address of an LDS object, as the DMA and ds_read instructions see it.
__device__ __forceinline__ unsigned lds_addr(const void* p) {
    return (unsigned)(size_t)(__attribute__((address_space(3))) const void*)p;
}

// Wave-wide DMA: lane i copies 16 bytes from global address g into LDS at
// byte lds_base + 16 i.  lds_base must be wave-uniform.  The asm sets M0
// itself, so the compiler's conservative wait before every LDS read does
// not apply: kernels order DMA and reads with wait_vmcnt and barriers.
// Nothing else in these kernels uses M0.  In the debug build each helper
// first poisons the destinations it is about to fill (lds_poison.h).
__device__ __forceinline__ void lds_dma16(const void* g, unsigned lds_base) {
    lds_poison_dma16(lds_base);
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                 :: "v"(g), "s"(lds_base) : "memory", "m0");
}
// The same from a scalar base and a 32-bit per-lane byte offset (lane i
// copies base + voff), 16 bytes (lds_dma16s) or 4 bytes (lds_dma4s, to
// lds_base + 4 i).  The address is formed without vector instructions.
__device__ __forceinline__ void lds_dma16s(const void* base, unsigned voff, unsigned lds_base) {
    lds_poison_dma16(lds_base);
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
                 :: "v"(voff), "s"(base), "s"(lds_base) : "memory", "m0");
}
// lds_dma16s for the lanes set in `lanes` only (a wave-uniform mask, held
// in SGPRs): the asm saves EXEC, copies with EXEC = lanes and restores it,
// so the compiler sees no divergent branch and puts no VALU work around it.
__device__ __forceinline__ void lds_dma16s_lanes(const void* base, unsigned voff, unsigned lds_base,
                                                 unsigned long long lanes) {
    lds_poison_dma16_lanes(lds_base, lanes);
    unsigned long long saved;
    asm volatile("s_mov_b64 %0, exec\n\ts_mov_b64 exec, %4\n\ts_nop 0\n\ts_mov_b32 m0, %3\n\t"
                 "global_load_lds_dwordx4 %1, %2\n\ts_mov_b64 exec, %0"
                 : "=&s"(saved) : "v"(voff), "s"(base), "s"(lds_base), "s"(lanes) : "memory", "m0");
}
__device__ __forceinline__ void lds_dma4s(const void* base, unsigned voff, unsigned lds_base) {
    lds_poison_dma4(lds_base);
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1"
                 :: "v"(voff), "s"(base), "s"(lds_base) : "memory", "m0");
}

// s_waitcnt with only the vector-memory count constrained: vmcnt(n), n <= 16
// (larger n waits for everything).
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
        case 9: __builtin_amdgcn_s_waitcnt(0x0F79); break;
        case 10: __builtin_amdgcn_s_waitcnt(0x0F7A); break;
        case 11: __builtin_amdgcn_s_waitcnt(0x0F7B); break;
        case 12: __builtin_amdgcn_s_waitcnt(0x0F7C); break;
        case 13: __builtin_amdgcn_s_waitcnt(0x0F7D); break;
        case 14: __builtin_amdgcn_s_waitcnt(0x0F7E); break;
        case 15: __builtin_amdgcn_s_waitcnt(0x0F7F); break;
        case 16: __builtin_amdgcn_s_waitcnt(0x4F70); break;   // vmcnt bits 5:4 at 15:14
        default: __builtin_amdgcn_s_waitcnt(0x0F70); break;
    }
}

// f(integral_constant<int, 0>) .. f(integral_constant<int, N - 1>), in order:
// the unrolling is part of the program, not left to the compiler's
// thresholds (a stage of 256 MFMAs exceeded them, and the partly rolled
// loops indexed the register arrays at run time).
template <class F, int... I>
__device__ __forceinline__ void static_for_seq(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_seq(f, std::make_integer_sequence<int, N>{});
}

}  // namespace sgemm
