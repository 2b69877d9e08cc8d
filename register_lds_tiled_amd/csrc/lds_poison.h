// lds_poison.h -- the stale-stage poisoning of the debug build.
//
// Built with -DSGEMM_LDS_POISON (the library variant
// libsgemm_mi355x_ldspoison.so), every kernel that reuses an LDS stage writes
// a quiet NaN over each location it is about to refill, at the earliest point
// where the schedule has retired that location (after the barrier, or the
// wave-level fence, that ends its last read), and refills it only once those
// writes have completed.  A read of a stage outside its lifetime -- a missing
// or misplaced barrier, a vmcnt wait that lets a read run ahead of its DMA --
// then yields NaN in C instead of the previous stage's plausible numbers, and
// a race whose window was a few cycles wide spans the whole refill latency.
// With a correct schedule no read ever sees a poisoned word, so the debug
// build's C is bit-identical to the release build's.  The pages name the
// synchronisation and load ordering of these kernels as what makes them hard
// to debug ("Register/Shared Memory Tiling", pros and cons, first drawback).
//
// The writes are inline asm with a "memory" clobber and end with a wait for
// their completion: the compiler can neither drop them as dead stores (the
// refill overwrites them) nor move them across the barriers, and a DMA
// issued after them cannot land first.  In the release build every helper is
// empty and kLdsPoison is false.
#pragma once

#include <hip/hip_runtime.h>

namespace sgemm {

#ifdef SGEMM_LDS_POISON
constexpr bool kLdsPoison = true;

// Pointer forms, for kernels that stage through registers: one word, or four
// consecutive words, at an LDS address.
__device__ __forceinline__ void lds_poison_f1(const void* p) {
    const unsigned a = (unsigned)(size_t)(__attribute__((address_space(3))) const void*)p;
    asm volatile("ds_write_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)"
                 :: "v"(a), "v"(0x7FC00000u) : "memory");
}
__device__ __forceinline__ void lds_poison_f4(const void* p) {
    const unsigned a = (unsigned)(size_t)(__attribute__((address_space(3))) const void*)p;
    asm volatile("ds_write_b32 %0, %1\n\tds_write_b32 %0, %1 offset:4\n\t"
                 "ds_write_b32 %0, %1 offset:8\n\tds_write_b32 %0, %1 offset:12\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 :: "v"(a), "v"(0x7FC00000u) : "memory");
}

// DMA forms: the destinations of a wave-wide DMA to the wave-uniform LDS
// byte address `base` -- lane i's 16 bytes at base + 16 i (W4) or its word
// at base + 4 i (W1).  The lane's address and the NaN are formed inside the
// asm, after a pause of 16 wait states, so that no vector write lands in
// the middle of the matrix instructions the DMA is interleaved with while
// one of them may still be reading its operands.
#define SGEMM_POISON_ADDR(SHIFT)                                              \
    "s_nop 7\n\ts_nop 7\n\t"                                                  \
    "v_mbcnt_lo_u32_b32 %[a], -1, 0\n\tv_mbcnt_hi_u32_b32 %[a], -1, %[a]\n\t" \
    "v_lshlrev_b32 %[a], " #SHIFT ", %[a]\n\tv_add_u32 %[a], %[base], %[a]\n\t" \
    "v_mov_b32 %[v], 0x7fc00000\n\t"
#define SGEMM_POISON_W4                                                       \
    "ds_write_b32 %[a], %[v]\n\tds_write_b32 %[a], %[v] offset:4\n\t"         \
    "ds_write_b32 %[a], %[v] offset:8\n\tds_write_b32 %[a], %[v] offset:12\n\t"

__device__ __forceinline__ void lds_poison_dma16(unsigned base) {
    unsigned a, v;
    asm volatile(SGEMM_POISON_ADDR(4) SGEMM_POISON_W4 "s_waitcnt lgkmcnt(0)"
                 : [a] "=&v"(a), [v] "=&v"(v) : [base] "s"(base) : "memory");
}
__device__ __forceinline__ void lds_poison_dma4(unsigned base) {
    unsigned a, v;
    asm volatile(SGEMM_POISON_ADDR(2) "ds_write_b32 %[a], %[v]\n\ts_waitcnt lgkmcnt(0)"
                 : [a] "=&v"(a), [v] "=&v"(v) : [base] "s"(base) : "memory");
}
// lds_poison_dma16 for the lanes set in `lanes` (wave-uniform): the lanes a
// masked DMA leaves off keep what they hold.
__device__ __forceinline__ void lds_poison_dma16_lanes(unsigned base, unsigned long long lanes) {
    unsigned a, v;
    unsigned long long saved;
    asm volatile(SGEMM_POISON_ADDR(4)
                 "s_mov_b64 %[saved], exec\n\ts_mov_b64 exec, %[lanes]\n\ts_nop 0\n\t"
                 SGEMM_POISON_W4 "s_waitcnt lgkmcnt(0)\n\ts_mov_b64 exec, %[saved]"
                 : [a] "=&v"(a), [v] "=&v"(v), [saved] "=&s"(saved)
                 : [base] "s"(base), [lanes] "s"(lanes) : "memory");
}
#undef SGEMM_POISON_ADDR
#undef SGEMM_POISON_W4
#else
constexpr bool kLdsPoison = false;
__device__ __forceinline__ void lds_poison_f1(const void*) {}
__device__ __forceinline__ void lds_poison_f4(const void*) {}
__device__ __forceinline__ void lds_poison_dma16(unsigned) {}
__device__ __forceinline__ void lds_poison_dma4(unsigned) {}
__device__ __forceinline__ void lds_poison_dma16_lanes(unsigned, unsigned long long) {}
#endif

}  // namespace sgemm
