// Direct global-to-LDS loads and the waits and barrier that order them,
// for kernels that stage operands through LDS (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// s_waitcnt with only the vector-memory counter limited (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// s_waitcnt: vector-memory counter <= N and all LDS reads returned
// (N = 63: LDS reads only).
template <int N>
__device__ __forceinline__ void wait_vmcnt_lgkm0() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
}

// 16 bytes per lane from global memory straight into LDS: lane i's bytes land
// at LDS address lds_base + 16 * i.  Issued as inline assembly so that the
// compiler does not treat every later LDS read as dependent on it; the caller
// orders it with wait_vmcnt and the workgroup barrier.  The LDS address is
// read from M0; it is an input operand bound to M0, so the compiler itself
// writes M0 before the statement (and knows what M0 then holds) instead of
// the statement overwriting a register the compiler may be using.  The load
// reads M0 one wait state after a scalar write of it at the earliest (the
// s_nop: the compiler's hazard checks do not look inside the statement).
__device__ __forceinline__ void lds_dma16(const void* gptr, uint32_t lds_base) {
    asm volatile(
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, off"
        :
        : "v"(gptr), "{m0}"(lds_base)
        : "memory");
}

// The same from a wave-uniform base address plus a 32-bit per-lane byte
// offset (the scalar-base form of the load).
__device__ __forceinline__ void lds_dma16_s(const void* sbase, uint32_t voff, uint32_t lds_base) {
    asm volatile(
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, %1"
        :
        : "v"(voff), "s"(sbase), "{m0}"(lds_base)
        : "memory");
}

// 4 bytes per lane from a wave-uniform base plus a 32-bit per-lane byte
// offset into LDS: lane i's dword lands at lds_base + 4 * i.
__device__ __forceinline__ void lds_dma4_s(const void* sbase, uint32_t voff, uint32_t lds_base) {
    asm volatile(
        "s_nop 0\n\t"
        "global_load_lds_dword %0, %1"
        :
        : "v"(voff), "s"(sbase), "{m0}"(lds_base)
        : "memory");
}

// Workgroup barrier without a memory fence (the LDS traffic it orders is
// waited for explicitly); the empty asm statements keep the compiler from
// moving memory accesses across it.
__device__ __forceinline__ void barrier_lds() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}

}  // namespace moe
