// global -> LDS copy helpers shared by the MFMA kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe_w4 {

__device__ __forceinline__ uint32_t uniform32(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ uint64_t uniform64(uint64_t v) {
    return ((uint64_t)uniform32((uint32_t)(v >> 32)) << 32) | uniform32((uint32_t)v);
}

// LDS byte address (wave-uniform) of a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const uint8_t* shared_obj) {
    return uniform32((uint32_t)(uintptr_t)(__attribute__((address_space(3))) const uint8_t*)shared_obj);
}

// global -> LDS copies.  `lds` is the same for the whole wavefront; lane i
// writes at lds + 16 i (dwordx4) or lds + 4 i (dword).  Issued through inline
// assembly so that the compiler's wait insertion does not see them (it would
// otherwise wait for every in-flight copy at each barrier); the callers wait for
// them explicitly.  M0 is restored after use.
// 16 bytes per lane from sbase + voff (sbase wave-uniform) to LDS address lds + 16 lane
__device__ __forceinline__ void dma16_to_lds(uint64_t sbase, uint32_t voff, uint32_t lds) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(uniform64(sbase)), "s"(uniform32(lds))
        : "memory");
}
// 16 bytes per lane from a per-lane address to LDS address lds + 16 lane
__device__ __forceinline__ void dma16v_to_lds(const void* src, uint32_t lds) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(src), "s"(uniform32(lds))
        : "memory");
}
// 4 bytes per lane from a per-lane address to LDS address lds + 4 lane
__device__ __forceinline__ void dma4_to_lds(const void* src, uint32_t lds) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dword %1, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(src), "s"(uniform32(lds))
        : "memory");
}

// s_waitcnt vmcnt(N) (expcnt and lgkmcnt left unconstrained).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

}  // namespace moe_w4
