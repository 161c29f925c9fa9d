// Direct global -> LDS loads (buffer_load ... lds) through inline asm, shared
// by the matrix-product and attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Direct global -> LDS loads (buffer_load ... lds), issued through inline asm.
// Issued as builtins, the compiler counts them and then makes every transpose
// read (ds_read_b64_tr_b16) wait for all of them, since it cannot tell which
// LDS bytes that read touches; that would drain the prefetch each k-step.
// Hidden from it, they are covered by the pipelines' explicit vmcnt waits; the
// compiler's own waits for other loads stay safe, as they count a subset of
// the operations in flight (a wait for "at most n outstanding" then leaves
// fewer, never more, incomplete). The instructions write no registers.
//
// Raw buffer resource (gfx9 layout): base, stride 0, num_records, dword 3,
// made wave-uniform (it lives in scalar registers).
__device__ __forceinline__ u32x4 raw_rsrc(const void* base) {
    const uint64_t a = (uint64_t)base;
    return u32x4{(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a),
                 (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xffffu),
                 0x7fffffffu, 0x00020000u};
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)__builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p);
}

// 16 bytes per lane from rsrc + soff + voff to LDS at lds + lane * 16 (lds is
// wave-uniform). M0, bound as an input, carries the LDS address; the leading
// s_nop gives the one wait state the hardware needs between writing M0 and
// the load that reads it. No memory clobber: the loads stay ordered against
// the pipelines' waits and barriers (volatile asm and barrier intrinsics,
// which do fence memory), while the compiler may schedule LDS reads of other
// ring slots around them.
__device__ __forceinline__ void lds_dma16(u32x4 rs, uint32_t voff, uint32_t soff, const void* lds) {
#if __HIP_DEVICE_COMPILE__
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
                 :
                 : "v"(voff), "s"(rs), "s"(soff), "{m0}"(lds_addr(lds)));
#endif
}

// 4 bytes per lane, to lds + lane * 4.
__device__ __forceinline__ void lds_dma4(u32x4 rs, uint32_t voff, uint32_t soff, const void* lds) {
#if __HIP_DEVICE_COMPILE__
    asm volatile("s_nop 0\n\tbuffer_load_dword %0, %1, %2 offen lds"
                 :
                 : "v"(voff), "s"(rs), "s"(soff), "{m0}"(lds_addr(lds)));
#endif
}
