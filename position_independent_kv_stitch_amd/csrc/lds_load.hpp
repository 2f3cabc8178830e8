// lds_load.hpp -- direct global -> LDS loads whose completion the kernels
// count themselves.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace pic {

// One 16-byte piece per lane from global memory straight into LDS: lane l's
// piece lands at lds + 16 l (global_load_lds_dwordx4 with the LDS address in
// M0).  Written as inline assembly so that the compiler does not wait for
// these loads before every LDS access (it cannot tell which staging buffer a
// load writes): the caller counts them with s_waitcnt vmcnt (they complete
// in issue order with the wave's other vector memory loads) and publishes
// them to the other waves with a barrier.  lds must be the same for every
// lane of the wave.
// M0 is saved and restored around the load, so the compiler's own use of it
// (it treats M0 as reserved) is not disturbed.  OFF is a byte offset that
// the instruction adds to src (no address arithmetic per load); it adds the
// same offset to the LDS address, so M0 is set OFF bytes before lds (lds
// must be at least OFF bytes into the LDS).
template <int OFF = 0>
__device__ __forceinline__ void load_lds16(const void *src, const void *lds) {
    static_assert(OFF >= 0 && OFF < 4096, "the instruction's offset field");
    const uint32_t base = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(
        reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void *)lds))) - OFF;
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off offset:%3\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(src), "s"(base), "n"(OFF)
        : "memory");
}

// Eighteen such loads in one asm block: load k takes the 16 bytes at
// src + 64 k (the instruction's offset field) into lds + 1024 k + 16 l, so a
// 576-dim bf16 row's 18 k-steps of 32 dims land in 18 consecutive 1 KB
// slabs.  M0 of load k is lds + 960 k (1024 k less the offset), computed by
// the compiler into scalar registers, so the block itself only moves them
// into M0 (no scalar arithmetic, which would clobber SCC); M0 is saved and
// restored around the block.  lds must be the same for every lane.
#define PIC_LDS_ROW_LOAD(k, o) \
    "s_mov_b32 m0, %" #k "\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off offset:" #o "\n\t"
__device__ __forceinline__ void load_lds16_row18(const void *src, const void *lds) {
    const uint32_t b = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(
        reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void *)lds)));
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        PIC_LDS_ROW_LOAD(2, 0) PIC_LDS_ROW_LOAD(3, 64) PIC_LDS_ROW_LOAD(4, 128)
        PIC_LDS_ROW_LOAD(5, 192) PIC_LDS_ROW_LOAD(6, 256) PIC_LDS_ROW_LOAD(7, 320)
        PIC_LDS_ROW_LOAD(8, 384) PIC_LDS_ROW_LOAD(9, 448) PIC_LDS_ROW_LOAD(10, 512)
        PIC_LDS_ROW_LOAD(11, 576) PIC_LDS_ROW_LOAD(12, 640) PIC_LDS_ROW_LOAD(13, 704)
        PIC_LDS_ROW_LOAD(14, 768) PIC_LDS_ROW_LOAD(15, 832) PIC_LDS_ROW_LOAD(16, 896)
        PIC_LDS_ROW_LOAD(17, 960) PIC_LDS_ROW_LOAD(18, 1024) PIC_LDS_ROW_LOAD(19, 1088)
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(src), "s"(b), "s"(b + 960), "s"(b + 2 * 960), "s"(b + 3 * 960), "s"(b + 4 * 960),
          "s"(b + 5 * 960), "s"(b + 6 * 960), "s"(b + 7 * 960), "s"(b + 8 * 960), "s"(b + 9 * 960),
          "s"(b + 10 * 960), "s"(b + 11 * 960), "s"(b + 12 * 960), "s"(b + 13 * 960),
          "s"(b + 14 * 960), "s"(b + 15 * 960), "s"(b + 16 * 960), "s"(b + 17 * 960)
        : "memory");
}
#undef PIC_LDS_ROW_LOAD

// Wait until at most N of the wave's vector memory loads are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N <= 63, "vmcnt holds 6 bits");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

}  // namespace pic
