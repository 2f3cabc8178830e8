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

// Wait until at most N of the wave's vector memory loads are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N <= 63, "vmcnt holds 6 bits");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

}  // namespace pic
