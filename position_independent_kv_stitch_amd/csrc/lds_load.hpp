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
__device__ __forceinline__ void load_lds16(const void *src, const void *lds) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(
        reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void *)lds)));
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(src), "s"(m0)
                 : "memory", "m0");
}

// Wait until at most N of the wave's vector memory loads are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N <= 63, "vmcnt holds 6 bits");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

}  // namespace pic
