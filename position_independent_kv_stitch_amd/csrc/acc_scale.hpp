// Rescaling of matrix-core accumulators held in accumulation registers
// (AGPRs), for the online softmax of the decode attention kernels: when a
// row's running maximum moves, its output accumulator is multiplied by
// 2^(m_old - m_new).
#pragma once

#include <hip/hip_runtime.h>

namespace pic {

// Wait states before the first AGPR read of a rescale: enough for the
// longest matrix-core instruction the kernels issue to have written its
// result, whatever the compiler placed just before the branch.
__device__ __forceinline__ void acc_read_guard() {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
}

// acc *= s for one 4-float accumulator fragment.  Each element is read out,
// multiplied and written back by one asm statement with the value tied to an
// AGPR, so the moves stay inside the caller's branch.  Written as plain
// `acc *= s`, the compiler hoisted the reads of every accumulator to the top
// of the step loop, paying them at every step although the branch is taken
// only when the running maximum moves.
template <typename V4>
__device__ __forceinline__ void scale_acc(V4 &acc, float s) {
#pragma unroll
    for (int e = 0; e < 4; e++) {
        float x = acc[e], tmp;
        asm volatile(
            "v_accvgpr_read_b32 %1, %0\n\t"
            "v_mul_f32_e32 %1, %2, %1\n\t"
            "v_accvgpr_write_b32 %0, %1"
            : "+a"(x), "=&v"(tmp)
            : "v"(s));
        acc[e] = x;
    }
}

}  // namespace pic
