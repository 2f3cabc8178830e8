// rotate.hpp -- storage conversions and the rotation of rotary units, in
// fp64 with one round-to-nearest-even into the storage type.  Shared by the
// stitch kernel (stitch.hip) and the latent attention kernel
// (attend_mla.hip), so that a key turned on load has exactly the bits the
// stitch would have stored.
//
// A pair (x, y) of plane i turns to (x c - y s, x s + y c), with c, s the
// cosine and sine of delta * theta_i (EPIC Guide: Position-Independent
// Caching for LLM Serving, "Mathematical Foundations", sections 1 and 2).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "pic_stitch.h"

namespace pic {

// ------------------------------------------------------ storage conversion

// bf16 -> fp32 is a 16-bit shift, exact; fp32 -> fp64 exact.
__device__ __forceinline__ double bf16_lo(uint32_t w) {
    return static_cast<double>(__uint_as_float(w << 16));
}
__device__ __forceinline__ double bf16_hi(uint32_t w) {
    return static_cast<double>(__uint_as_float(w & 0xFFFF0000u));
}

// fp64 -> bf16 with one round-to-nearest-even: first to fp32 with
// round-to-odd (truncate, then set the last bit when inexact), which keeps
// enough information for the final 8-bit rounding to be the correct one,
// then fp32 -> bf16 round-to-nearest-even on the bit pattern.
__device__ __forceinline__ uint32_t f64_to_bf16(double d) {
    const float f = static_cast<float>(d);  // nearest
    uint32_t u = __float_as_uint(f);
    const double back = static_cast<double>(f);
    if (back != d) {
        if (fabs(back) > fabs(d)) u -= 1u;  // step the magnitude down: truncation
        u |= 1u;                            // sticky bit: round-to-odd
    }
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16(double lo, double hi) {
    return f64_to_bf16(lo) | (f64_to_bf16(hi) << 16);
}

// ----------------------------------------------------------------- rotation

template <typename E>
struct Vec;

template <>
struct Vec<float> {
    static constexpr int kElems = 4;
};
template <>
struct Vec<uint16_t> {
    static constexpr int kElems = 8;
};

// Rotation of one rotary unit held in NW 32-bit words, with c[p], s[p] the
// cosine and sine of the unit's plane p.
//   HALF pairing: words a hold the x of the unit's planes, words b their y
//     (bf16: two planes per word, low half first; f32: one plane per word).
//   INTERLEAVED pairing: words a hold (x, y) of consecutive planes (bf16:
//     one plane per word; f32: one plane per two words); b is unused.
template <typename E, int STYLE, int NW>
__device__ __forceinline__ void rotate_unit(uint32_t (&a)[NW], uint32_t (&b)[NW],
                                            const double *c, const double *s) {
    if constexpr (sizeof(E) == 2) {
        if constexpr (STYLE == PIC_ROPE_HALF) {
#pragma unroll
            for (int k = 0; k < NW; k++) {
                const double x0 = bf16_lo(a[k]), x1 = bf16_hi(a[k]);
                const double y0 = bf16_lo(b[k]), y1 = bf16_hi(b[k]);
                const double c0 = c[2 * k], s0 = s[2 * k], c1 = c[2 * k + 1], s1 = s[2 * k + 1];
                a[k] = pack_bf16(x0 * c0 - y0 * s0, x1 * c1 - y1 * s1);
                b[k] = pack_bf16(x0 * s0 + y0 * c0, x1 * s1 + y1 * c1);
            }
        } else {
#pragma unroll
            for (int k = 0; k < NW; k++) {
                const double x = bf16_lo(a[k]), y = bf16_hi(a[k]);
                a[k] = pack_bf16(x * c[k] - y * s[k], x * s[k] + y * c[k]);
            }
        }
    } else {
        if constexpr (STYLE == PIC_ROPE_HALF) {
#pragma unroll
            for (int k = 0; k < NW; k++) {
                const double x = __uint_as_float(a[k]), y = __uint_as_float(b[k]);
                a[k] = __float_as_uint(static_cast<float>(x * c[k] - y * s[k]));
                b[k] = __float_as_uint(static_cast<float>(x * s[k] + y * c[k]));
            }
        } else {
#pragma unroll
            for (int k = 0; k < NW / 2; k++) {
                const double x = __uint_as_float(a[2 * k]), y = __uint_as_float(a[2 * k + 1]);
                a[2 * k] = __float_as_uint(static_cast<float>(x * c[k] - y * s[k]));
                a[2 * k + 1] = __float_as_uint(static_cast<float>(x * s[k] + y * c[k]));
            }
        }
    }
}

}  // namespace pic
