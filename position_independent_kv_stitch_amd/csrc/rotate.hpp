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

// ------------------------------------------------- fp32 fast path of a turn
//
// A turned element r = x c - y s (or x s + y c) computed in fp32 from bf16 x,
// y and the fp32-rounded c, s lies within 3 * 2^-24 (|x c| + |y s|) of the
// value the fp64 turn rounds (itself within 2^-52 of that sum of the exact
// one).  Its round-to-nearest-even bf16 is therefore the fp64 path's unless a
// bf16 rounding midpoint lies that close to r: near_midpoint() reports that
// case with a 2^-21 margin, and also non-finite values and products so small
// that fp32 may have lost them, so that the caller redoes the element in
// fp64.  The midpoint nearest r keeps r's sign, exponent and top 7 fraction
// bits and has 0x8000 below; r and it share a binade, so r - mid is exact.
__device__ __forceinline__ bool near_midpoint(float r, float mag) {
    const float mid = __uint_as_float((__float_as_uint(r) & 0xFFFF0000u) | 0x8000u);
    return !(fabsf(r - mid) > mag * 0x1p-21f) || !(mag > 0x1p-100f);
}

// Two fp32 values rounded to bf16 (nearest even), packed low first.
__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// Turn of one plane in fp32: *rx = x c - y s, *ry = x s + y c; returns true
// when either result needs the fp64 path.
__device__ __forceinline__ bool turn_f32(float x, float y, float c, float s, float *rx, float *ry) {
    const float p1 = x * c, q1 = y * s, p2 = x * s, q2 = y * c;
    *rx = p1 - q1;
    *ry = p2 + q2;
    const bool bx = near_midpoint(*rx, fabsf(p1) + fabsf(q1));
    const bool by = near_midpoint(*ry, fabsf(p2) + fabsf(q2));
    return bx || by;
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
