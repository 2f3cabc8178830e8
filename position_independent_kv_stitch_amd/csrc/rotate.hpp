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
// one), plus at most 2^-123 lost to underflow or flushed subnormals; and
// |x c| + |y s| <= |x| + |y| for either element.  Its round-to-nearest-even
// bf16 is therefore the fp64 path's unless a rounding boundary lies that
// close to r.  near_midpoint() takes T = 2^-21 (|x| + |y|) + 2^-120 (the
// caller's t) and reports |r - mid| <= T, mid being the midpoint above r's
// bf16 truncation (r's sign, exponent and top 7 fraction bits, then 0x8000;
// r and mid share a binade, so r - mid is exact).  When it does not, the
// error is below T / 2 and below |r - mid| / 2, and the boundary under the
// truncation is at least |r - mid| / 2 away (a quarter of a bf16 step, where
// the truncation is a power of two), so both round alike.  Non-finite r or T
// also report, and the caller redoes the plane in fp64.
__device__ __forceinline__ bool near_midpoint(float r, float t) {
    const float mid = __uint_as_float((__float_as_uint(r) & 0xFFFF0000u) | 0x8000u);
    return !(fabsf(r - mid) > t);
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
    *rx = fmaf(x, c, -(y * s));
    *ry = fmaf(x, s, y * c);
    const float t = fmaf(fabsf(x) + fabsf(y), 0x1p-21f, 0x1p-120f);
    return near_midpoint(*rx, t) || near_midpoint(*ry, t);
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
