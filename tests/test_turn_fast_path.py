"""The fp32 fast path of the attention kernels' key turn, checked against
exact rounding on the CPU.

The latent and boundary kernels turn a stitched key element r = x c - y s
(or x s + y c) from bf16 x, y and the plan's fp64 cos/sin.  They compute it
in fp32 with the fp32-rounded c, s and keep its bf16 rounding unless the
rounding midpoint above its bf16 truncation lies within
T = 2^-21 (|x| + |y|) + 2^-120 of the fp32 value (rotate.hpp, turn_f32 and
near_midpoint), in which case they redo the plane in fp64.  The argument:
the fp32 value is within about 3 * 2^-24 (|x c| + |y s|) <= 3 * 2^-24
(|x| + |y|) (plus underflow) of the exact one, under half of T and of its
distance to either rounding boundary, so both round the same way.

This test states the rule independently in numpy (fp32 products and sum,
with and without a fused multiply-add) and checks, over millions of
elements and over elements steered next to midpoints, that every element the
rule keeps rounds exactly as the oracle's fp64 turn does.
"""
import numpy as np

import oracle

F32 = np.float32


def bf16_of_f32(v):
    """bf16 bits of fp32 values, round to nearest even (finite values)."""
    u = v.astype(F32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def near_midpoint(r, mag, margin=2.0 ** -21):
    bits = r.view(np.uint32)
    mid = ((bits & np.uint32(0xFFFF0000)) | np.uint32(0x8000)).view(F32)
    with np.errstate(invalid="ignore", over="ignore"):
        # T as one fp32 fused multiply-add (fp64 holds the product exactly)
        t = (mag.astype(np.float64) * margin + 2.0 ** -120).astype(F32)
        return ~(np.abs(r - mid) > t)


def to_bf16_values(bits):
    return (bits.astype(np.uint32) << 16).view(F32)


def check(x, y, c, s, margin=2.0 ** -21):
    """x, y: bf16-exact fp32 arrays; c, s: fp64.  Returns (kept, mismatches)
    over both turned elements, for plain and fused fp32 evaluation."""
    exact_x = oracle.round_bf16(x.astype(np.float64) * c - y.astype(np.float64) * s)
    exact_y = oracle.round_bf16(x.astype(np.float64) * s + y.astype(np.float64) * c)
    c32, s32 = c.astype(F32), s.astype(F32)
    kept = bad = 0
    with np.errstate(over="ignore", invalid="ignore"):
        p1, q1, p2, q2 = x * c32, y * s32, x * s32, y * c32
        variants = [
            (p1 - q1, p2 + q2),
            # fused: one rounding of x c32 - q1 (fp64 holds the product exactly)
            ((x.astype(np.float64) * c32.astype(np.float64) - q1.astype(np.float64)).astype(F32),
             (x.astype(np.float64) * s32.astype(np.float64) + q2.astype(np.float64)).astype(F32)),
        ]
    rho = np.abs(x) + np.abs(y)  # fp32 sum, as the kernel forms it
    for rx, ry in variants:
        for r, mag, exact in ((rx, rho, exact_x), (ry, rho, exact_y)):
            keep = ~near_midpoint(r, mag, margin)
            kept += int(keep.sum())
            bad += int((bf16_of_f32(r[keep]) != exact[keep]).sum())
    return kept, bad


def random_bf16(rng, n, scale=1.0):
    v = (rng.standard_normal(n) * scale).astype(F32)
    return to_bf16_values(bf16_of_f32(v))


def test_random_elements_round_exactly():
    rng = np.random.default_rng(0)
    n = 2_000_000
    x, y = random_bf16(rng, n), random_bf16(rng, n)
    ang = rng.uniform(-1e5, 1e5, n)
    kept, bad = check(x, y, np.cos(ang), np.sin(ang))
    assert kept > 0.99 * 4 * n
    assert bad == 0


def test_wide_magnitudes_and_cancellation():
    rng = np.random.default_rng(1)
    n = 1_000_000
    x = random_bf16(rng, n, 1.0) * F32(2.0) ** rng.integers(-60, 60, n).astype(F32)
    y = x * F32(1.0) + random_bf16(rng, n, 1e-3)  # near-equal pairs: heavy cancellation
    y = to_bf16_values(bf16_of_f32(y))
    ang = rng.uniform(0, 2 * np.pi, n)
    kept, bad = check(x, y, np.cos(ang), np.sin(ang))
    assert bad == 0


def steered_to_midpoints(rng, n):
    """Elements and angles whose turned x lands within a few fp32 ulps of a
    bf16 rounding midpoint."""
    x, y = random_bf16(rng, n), random_bf16(rng, n)
    # target values on bf16 midpoints, then the angle that produces them
    # approximately (x c - y s = rho cos(a + phi))
    rho = np.hypot(x.astype(np.float64), y.astype(np.float64))
    t = rng.uniform(-0.95, 0.95, n) * rho
    tb = to_bf16_values(bf16_of_f32(t.astype(F32))).astype(np.float64)
    ulp = np.abs(tb) * 2.0 ** -8
    mid = tb + 0.5 * ulp * np.sign(rng.standard_normal(n))
    mid = mid + rng.uniform(-4, 4, n) * np.abs(mid) * 2.0 ** -24
    phi = np.arctan2(y.astype(np.float64), x.astype(np.float64))
    a = np.arccos(np.clip(mid / np.maximum(rho, 1e-300), -1, 1)) - phi
    return x, y, np.cos(a), np.sin(a)


def test_elements_steered_next_to_midpoints_are_redone():
    """The rule must keep none of the elements next to midpoints that it
    would round wrongly."""
    rng = np.random.default_rng(2)
    n = 400_000
    kept, bad = check(*steered_to_midpoints(rng, n))
    assert bad == 0
    assert kept < 4 * n  # some were sent to fp64


def test_a_margin_sixteen_times_too_small_fails():
    """The steered elements do come within the fp32 error of a midpoint:
    with 2^-25 in place of 2^-21 some kept element rounds wrongly (the
    typical error is about 2^-24 of the magnitude, the bound 3 * 2^-24)."""
    rng = np.random.default_rng(2)
    kept, bad = check(*steered_to_midpoints(rng, 400_000), margin=2.0 ** -25)
    assert bad > 0


def test_cancellation_next_to_powers_of_two():
    """Heavy cancellation (|x c|, |y s| about 2^12 times the result) with
    results just above or below a power of two, where the bf16 step halves
    and the rounding boundary under the truncation is a quarter step away."""
    rng = np.random.default_rng(3)
    n = 400_000
    e = rng.integers(-20, 20, n).astype(np.float64)
    big = 2.0 ** (e + rng.uniform(11.0, 13.0, n))
    ang0 = rng.uniform(0, 2 * np.pi, n)
    x = to_bf16_values(bf16_of_f32((big * np.cos(ang0)).astype(F32)))
    y = to_bf16_values(bf16_of_f32((big * np.sin(ang0)).astype(F32)))
    rho = np.hypot(x.astype(np.float64), y.astype(np.float64))
    t = 2.0 ** e * (1.0 + rng.integers(-64, 65, n) * 2.0 ** -23)
    t *= np.sign(rng.standard_normal(n))
    phi = np.arctan2(y.astype(np.float64), x.astype(np.float64))
    a = np.arccos(np.clip(t / rho, -1, 1)) - phi
    kept, bad = check(x, y, np.cos(a), np.sin(a))
    assert bad == 0
    assert kept > 0
