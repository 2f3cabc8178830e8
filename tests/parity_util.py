"""Comparison helpers for GPU-vs-oracle parity (test infrastructure).

The bar: every element outside the rotary slice of K (V rows, the MLA
content latent, untouched destination rows) is bit-identical to the
oracle; rotated fp32 elements are within 1e-5 * max|k| (max over the
case's input keys) in absolute value; rotated bf16 elements are within one
bf16 ulp (distance of the ordered bit patterns).
"""
from __future__ import annotations

import numpy as np

import oracle
from pic_workloads import to_host  # noqa: F401  (re-exported for the tests)

F32_TOL = 1e-5   # x max|k|, absolute
BF16_ULPS = 1




def to_device(a: np.ndarray, device):
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def max_abs(a: np.ndarray) -> float:
    if a.dtype == np.uint16:
        a = (a.astype(np.uint32) << 16).view(np.float32)
    return float(np.max(np.abs(a))) if a.size else 0.0


def _ordered(bits: np.ndarray) -> np.ndarray:
    b = bits.astype(np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def compare_k(got: np.ndarray, want: np.ndarray, rope_offset: int, rope_dim: int,
              maxk: float, what: str = "K") -> dict:
    """Compare K arrays [..., H, D]: bit-exact outside the rotary slice, the
    stated tolerance inside it.  Returns counts; raises AssertionError."""
    assert got.shape == want.shape and got.dtype == want.dtype, (got.shape, want.shape)
    gb = got.view(np.uint32 if got.dtype == np.float32 else np.uint16)
    wb = want.view(gb.dtype)
    diff = gb != wb
    n_diff = int(diff.sum())
    stats = {"elements": int(got.size), "bit_diffs": n_diff, "max_err": 0.0}
    if n_diff == 0:
        return stats
    rot = np.zeros(got.shape[-1], dtype=bool)
    rot[rope_offset:rope_offset + rope_dim] = True
    outside = diff & ~rot
    if outside.any():
        idx = np.argwhere(outside)[0]
        raise AssertionError(f"{what}: {int(outside.sum())} non-rotary elements differ, first "
                             f"at {tuple(idx)}: got {gb[tuple(idx)]:#x} want {wb[tuple(idx)]:#x}")
    if got.dtype == np.float32:
        g, w = got[diff].astype(np.float64), want[diff].astype(np.float64)
        err = np.abs(g - w)
        bad = ~(err <= F32_TOL * maxk)
        stats["max_err"] = float(np.nanmax(err)) if err.size else 0.0
    else:
        d = np.abs(_ordered(gb[diff]) - _ordered(wb[diff]))
        bad = d > BF16_ULPS
        stats["max_err"] = int(d.max())
    if bad.any():
        raise AssertionError(f"{what}: {int(bad.sum())} rotated elements beyond tolerance "
                             f"(max {stats['max_err']})")
    return stats


def compare_bits(got: np.ndarray, want: np.ndarray, what: str):
    assert got.shape == want.shape, (got.shape, want.shape)
    if not np.array_equal(got.view(np.uint8), want.view(np.uint8)):
        gb = got.view(np.uint32 if got.dtype == np.float32 else np.uint16)
        wb = want.view(gb.dtype)
        idx = np.argwhere(gb != wb)
        raise AssertionError(f"{what}: {len(idx)} elements differ, first at {tuple(idx[0])}")


def check_stitch_case(wl, device="cuda:0", seed=0, layer_begin=0, layer_end=None):
    """Stitch `wl` on the GPU through the C ABI and compare everything with the
    oracle on the same inputs.  Returns the comparison counts."""
    import torch

    import position_independent_kv_stitch_amd as pic
    from pic_workloads import pool_values, sentinel_like

    le = wl.n_layers if layer_end is None else layer_end
    pk, pv = pool_values(wl, seed=seed, device=device)
    dk = sentinel_like(wl.dst_shape(), wl.dtype, device)
    dv = sentinel_like(wl.dst_shape(), wl.dtype, device) if wl.has_v else None
    plan = pic.Plan.from_workload(wl)
    pic.stitch(plan, pk, pv, dk, dv, layer_begin, le)
    torch.cuda.synchronize()
    hk, hv = to_host(pk), to_host(pv) if pv is not None else None
    rk = to_host(sentinel_like(wl.dst_shape(), wl.dtype, "cpu"))
    rv = rk.copy() if wl.has_v else None
    assert oracle.stitch(wl, hk, hv, rk, rv, layer_begin, le) == "ok"
    stats = compare_k(to_host(dk), rk, wl.rope_offset, wl.rope_dim, max_abs(hk))
    if wl.has_v:
        compare_bits(to_host(dv), rv, "V")
    plan.destroy()
    return stats
