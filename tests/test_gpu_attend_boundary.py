"""GPU parity of pic_attend_boundary (LegoLink boundary reconnection: the
first boundary_k tokens of every relocated chunk attend causally over the
stitched context, chunk keys turned on load) against the fp64 oracle.

Tolerance, from the arithmetic (as for the latent attention): bf16 query and
row elements multiply exactly on the matrix cores and accumulate in fp32,
so a logit carries at most scale * (D + 1) * u * S_pj error (u = 2^-24,
D = 128, S_pj = sum_d |q_jd k_pd|; the oracle's rows hold the bits the
kernel turns on load).  Weights differ by a factor within exp(+-2 dz),
times the fast exponential and online rescaling (< 1e-5) and the hi + lo
bf16 split (< 2^-16); the value product and the merge add < 300 u.  So
|out - oracle| <= 2 (2 dz + 1e-5 + 2^-16 + 300 u) max|V|, dz from the case's
data.  The observed error is printed.
"""
import sys

import numpy as np
import pytest

import oracle
from parity_util import to_host
from pic_workloads import (Request, Workload, decode_batch, normal_values, pool_values,
                           random_small, with_paged_pool)

pytestmark = pytest.mark.gpu
U = 2.0 ** -24


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch_cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import position_independent_kv_stitch_amd  # noqa: F401
    return torch


def f64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def run_case(torch, wl, group, k, seed, layer=0, sink_tokens=0, sink_bias=0.0, scale=0.09):
    import position_independent_kv_stitch_amd as pic
    pk, pv = pool_values(wl, seed=seed, device="cuda:0")
    ck = normal_values(wl.dst_shape(), wl.dtype, seed + 10, "cuda:0")
    cv = normal_values(wl.dst_shape(), wl.dtype, seed + 11, "cuda:0")
    plan = pic.Plan.from_workload(wl)
    n = pic.boundary_row_count(plan, k)
    rows = oracle.boundary_rows(wl, k)
    assert n == len(rows)
    if n == 0:
        plan.destroy()
        return 0.0, 0.0, 0
    q = normal_values((n, wl.n_heads * group, wl.row_dim), wl.dtype, seed + 12, "cuda:0")
    out = pic.attend_boundary(plan, pk, pv, ck, cv, q, layer=layer, boundary_k=k, scale=scale,
                              sink_tokens=sink_tokens, sink_bias=sink_bias)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    L1 = slice(layer, layer + 1)
    hq = to_host(q)
    want = oracle.attend_boundary(wl, to_host(pk[L1]), to_host(pv[L1]), to_host(ck[L1]),
                                  to_host(cv[L1]), hq, layer, k, scale=scale,
                                  sink_tokens=sink_tokens, sink_bias=sink_bias, layer_base=layer)
    keys = np.concatenate([to_host(pk[L1]).reshape(-1, wl.row_dim),
                           to_host(ck[L1]).reshape(-1, wl.row_dim)])
    vals = np.concatenate([to_host(pv[L1]).reshape(-1, wl.row_dim),
                           to_host(cv[L1]).reshape(-1, wl.row_dim)])
    s = np.abs(f64(hq)).reshape(-1, wl.row_dim) @ np.abs(f64(keys)).T
    dz = scale * (wl.row_dim + 1) * U * float(s.max())
    tol = 2 * (2 * dz + 1e-5 + 2.0 ** -16 + 300 * U) * float(np.abs(f64(vals)).max())
    err = float(np.abs(got - want).max())
    plan.destroy()
    return err, tol, n


@pytest.mark.parametrize("seed", range(16))
def test_random_small(torch_cuda, seed):
    style = "interleaved" if seed % 4 == 3 else "half"
    paged = seed % 2 == 1
    wl = random_small(500 + seed, dtype="bf16", style=style, paged=paged,
                      n_requests=1 + seed % 3, n_layers=2, max_len=60 + 30 * (seed % 4))
    if seed % 5 == 4:
        wl = with_paged_pool(wl, page_size=16, seed=seed)
    group = (1, 2, 4, 8)[seed % 4]
    k = (16, 5, 1, 16)[seed % 4] if group < 8 else 16
    sink = (4, -15.0) if seed % 2 == 0 else (0, 0.0)
    say(f"boundary random seed={seed} style={style} paged={paged} group={group} k={k} sink={sink}")
    err, tol, n = run_case(torch_cuda, wl, group, k, seed, layer=seed % 2, sink_tokens=sink[0],
                           sink_bias=sink[1])
    say(f"  rows {n}: max err {err:.3g} (bound {tol:.3g})")
    assert err <= tol


@pytest.mark.parametrize("style,dims", [("half", (2, 128, 32, 64)), ("interleaved", (2, 128, 16, 64)),
                                        ("half", (1, 128, 96, 32)), ("interleaved", (2, 128, 112, 16))])
def test_partial_rotary_slices(torch_cuda, style, dims):
    """Rotary slices narrower than the row and away from dim 0: only some
    waves hold turn units, and the turned pieces sit at other offsets."""
    seed = dims[2] + dims[3]
    wl = random_small(1200 + seed, dtype="bf16", style=style, n_requests=2, n_layers=1,
                      max_len=90, dims=dims)
    say(f"boundary partial rotary style={style} dims={dims}")
    err, tol, n = run_case(torch_cuda, wl, 4, 16, seed, sink_tokens=4, sink_bias=-15.0)
    say(f"  rows {n}: max err {err:.3g} (bound {tol:.3g})")
    assert n > 0
    assert err <= tol


def test_long_k_and_short_entries(torch_cuda):
    """boundary_k larger than some entries (rows = their length), k x group
    = 128 (eight row tiles)."""
    wl = random_small(777, dtype="bf16", n_requests=2, n_layers=1, max_len=40)
    err, tol, n = run_case(torch_cuda, wl, 4, 32, 3)
    say(f"boundary k=32 group=4: rows {n}, max err {err:.3g} (bound {tol:.3g})")
    assert err <= tol


@pytest.mark.parametrize("k,group", [(17, 8), (40, 8), (64, 3)])
def test_many_rows_per_request(torch_cuda, k, group):
    """More rows per request and KV head than one workgroup holds (256):
    the rows are split over row sets that read the same context."""
    wl = random_small(900 + k, dtype="bf16", n_requests=3, n_layers=1, max_len=120)
    err, tol, n = run_case(torch_cuda, wl, group, k, 4, sink_tokens=4, sink_bias=-15.0)
    say(f"boundary k={k} group={group}: rows {n}, max err {err:.3g} (bound {tol:.3g})")
    assert err <= tol


def test_llama3_decode_batch_two_requests(torch_cuda):
    """Two requests of the Llama-3-8B decode batch (8 chunks x 2048 behind a
    128-token prefix, recompute_k 32, 16-token pages): k = 16, 32 query
    heads, LegoLink damping; contexts of up to 14,464 positions."""
    base = decode_batch(n_requests=2, n_layers=2)
    say("boundary llama3 decode batch, 2 requests")
    err, tol, n = run_case(torch_cuda, base, 4, 16, 5, layer=1, sink_tokens=4, sink_bias=-15.0,
                           scale=128 ** -0.5)
    say(f"  rows {n}: max err {err:.3g} (bound {tol:.3g})")
    assert n == 2 * 8 * 16
    assert err <= tol


def test_errors(torch_cuda):
    import position_independent_kv_stitch_amd as pic
    wl = random_small(9, dtype="bf16", n_requests=1, n_layers=1)
    plan = pic.Plan.from_workload(wl)
    pk, pv = pool_values(wl, seed=1, device="cuda:0")
    ck = normal_values(wl.dst_shape(), wl.dtype, 2, "cuda:0")
    n = pic.boundary_row_count(plan, 17)
    assert n > 0
    q = normal_values((n, 16, wl.row_dim), wl.dtype, 3, "cuda:0")
    import ctypes as C
    from position_independent_kv_stitch_amd import _binding as B
    out = torch_cuda.empty(q.shape, dtype=torch_cuda.float32, device="cuda:0")
    with pytest.raises(pic.PicError, match="invalid_arg"):  # boundary_k < 1
        a = B.BoundaryArgs(q.data_ptr(), q.stride(0), q.stride(1), out.data_ptr(), out.stride(0),
                           out.stride(1), 16, 0, 0.1, 0, 0, 0.0)
        B._check(plan._lib.pic_attend_boundary(
            plan.handle, C.byref(B._view(pk, pv, "pool")), C.byref(B._view(ck, ck, "contig")),
            C.byref(a), None), plan._lib)
    with pytest.raises(pic.PicError, match="invalid_arg"):  # f32 plans are refused
        f32 = random_small(9, dtype="f32", n_requests=1, n_layers=1)
        fplan = pic.Plan.from_workload(f32)
        fk, fv = pool_values(f32, seed=1, device="cuda:0")
        fc = normal_values(f32.dst_shape(), f32.dtype, 2, "cuda:0")
        a = B.BoundaryArgs(q.data_ptr(), q.stride(0), q.stride(1), q.data_ptr(), 0, 0, 4, 0,
                           0.1, 4, 0, 0.0)
        B._check(fplan._lib.pic_attend_boundary(
            fplan.handle, C.byref(B._view(fk, fv, "pool")), C.byref(B._view(fc, fc, "contig")),
            C.byref(a), None), fplan._lib)


# ------------------------------------------------------------ caller rows

def pick_rows(wl, rng, per_request=24, spread=1.0):
    """(entry, token) rows chosen at random, request by request: any entry
    (those at position 0 too), tokens anywhere in the entry, shuffled within
    the request, some repeated."""
    rows, e0 = [], 0
    for rq in wl.requests:
        mine = []
        for i, e in enumerate(rq.entries):
            n = max(1, int(per_request * spread * e.length / max(1, sum(x.length for x in rq.entries))))
            for j in rng.integers(0, e.length, size=n):
                mine.append((e0 + i, int(j)))
        if mine:
            mine.append(mine[int(rng.integers(0, len(mine)))])  # a repeat
        rng.shuffle(mine)
        rows += mine
        e0 += len(rq.entries)
    return rows


def run_rows_case(torch, wl, group, rows, seed, layer=0, sink_tokens=0, sink_bias=0.0, scale=0.09):
    import position_independent_kv_stitch_amd as pic
    pk, pv = pool_values(wl, seed=seed, device="cuda:0")
    ck = normal_values(wl.dst_shape(), wl.dtype, seed + 10, "cuda:0")
    cv = normal_values(wl.dst_shape(), wl.dtype, seed + 11, "cuda:0")
    plan = pic.Plan.from_workload(wl)
    q = normal_values((len(rows), wl.n_heads * group, wl.row_dim), wl.dtype, seed + 12, "cuda:0")
    out = pic.attend_boundary(plan, pk, pv, ck, cv, q, layer=layer, rows=rows, scale=scale,
                              sink_tokens=sink_tokens, sink_bias=sink_bias)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    L1 = slice(layer, layer + 1)
    hq = to_host(q)
    want = oracle.attend_boundary(wl, to_host(pk[L1]), to_host(pv[L1]), to_host(ck[L1]),
                                  to_host(cv[L1]), hq, layer, 0, scale=scale,
                                  sink_tokens=sink_tokens, sink_bias=sink_bias, layer_base=layer,
                                  rows=rows)
    keys = np.concatenate([to_host(pk[L1]).reshape(-1, wl.row_dim),
                           to_host(ck[L1]).reshape(-1, wl.row_dim)])
    vals = np.concatenate([to_host(pv[L1]).reshape(-1, wl.row_dim),
                           to_host(cv[L1]).reshape(-1, wl.row_dim)])
    s = np.abs(f64(hq)).reshape(-1, wl.row_dim) @ np.abs(f64(keys)).T
    dz = scale * (wl.row_dim + 1) * U * float(s.max())
    tol = 2 * (2 * dz + 1e-5 + 2.0 ** -16 + 300 * U) * float(np.abs(f64(vals)).max())
    err = float(np.abs(got - want).max())
    plan.destroy()
    return err, tol


@pytest.mark.parametrize("seed", range(8))
def test_caller_rows_random(torch_cuda, seed):
    """Rows the caller names (the page leaves the choice of "top-k" boundary
    tokens open): random tokens of every entry, repeats, shuffled within
    each request, several requests, paged and contiguous caches, pools
    paged or not, groups 1-8."""
    rng = np.random.default_rng(seed)
    wl = random_small(1500 + seed, dtype="bf16", style="interleaved" if seed % 4 == 3 else "half",
                      paged=seed % 2 == 1, n_requests=1 + seed % 3, n_layers=2,
                      max_len=60 + 40 * (seed % 3))
    if seed % 4 == 2:
        wl = with_paged_pool(wl, page_size=16, seed=seed)
    group = (1, 2, 4, 8)[seed % 4]
    rows = pick_rows(wl, rng, per_request=(8, 40, 120)[seed % 3])
    sink = (4, -15.0) if seed % 2 == 0 else (0, 0.0)
    say(f"caller rows seed={seed}: {len(rows)} rows, group {group}, sink {sink}")
    err, tol = run_rows_case(torch_cuda, wl, group, rows, seed, layer=seed % 2,
                             sink_tokens=sink[0], sink_bias=sink[1])
    say(f"  max err {err:.3g} (bound {tol:.3g})")
    assert err <= tol


def test_caller_rows_top_k_of_decode_batch(torch_cuda):
    """Two Llama-3-8B decode requests: for every relocated chunk 16 tokens
    picked from its first 64 (a top-k selection as a caller would make
    it), 32 query heads, LegoLink damping; and the first-16 selection given
    as rows equals the default path bit for bit."""
    import position_independent_kv_stitch_amd as pic
    torch = torch_cuda
    wl = decode_batch(n_requests=2, n_layers=2)
    rng = np.random.default_rng(7)
    rows, e0 = [], 0
    for rq in wl.requests:
        for i, e in enumerate(rq.entries):
            for j in np.sort(rng.choice(64, size=16, replace=False)):
                rows.append((e0 + i, int(j)))
        e0 += len(rq.entries)
    say(f"top-k rows of the decode batch: {len(rows)}")
    err, tol = run_rows_case(torch, wl, 4, rows, 5, layer=1, sink_tokens=4, sink_bias=-15.0,
                             scale=128 ** -0.5)
    say(f"  max err {err:.3g} (bound {tol:.3g})")
    assert err <= tol
    # the default selection, given explicitly
    pk, pv = pool_values(wl, seed=5, device="cuda:0")
    ck = normal_values(wl.dst_shape(), wl.dtype, 15, "cuda:0")
    cv = normal_values(wl.dst_shape(), wl.dtype, 16, "cuda:0")
    plan = pic.Plan.from_workload(wl)
    first = [(e, j) for e, (_, b, end) in enumerate(plan.ranges()[0]) if b > 0
             for j in range(min(16, int(end - b)))]
    q = normal_values((len(first), 32, 128), wl.dtype, 17, "cuda:0")
    a = pic.attend_boundary(plan, pk, pv, ck, cv, q, layer=0, boundary_k=16, sink_tokens=4,
                            sink_bias=-15.0)
    b = pic.attend_boundary(plan, pk, pv, ck, cv, q, layer=0, rows=first, sink_tokens=4,
                            sink_bias=-15.0)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    plan.destroy()
