"""GPU parity of pic_attend_latent (MLA decode attention with the chunks'
rotary keys turned on load) against the fp64 oracle.

Tolerance, from the arithmetic.  The kernel multiplies bf16 query and row
elements on the matrix cores (each product exact in fp32) and accumulates
in fp32, so a logit carries at most scale * (D + 1) * u * S_pj error, with
u = 2^-24, D = 576 and S_pj = sum_d |q_jd k_pd| (the oracle's rows hold the
same bf16 bits the kernel turns on load).  Weights then differ from the
exact ones by a factor within exp(+-2 dz) (the max shift cancels), times
the fast exponential's and the online rescaling's error (< 1e-5 together),
times the hi + lo bf16 split of the weights (< 2^-16).  The value product
(fp32, <= 256 positions per block, then the block merge) adds < 300 u.  The
output is a ratio of weighted sums, so
|out - oracle| <= 2 (2 dz + 1e-5 + 2^-16 + 300 u) max|V|,
with dz taken from the case's own data.  The observed error is printed.
"""
import sys

import numpy as np
import pytest

import oracle
from parity_util import to_host
from pic_workloads import (Chunk, Entry, Request, Workload, config4, normal_values, pool_values,
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


def bound(q, rows, scale, vmax):
    """The derived worst-case error for query rows q [R][Hq][D] over context
    rows [N][D] (all requests' rows pooled: an upper bound)."""
    s = np.abs(f64(q)).reshape(-1, q.shape[-1]) @ np.abs(f64(rows)).T
    dz = scale * (q.shape[-1] + 1) * U * float(s.max())
    return 2 * (2 * dz + 1e-5 + 2.0 ** -16 + 300 * U) * vmax


def run_case(torch, wl, n_heads, seed, layer=0, sink_tokens=0, sink_bias=0.0,
             scale=192 ** -0.5):
    import position_independent_kv_stitch_amd as pic
    pk, _ = pool_values(wl, seed=seed, device="cuda:0")
    ck = normal_values(wl.dst_shape(), wl.dtype, seed + 10, "cuda:0")
    q = normal_values((len(wl.requests), n_heads, wl.row_dim), wl.dtype, seed + 12, "cuda:0")
    plan = pic.Plan.from_workload(wl)
    out = pic.attend_latent(plan, pk, ck, q, layer=layer, scale=scale, sink_tokens=sink_tokens,
                            sink_bias=sink_bias)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    hpk, hck, hq = to_host(pk[layer:layer + 1]), to_host(ck[layer:layer + 1]), to_host(q)
    want = oracle.attend_latent(wl, hpk, hck, hq, layer, scale=scale, sink_tokens=sink_tokens,
                                sink_bias=sink_bias, layer_base=layer)
    rows = np.concatenate([hpk.reshape(-1, wl.row_dim), hck.reshape(-1, wl.row_dim)])
    vmax = float(np.abs(f64(rows[:, :wl.rope_offset])).max())
    tol = bound(hq, rows, scale, vmax)
    err = float(np.abs(got - want).max())
    plan.destroy()
    return err, tol, vmax


@pytest.mark.parametrize("seed", range(16))
def test_random_small(torch_cuda, seed):
    style = "interleaved" if seed % 4 == 3 else "half"
    paged = seed % 2 == 1
    wl = random_small(300 + seed, dtype="bf16", style=style, paged=paged, mla=True,
                      n_requests=1 + seed % 3, n_layers=2, max_len=150 + 40 * (seed % 5))
    if seed % 5 == 4:
        wl = with_paged_pool(wl, page_size=16, seed=seed)
    heads = (16, 32, 128)[seed % 3]
    sink = (4, -15.0) if seed % 2 == 0 else (0, 0.0)
    say(f"latent random seed={seed} style={style} paged={paged} heads={heads} sink={sink}")
    err, tol, vmax = run_case(torch_cuda, wl, heads, seed, layer=seed % 2, sink_tokens=sink[0],
                              sink_bias=sink[1])
    say(f"  max err {err:.3g} (bound {tol:.3g}, max|V| {vmax:.3g})")
    assert err <= tol


@pytest.mark.parametrize("heads", [16, 32, 128])
def test_running_max_moves_late(torch_cuda, heads):
    """Scale 0.5 over 576-dim N(0, 1) rows puts the logits' spread at about
    17 in log2 units, so a later position passes the running maximum by more
    than the lazy slack (2^12) many times after the first step, and the
    accumulators are rescaled while they hold partial sums (the rescale
    differs between one- or two-wave workgroups, 16 and 32 heads, and
    eight-wave ones)."""
    wl = random_small(360 + heads, dtype="bf16", style="half", paged=True, mla=True,
                      n_requests=2, n_layers=1, max_len=700)
    say(f"latent late max heads={heads}")
    err, tol, vmax = run_case(torch_cuda, wl, heads, 21, scale=0.5)
    say(f"  max err {err:.3g} (bound {tol:.3g}, max|V| {vmax:.3g})")
    assert err <= tol


@pytest.mark.parametrize("layer,heads", [(0, 16), (60, 128)])
def test_deepseek_v3_request_full(torch_cuda, layer, heads):
    """The DeepSeek-V3 MLA request (16 chunks x 4096 tokens at random offsets,
    the first at 0 with 32 recompute tokens): one layer, full context."""
    wl = config4()
    say(f"latent deepseek-v3 full layer={layer} heads={heads}")
    err, tol, vmax = run_case(torch_cuda, wl, heads, 7, layer=layer, sink_tokens=4,
                              sink_bias=-15.0)
    say(f"  max err {err:.3g} (bound {tol:.3g})")
    assert err <= tol


def _many_chunk_request(n_chunks, seed):
    """One request: a 64-token cache prefix, then n_chunks chunks of 64 tokens
    from a paged pool of 8-token pages, each moved by its own shift (chunk c
    cached at base 3 c), behind 16-token cache pages; every 4th chunk keeps
    its first 8 tokens for recompute."""
    n, length, prefix, ps = n_chunks, 64, 64, 16
    chunks = [Chunk(i * length, length, 3 * i) for i in range(n)]
    ctx = prefix + n * length
    pages = np.random.default_rng(seed).permutation(-(-ctx // ps)).astype(np.int32)
    entries = [Entry(c, prefix + c * length, length, 8 if c % 4 == 0 else 0) for c in range(n)]
    wl = Workload("many-chunk MLA request", "bf16", 1, 1, 576, 512, 64, "half", 10000.0, False,
                  pool_tokens=n * length, chunks=chunks, requests=[Request(entries, pages, ctx)],
                  page_size=ps, n_phys_pages=len(pages))
    return with_paged_pool(wl, page_size=8, seed=seed)


@pytest.mark.parametrize("heads", [128, 256])
def test_items_of_several_blocks(torch_cuda, heads):
    """The 128-head kernel (four waves of two head groups) on work items of
    several blocks: 1,024 chunks of 64 tokens, each with its own shift, so a
    block (at most 4 shift tables) covers at most 4 chunks while an item
    covers about 5 (128 heads: 256 items) or 9 (256 heads: two head-group
    sets, 128 items) of them; pool pages of 8 tokens make tiles of 8
    positions."""
    wl = _many_chunk_request(1024, 40 + heads)
    say(f"latent items of several blocks heads={heads}")
    err, tol, vmax = run_case(torch_cuda, wl, heads, 40 + heads, sink_tokens=4, sink_bias=-15.0)
    say(f"  max err {err:.3g} (bound {tol:.3g})")
    assert err <= tol


def test_equals_attention_over_the_stitched_cache(torch_cuda):
    """Turning on load equals stitching first and attending over the cache
    (a plan with no placed chunks reads every row from the cache); only the
    accumulation order differs."""
    import position_independent_kv_stitch_amd as pic
    from pic_workloads import Request, Workload
    torch = torch_cuda
    wl = random_small(411, dtype="bf16", mla=True, n_requests=3, n_layers=1, max_len=300)
    pk, _ = pool_values(wl, seed=3, device="cuda:0")
    ck = normal_values(wl.dst_shape(), wl.dtype, 4, "cuda:0")
    q = normal_values((len(wl.requests), 32, wl.row_dim), wl.dtype, 5, "cuda:0")
    plan = pic.Plan.from_workload(wl)
    fused = pic.attend_latent(plan, pk, ck, q, layer=0, scale=0.07)
    stitched = ck.clone()
    pic.stitch(plan, pk, None, stitched, None)
    ctx = [rq.context_len or max(e.dst_offset + e.length for e in rq.entries)
           for rq in wl.requests]
    plain_wl = Workload(wl.name, wl.dtype, 1, 1, wl.row_dim, wl.rope_offset, wl.rope_dim,
                        wl.style, wl.theta, False, pool_tokens=wl.pool_tokens, chunks=wl.chunks,
                        requests=[Request([], rq.page_table, L)
                                  for rq, L in zip(wl.requests, ctx)],
                        capacity=wl.capacity)
    plain = pic.Plan.from_workload(plain_wl)
    over = pic.attend_latent(plain, pk, stitched, q, layer=0, scale=0.07)
    torch.cuda.synchronize()
    vmax = float(stitched[..., :512].abs().max())
    err = float((fused - over).abs().max())
    say(f"latent fused vs stitched: max diff {err:.3g} (max|V| {vmax:.3g})")
    assert err <= 1e-4 * vmax


def test_errors(torch_cuda):
    import position_independent_kv_stitch_amd as pic
    wl = random_small(5, dtype="bf16", mla=True, n_requests=1, n_layers=1)
    pk, _ = pool_values(wl, seed=1, device="cuda:0")
    ck = normal_values(wl.dst_shape(), wl.dtype, 2, "cuda:0")
    plan = pic.Plan.from_workload(wl)
    q = normal_values((1, 24, wl.row_dim), wl.dtype, 3, "cuda:0")
    with pytest.raises(pic.PicError, match="invalid_arg"):
        pic.attend_latent(plan, pk, ck, q, layer=0)  # 24 heads: not a multiple of 16
    q = normal_values((1, 16, wl.row_dim), wl.dtype, 3, "cuda:0")
    with pytest.raises(pic.PicError, match="invalid_arg"):
        pic.attend_latent(plan, pk, ck, q, layer=0, sink_tokens=-1)
    gqa = random_small(6, dtype="bf16", n_requests=1, n_layers=1)
    gplan = pic.Plan.from_workload(gqa)
    gk, _ = pool_values(gqa, seed=1, device="cuda:0")
    gc = normal_values(gqa.dst_shape(), gqa.dtype, 2, "cuda:0")
    with pytest.raises(pic.PicError, match="invalid_arg"):  # not an MLA plan
        lib = gplan._lib
        import ctypes as C
        from position_independent_kv_stitch_amd import _binding as B
        pv = B._view(gk, None, "pool")
        cv = B._view(gc, None, "contig")
        a = B.LatentArgs(q.data_ptr(), q.stride(0), q.stride(1), q.data_ptr(), 0, 0, 16, 0,
                         0.1, 0, 0.0, 0)
        B._check(lib.pic_attend_latent(gplan.handle, C.byref(pv), C.byref(cv), C.byref(a),
                                       None), lib)
