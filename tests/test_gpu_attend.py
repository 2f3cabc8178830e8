"""GPU parity of pic_attend (decode attention with the chunks' delta-rotation
done on load) against the fp64 oracle.

Tolerance, from the arithmetic: the kernel computes logits, weights and
sums in fp32 (unit roundoff u = 2^-24).  A logit carries at most
scale * (D + 4) * u * sum_i |q_i k_i| error (dot product plus the fp32
rotation with cos/sin rounded to fp32); for N(0, 1) rows and D = 128 that is
below 6e-5.  The weights then carry relative error <= 2 * 6e-5 + 4u, the
block sums (<= 256 terms) and the cross-block combine add <= 320u, and the
output is a convex combination of value rows.  So
|out - oracle| <= 2e-4 * max|V| covers the worst case with margin; the test
asserts 5e-4 * max|V|.

bf16 plans with 128-dim rows take the matrix-core path, which turns the
query instead of the keys and keeps the turned query as three bf16 terms
(within 2^-24 of it, so the logit bound above holds) and the weights as two
(relative error < 2^-16, adding < 2e-5 * max|V| to the output bound).
"""
import sys

import numpy as np
import pytest

import oracle
from parity_util import to_host
from pic_workloads import (Chunk, Entry, Request, Workload, config2, normal_values,
                           pool_values, random_small, with_paged_pool)

pytestmark = pytest.mark.gpu
TOL = 5e-4


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


def cache_shape(wl):
    return wl.dst_shape()


def run_case(torch, wl, group, seed, layer=0, sink_tokens=0, sink_bias=0.0, scale=None):
    import position_independent_kv_stitch_amd as pic
    pk, pv = pool_values(wl, seed=seed, device="cuda:0")
    ck = normal_values(cache_shape(wl), wl.dtype, seed + 10, "cuda:0")
    cv = normal_values(cache_shape(wl), wl.dtype, seed + 11, "cuda:0")
    q = normal_values((len(wl.requests), wl.n_heads * group, wl.row_dim), wl.dtype, seed + 12,
                      "cuda:0")
    plan = pic.Plan.from_workload(wl)
    out = pic.attend(plan, pk, pv, ck, cv, q, layer=layer, sink_tokens=sink_tokens,
                     sink_bias=sink_bias, scale=scale)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    hcv = to_host(cv[layer:layer + 1])
    want = oracle.attend(wl, to_host(pk[layer:layer + 1]), to_host(pv[layer:layer + 1]),
                         to_host(ck[layer:layer + 1]), hcv, to_host(q), layer, scale=scale,
                         sink_tokens=sink_tokens, sink_bias=sink_bias, layer_base=layer)
    vmax = max(np.abs(oracle.ref._to_f64(hcv)).max(),
               np.abs(oracle.ref._to_f64(to_host(pv[layer:layer + 1]))).max())
    err = np.abs(got - want).max()
    plan.destroy()
    return err, vmax


def with_context(wl, rng, extra=7):
    """Give every request a context reaching a little past its last entry."""
    for r, rq in enumerate(wl.requests):
        end = max([e.dst_offset + e.length for e in rq.entries] + [1])
        span = len(rq.page_table) * wl.page_size if wl.page_size else wl.capacity
        rq.context_len = int(min(span, end + int(rng.integers(0, extra + 1))))
    return wl


CASES = [(seed, dt, paged, group, pp)
         for seed in range(2)
         for dt in ("f32", "bf16")
         for paged in (False, True)
         for group in (1, 4, 8)
         for pp in (False, True)]


@pytest.mark.parametrize("seed,dt,paged,group,pp", CASES)
def test_attend_small(torch_cuda, seed, dt, paged, group, pp):
    rng = np.random.default_rng(seed)
    wl = random_small(30 + seed, dtype=dt, paged=paged, n_requests=3, n_layers=2, max_len=300,
                      deltas=[0, 1, -7, 65536, -65536, 12345])
    if pp:
        wl = with_paged_pool(wl, page_size=16, seed=seed, first_offsets=True)
    wl = with_context(wl, rng)
    say(f"attend seed={seed} {dt} paged={paged} group={group} paged_pool={pp}")
    err, vmax = run_case(torch_cuda, wl, group, seed, layer=1)
    assert err <= TOL * vmax, (err, vmax)


SHAPES = [  # (storage, pairing, (kv heads, row_dim, rope_offset, rope_dim), group)
    ("bf16", "half", (4, 64, 0, 64), 2),
    ("bf16", "half", (4, 64, 0, 64), 8),
    ("bf16", "half", (2, 128, 64, 64), 4),
    ("bf16", "half", (2, 128, 0, 64), 3),
    ("bf16", "interleaved", (2, 128, 32, 64), 6),
    ("f32", "half", (2, 64, 0, 32), 8),
    ("bf16", "half", (1, 256, 0, 128), 4),
    ("f32", "interleaved", (2, 256, 128, 128), 1),
]


@pytest.mark.parametrize("dt,style,dims,group", SHAPES)
def test_attend_shapes(torch_cuda, dt, style, dims, group):
    """Partial rotary slices at an offset, narrow and wide rows, groups that
    do not fill the kernel's head slots."""
    rng = np.random.default_rng(11)
    wl = with_context(random_small(50, dtype=dt, style=style, paged=True, n_requests=2,
                                   n_layers=1, max_len=200, deltas=[0, 3, -4096, 70000],
                                   dims=dims), rng)
    say(f"attend shape {dt} {style} {dims} group={group}")
    err, vmax = run_case(torch_cuda, wl, group, 5, layer=0, sink_tokens=4, sink_bias=-15.0)
    assert err <= TOL * vmax, (err, vmax)


@pytest.mark.parametrize("style,dims", [("half", (2, 128, 0, 128)), ("interleaved", (2, 128, 32, 64))])
def test_attend_many_short_chunks(torch_cuda, style, dims):
    """Many short chunks at distinct shifts in one request (bf16, 128-dim
    rows: the matrix-core path): 16-position tiles that mix chunks, blocks cut
    at their shift-table limit, a context shorter than one step in another
    request, and a one-position context."""
    rng = np.random.default_rng(77)
    heads, row, roff, rdim = dims
    lens = [int(n) for n in rng.integers(3, 24, size=14)]
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]])
    chunks = [Chunk(int(st), n, int(rng.integers(0, 500))) for st, n in zip(starts, lens)]
    entries, pos = [], 5
    for c in range(len(chunks)):
        entries.append(Entry(c, pos, lens[c], int(rng.integers(0, 2))))
        pos += lens[c] + int(rng.integers(0, 3))
    reqs = [Request(entries, None, pos + 3),
            Request([Entry(0, 2, lens[0], 0)], None, lens[0] + 2 + 5),  # shorter than one step
            Request([], None, 1)]  # one position, no chunk
    cap = pos + 8
    wl = Workload("short-chunks", "bf16", 2, heads, row, roff, rdim, style, 500000.0, True,
                  pool_tokens=int(sum(lens)), chunks=chunks, requests=reqs, capacity=cap)
    for group in (1, 4, 8):
        say(f"attend many short chunks style={style} group={group}")
        err, vmax = run_case(torch_cuda, wl, group, 3, layer=1, sink_tokens=2, sink_bias=-5.0)
        say(f"  max err {err:.3g} (tol {TOL * vmax:.3g})")
        assert err <= TOL * vmax, (err, vmax)


def test_attend_one_token_pool_pages(torch_cuda):
    """A pool of 1-token pages: every pool position is its own tile, so blocks
    stop at the per-block tile limit rather than at their length."""
    rng = np.random.default_rng(12)
    wl = with_paged_pool(random_small(51, dtype="bf16", n_requests=2, n_layers=1, max_len=120),
                         page_size=1, seed=3)
    wl = with_context(wl, rng)
    err, vmax = run_case(torch_cuda, wl, 4, 6)
    assert err <= TOL * vmax, (err, vmax)


@pytest.mark.parametrize("style", ["half", "interleaved"])
def test_attend_sink_damping(torch_cuda, style):
    """LegoLink pseudo-sink damping (-15 on 4 tokens) on chunks placed after
    position 0; a chunk at position 0 keeps its sink."""
    rng = np.random.default_rng(5)
    wl = random_small(41, dtype="bf16", style=style, n_requests=2, n_layers=1, max_len=200)
    wl.requests[0].entries[0] = Entry(wl.requests[0].entries[0].chunk_id, 0,
                                      wl.requests[0].entries[0].length, 0)
    wl = with_context(wl, rng)
    err, vmax = run_case(torch_cuda, wl, 4, 3, sink_tokens=4, sink_bias=-15.0)
    assert err <= TOL * vmax, (err, vmax)


def test_attend_llama3_decode_full(torch_cuda):
    """Llama-3-8B shape: 32 query heads over 8 KV heads, one request whose
    16,512-position context is 8 stitched chunks of 2048 tokens (the first
    32 of each from the request's own cache) behind a 128-token prefix,
    paged cache; sampled layers; with and without LegoLink damping."""
    wl = config2()
    wl.requests[0].context_len = 128 + 8 * 2048
    for layer, sink in [(0, 0), (31, 4)]:
        say(f"llama3 decode layer {layer} sink {sink}")
        err, vmax = run_case(torch_cuda, wl, 4, 7, layer=layer, sink_tokens=sink,
                             sink_bias=-15.0)
        say(f"  max err {err:.3g} (tol {TOL * vmax:.3g})")
        assert err <= TOL * vmax


def test_attend_decode_batch(torch_cuda):
    """Sixteen Llama-3-shaped decode requests of 16,512 positions each (each
    request's own 8 chunks of 2048): 256-position blocks, one layer."""
    from pic_workloads import decode_batch
    wl = decode_batch(n_requests=16, n_layers=1)
    say("decode batch 16 x 16512")
    err, vmax = run_case(torch_cuda, wl, 4, 8, layer=0, sink_tokens=4, sink_bias=-15.0)
    say(f"  max err {err:.3g} (tol {TOL * vmax:.3g})")
    assert err <= TOL * vmax


def test_attend_matches_stitch_then_attend(torch_cuda):
    """Rotate-on-load equals stitching the chunks into the cache and then
    attending over the cache alone, up to the bf16 rounding of the stitched
    keys (one storage rounding: tolerance 1e-2 * max|V|)."""
    torch = torch_cuda
    import position_independent_kv_stitch_amd as pic
    rng = np.random.default_rng(9)
    wl = with_context(random_small(44, dtype="bf16", paged=True, n_requests=2, n_layers=1,
                                   max_len=250), rng)
    pk, pv = pool_values(wl, seed=1, device="cuda:0")
    ck = normal_values(wl.dst_shape(), "bf16", 2, "cuda:0")
    cv = normal_values(wl.dst_shape(), "bf16", 3, "cuda:0")
    q = normal_values((len(wl.requests), wl.n_heads * 4, wl.row_dim), "bf16", 4, "cuda:0")
    plan = pic.Plan.from_workload(wl)
    fused = pic.attend(plan, pk, pv, ck, cv, q, layer=0)
    pic.stitch(plan, pk, pv, ck, cv)
    empty = Workload(wl.name, wl.dtype, wl.n_layers, wl.n_heads, wl.row_dim, wl.rope_offset,
                     wl.rope_dim, wl.style, wl.theta, True, pool_tokens=wl.pool_tokens,
                     chunks=wl.chunks,
                     requests=[Request([], rq.page_table, rq.context_len) for rq in wl.requests],
                     page_size=wl.page_size, n_phys_pages=wl.n_phys_pages)
    plan2 = pic.Plan.from_workload(empty)
    two_step = pic.attend(plan2, pk, pv, ck, cv, q, layer=0)
    torch.cuda.synchronize()
    vmax = float(max(cv.float().abs().max(), pv.float().abs().max()))
    assert float((fused - two_step).abs().max()) <= 1e-2 * vmax
