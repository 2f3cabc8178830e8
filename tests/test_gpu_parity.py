"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Small cases are compared element by element in full; the full-size
workloads run in the launch configuration the benchmark times (one launch
over all layers) and are compared with the oracle on sampled layers (and,
for the batched RAG pool, sampled requests), plus properties checked on
every layer.  Tolerances: see parity_util (bit-exact outside rotated
elements; rotated fp32 within 1e-5 * max|k|, rotated bf16 within 1 ulp).
"""
import sys

import numpy as np
import pytest

import oracle
from parity_util import (check_stitch_case, compare_bits, compare_k, max_abs, to_host)
from pic_workloads import (Chunk, Entry, Request, Segment, Workload, config1, config2, config3,
                           config4, config5, pool_values, random_small, repeat_heavy,
                           sentinel_like, with_paged_pool)

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch_cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import position_independent_kv_stitch_amd  # noqa: F401  (fails loudly if not built)
    return torch


# ------------------------------------------------------------- small cases

CASES = [(seed, dt, style, paged, mla)
         for seed in range(3)
         for dt in ("f32", "bf16")
         for style in ("half", "interleaved")
         for paged in (False, True)
         for mla in (False, True)]


@pytest.mark.parametrize("seed,dt,style,paged,mla", CASES)
def test_random_small(torch_cuda, seed, dt, style, paged, mla):
    wl = random_small(seed, dtype=dt, style=style, paged=paged, mla=mla, n_requests=3,
                      n_layers=3, max_len=200)
    say(f"random_small seed={seed} {dt} {style} paged={paged} mla={mla}")
    check_stitch_case(wl, seed=seed)


@pytest.mark.parametrize("seed,dt,style,pool", [(0, "bf16", "half", False),
                                               (1, "f32", "interleaved", False),
                                               (2, "bf16", "interleaved", True),
                                               (3, "f32", "half", True)])
def test_repeated_chunks(torch_cuda, seed, dt, style, pool):
    """Chunks placed many times over many requests: the planner launches the
    placements of a chunk together, merged by source token and dealt to the
    XCD queues, which must change no output.  Everything against the oracle."""
    wl = repeat_heavy(seed, dtype=dt, style=style)
    if pool:
        wl = with_paged_pool(wl, page_size=16, seed=seed)
    say(f"repeat_heavy seed={seed} {dt} {style} pool={pool}: "
        f"{sum(len(r.entries) for r in wl.requests)} placements of {len(wl.chunks)} chunks")
    check_stitch_case(wl, seed=seed)


@pytest.mark.parametrize("seed,heads,dt,pool", [(10, 1, "bf16", False), (11, 4, "bf16", True),
                                                (12, 4, "f32", False), (13, 1, "f32", True),
                                                (14, 4, "bf16", False), (15, 8, "bf16", True)])
def test_tiles_grouped_per_workgroup(torch_cuda, seed, heads, dt, pool):
    """Narrow rows into paged destinations: one or two waves' steps cover a
    page of tokens, so a workgroup takes four or two tiles (ragged tiles, a
    last workgroup with spare waves); then chunks placed many times at 4 KV
    heads, whose source-ordered launch deals tiles to its queues two at a
    time.  Everything against the oracle."""
    from dataclasses import replace
    wl = random_small(seed, dtype=dt, paged=True, n_requests=3, n_layers=2, max_len=200,
                      dims=(heads, 128, 0, 128))
    if pool:
        wl = with_paged_pool(wl, page_size=8, seed=seed)
    say(f"grouped tiles seed={seed} {heads} heads {dt} pool={pool} page={wl.page_size}")
    check_stitch_case(wl, seed=seed)
    rh = replace(repeat_heavy(seed, dtype=dt, n_layers=1), n_heads=4)
    say(f"repeat_heavy at 4 heads, seed={seed}")
    check_stitch_case(rh, seed=seed)


SWEEP_HEADS = (1, 2, 4, 8)


@pytest.mark.parametrize("seed", range(100, 148))
def test_random_shape_sweep(torch_cuda, seed):
    """Seeded random shapes: 1-8 KV heads of 64 or 128 dims (rotary slice
    all or part of the row), or latent MLA rows; fp32 or bf16, both pairings;
    contiguous or paged destination, contiguous or paged pool.  Every element
    against the oracle."""
    rng = np.random.default_rng(seed)
    dt = str(rng.choice(["f32", "bf16"]))
    mla = bool(rng.random() < 0.2)
    style = "half" if mla else str(rng.choice(["half", "interleaved"]))
    dims = None
    if not mla:
        heads = int(rng.choice(SWEEP_HEADS))
        row = int(rng.choice([64, 128]))
        rdim = int(rng.choice([row, row // 2])) if style == "half" or dt == "f32" else row
        dims = (heads, row, row - rdim, rdim)
    wl = random_small(seed, dtype=dt, style=style, paged=bool(rng.random() < 0.6), mla=mla,
                      n_requests=int(rng.integers(1, 4)), n_layers=int(rng.integers(1, 4)),
                      max_len=int(rng.choice([40, 120, 300])), dims=dims)
    if rng.random() < 0.4:
        wl = with_paged_pool(wl, page_size=int(rng.choice([4, 8, 16])), seed=seed)
    say(f"sweep seed={seed}: {wl.n_heads} heads x {wl.row_dim} (rotary {wl.rope_offset}+"
        f"{wl.rope_dim}) {dt} {style} dst pages {wl.page_size} pool pages {wl.src_page_size}")
    check_stitch_case(wl, seed=seed)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("paged", [False, True])
def test_special_shifts(torch_cuda, dt, paged):
    """Shifts 0, +-1, +-65536 and large random ones, recompute_k in {0, 1,
    length}, ragged tails around the 64-token tile size."""
    for seed in range(4):
        wl = random_small(50 + seed, dtype=dt, paged=paged, n_requests=3, n_layers=2,
                          max_len=300, deltas=[0, 1, -1, 65536, -65536, 123457, -98765])
        say(f"special shifts seed={50 + seed} {dt} paged={paged}")
        check_stitch_case(wl, seed=seed)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_huge_shifts(torch_cuda, dt):
    """Shifts far beyond any context (chunks cached at base positions up to
    +-2^61 away): angles of up to 2^61 radians on plane 0, tables from the
    host's fp64 libm on both sides; copy mode on a paged destination and
    the in-place rotation."""
    torch = torch_cuda
    import position_independent_kv_stitch_amd as pic
    from pic_workloads import normal_values
    huge = [2 ** 40, -(2 ** 40), 2 ** 52 + 7, -(2 ** 52) - 3, 2 ** 61, -(2 ** 61) + 11]
    wl = random_small(77, dtype=dt, paged=True, n_requests=3, n_layers=2, max_len=200,
                      deltas=huge)
    say(f"huge shifts {dt}: copy mode")
    check_stitch_case(wl, seed=9)
    segs, at = [], 0
    for i, d in enumerate(huge):
        segs.append(Segment(at, 40 + 17 * i, d, i % 3))
        at += 40 + 17 * i
    ip = Workload("huge in place", dt, 2, 8, 128, 0, 128, "half", 1e6, False, inplace=True,
                  n_tokens=at, segments=segs)
    buf = normal_values(ip.buf_shape(), dt, 10, "cuda:0")
    before = to_host(buf)
    pic.rotate_workload(ip, buf)
    torch.cuda.synchronize()
    want = before.copy()
    assert oracle.rotate_inplace(ip, want) == "ok"
    stats = compare_k(to_host(buf), want, 0, 128, max_abs(before), what="huge in place")
    say(f"  in place: {stats}")


PAGED_POOL_CASES = [(seed, dt, paged, mla, ps)
                    for seed in range(2)
                    for dt in ("f32", "bf16")
                    for paged in (False, True)
                    for mla in (False, True)
                    for ps in (4, 16)]


@pytest.mark.parametrize("seed,dt,paged,mla,ps", PAGED_POOL_CASES)
def test_paged_pool_small(torch_cuda, seed, dt, paged, mla, ps):
    """Chunks read through their pool page tables (first tokens part-way into
    a page, pages in random order), into contiguous or paged destinations."""
    wl = with_paged_pool(random_small(20 + seed, dtype=dt, paged=paged, mla=mla, n_requests=3,
                                      n_layers=2, max_len=120),
                         page_size=ps, seed=seed, first_offsets=True, spare_pages=2)
    say(f"paged pool seed={seed} {dt} paged={paged} mla={mla} ps={ps}")
    check_stitch_case(wl, seed=seed)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_zero_shift_is_bit_exact(torch_cuda, dt):
    """Chunks placed where they were cached are copied bit for bit."""
    wl = random_small(7, dtype=dt, n_requests=2, n_layers=2, deltas=[0])
    stats = check_stitch_case(wl, seed=3)
    assert stats["bit_diffs"] == 0


def test_config1_full(torch_cuda):
    """Single layer, fp32, three chunks behind a 64-token prefix: every
    element of the destination compared with the oracle."""
    stats = check_stitch_case(config1(), seed=0)
    say("config1", stats)


def test_degenerate_tables(torch_cuda):
    """An empty request, fully masked entries and 1-token chunks."""
    wl = Workload("degenerate", "bf16", 2, 8, 128, 0, 128, "half", 5e5, True, pool_tokens=70,
                  chunks=[Chunk(0, 1), Chunk(1, 64), Chunk(65, 5, 3)], capacity=200,
                  requests=[Request([]),
                            Request([Entry(1, 0, 64, 64), Entry(0, 70, 1), Entry(2, 71, 5, 1)]),
                            Request([Entry(1, 100, 64, 0), Entry(1, 10, 65 - 2, 63)])])
    check_stitch_case(wl, seed=5)


# ---------------------------------------------------------- strided views

def test_strided_views(torch_cuda):
    """A head-major pool ([L][H][T][D] memory, viewed as [L][T][H][D]) stitched
    into a destination whose token rows are padded: the kernels follow the
    strides; the result equals the oracle's on dense copies."""
    torch = torch_cuda
    import position_independent_kv_stitch_amd as pic
    wl = random_small(11, dtype="bf16", n_requests=2, n_layers=2)
    pk, pv = pool_values(wl, seed=1, device="cuda:0")
    L, T, H, D = pk.shape
    pk_hm = pk.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)  # head-major memory
    pv_hm = pv.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    R, S = len(wl.requests), wl.capacity
    big_k = sentinel_like((L, R, S, H, D + 64), "bf16", "cuda:0")
    big_v = sentinel_like((L, R, S, H, D + 64), "bf16", "cuda:0")
    dk, dv = big_k[..., :D], big_v[..., :D]
    plan = pic.Plan.from_workload(wl)
    pic.stitch(plan, pk_hm, pv_hm, dk, dv)
    torch.cuda.synchronize()
    rk = to_host(sentinel_like(wl.dst_shape(), "bf16", "cpu"))
    rv = rk.copy()
    assert oracle.stitch(wl, to_host(pk), to_host(pv), rk, rv) == "ok"
    compare_k(to_host(dk), rk, 0, 128, max_abs(to_host(pk)))
    compare_bits(to_host(dv), rv, "V")
    # the padding beyond each head row was not touched
    pad = to_host(big_k[..., D:])
    assert np.all(pad == 0x7FC5)


def test_layer_subrange_and_repeat(torch_cuda):
    """A layer sub-range writes only those layers; running a plan twice gives
    the same bits."""
    torch = torch_cuda
    import position_independent_kv_stitch_amd as pic
    wl = random_small(12, dtype="f32", paged=True, n_requests=2, n_layers=4)
    pk, pv = pool_values(wl, seed=2, device="cuda:0")
    dk = sentinel_like(wl.dst_shape(), "f32", "cuda:0")
    dv = sentinel_like(wl.dst_shape(), "f32", "cuda:0")
    plan = pic.Plan.from_workload(wl)
    pic.stitch(plan, pk, pv, dk, dv, 1, 3)
    torch.cuda.synchronize()
    hk = to_host(dk)
    sentinel = to_host(sentinel_like(wl.dst_shape(), "f32", "cpu"))
    compare_bits(hk[[0, 3]], sentinel[[0, 3]], "layers outside the range")
    rk, rv = sentinel.copy(), sentinel.copy()
    assert oracle.stitch(wl, to_host(pk), to_host(pv), rk, rv, 1, 3) == "ok"
    compare_k(hk, rk, 0, 128, max_abs(to_host(pk)))
    first = hk.copy()
    pic.stitch(plan, pk, pv, dk, dv, 1, 3)
    torch.cuda.synchronize()
    compare_bits(to_host(dk), first, "second run")


def test_errors_write_nothing(torch_cuda):
    torch = torch_cuda
    import position_independent_kv_stitch_amd as pic
    wl = random_small(13, dtype="bf16", n_requests=1, n_layers=2)
    pk, pv = pool_values(wl, seed=2, device="cuda:0")
    dk = sentinel_like(wl.dst_shape(), "bf16", "cuda:0")
    dv = sentinel_like(wl.dst_shape(), "bf16", "cuda:0")
    plan = pic.Plan.from_workload(wl.with_layers(1))  # tensors hold 2 layers, the plan 1
    with pytest.raises(pic.PicError) as e:
        pic.stitch(plan, pk, pv, dk, dv, 0, 2)
    assert e.value.name == "invalid_arg"
    flat = torch.empty(pk.numel() + 8, dtype=pk.dtype, device="cuda:0")
    mis = flat[1:1 + pk.numel()].view(pk.shape)  # 2-byte offset: misaligned
    mis.copy_(pk)
    with pytest.raises(pic.PicError) as e:
        pic.stitch(plan, mis, pv, dk, dv, 0, 1)
    assert e.value.name == "align"
    torch.cuda.synchronize()
    assert np.all(to_host(dk) == 0x7FC5) and np.all(to_host(dv) == 0x7FC5)


# ------------------------------------------------------- full-size configs

def _layer_compare_stitch(wl, pk, pv, dk, dv, layers):
    for layer in layers:
        hk = to_host(pk[layer:layer + 1])
        hv = to_host(pv[layer:layer + 1]) if pv is not None else None
        rk = to_host(sentinel_like((1,) + tuple(wl.dst_shape()[1:]), wl.dtype, "cpu"))
        rv = rk.copy() if wl.has_v else None
        assert oracle.stitch(wl, hk, hv, rk, rv, layer, layer + 1, layer_base=layer) == "ok"
        stats = compare_k(to_host(dk[layer:layer + 1]), rk, wl.rope_offset, wl.rope_dim,
                          max_abs(hk), what=f"K layer {layer}")
        if wl.has_v:
            compare_bits(to_host(dv[layer:layer + 1]), rv, f"V layer {layer}")
        say(f"  layer {layer}: {stats}")


def _placement_rows(wl):
    """(flat destination row, flat pool row) of every written token, by the
    definition of the placement (test-side brute force)."""
    dst_rows, src_rows = [], []
    for r, req in enumerate(wl.requests):
        for e in req.entries:
            ch = wl.chunks[e.chunk_id]
            t = np.arange(e.recompute_k, e.length)
            pos = e.dst_offset + t
            if wl.page_size:
                rows = req.page_table[pos // wl.page_size].astype(np.int64) * wl.page_size + \
                    pos % wl.page_size
            else:
                rows = r * wl.capacity + pos
            dst_rows.append(rows)
            src_rows.append(ch.token_start + t)
    return np.concatenate(dst_rows), np.concatenate(src_rows)


def _all_layer_properties(torch, wl, pk, pv, dk, dv):
    """On every layer: V rows are the pool's bits, rows not written keep the
    sentinel (checked on the GPU with torch indexing)."""
    d_rows, s_rows = _placement_rows(wl)
    L = wl.n_layers
    rowlen = wl.n_heads * wl.row_dim
    dkf = dk.reshape(L, -1, rowlen)
    n_rows = dkf.shape[1]
    written = torch.zeros(n_rows, dtype=torch.bool, device=dk.device)
    di = torch.from_numpy(d_rows).to(dk.device)
    si = torch.from_numpy(s_rows).to(dk.device)
    written[di] = True
    assert int(written.sum()) == len(d_rows)  # no row written twice
    sent = sentinel_like((1,), wl.dtype, dk.device).view(torch.int16 if wl.dtype == "bf16"
                                                          else torch.int32)
    for layer in range(L):
        bits = dkf[layer].view(torch.int16 if wl.dtype == "bf16" else torch.int32)
        assert bool((bits[~written] == sent).all()), f"layer {layer}: unwritten K row changed"
        if pv is not None:
            dvf = dv.reshape(L, -1, rowlen)[layer]
            pvf = pv.reshape(L, -1, rowlen)[layer]
            assert torch.equal(dvf.index_select(0, di).view(torch.int16),
                               pvf.index_select(0, si).view(torch.int16)), f"V layer {layer}"


def test_config2_full(torch_cuda):
    """Llama-3-8B-shaped paged stitch, 32 layers in one launch."""
    torch = torch_cuda
    import position_independent_kv_stitch_amd as pic
    wl = config2()
    say("config2: generating inputs")
    pk, pv = pool_values(wl, seed=0, device="cuda:0")
    dk = sentinel_like(wl.dst_shape(), wl.dtype, "cuda:0")
    dv = sentinel_like(wl.dst_shape(), wl.dtype, "cuda:0")
    plan = pic.Plan.from_workload(wl)
    pic.stitch(plan, pk, pv, dk, dv)
    torch.cuda.synchronize()
    say("config2: oracle on sampled layers")
    _layer_compare_stitch(wl, pk, pv, dk, dv, [0, 13, 31])
    _all_layer_properties(torch, wl, pk, pv, dk, dv)


def test_config2_paged_pool_full(torch_cuda):
    """The Llama-3-8B-shaped stitch reading its chunks from a paged pool of
    16-token blocks in random order: 32 layers in one launch."""
    torch = torch_cuda
    import position_independent_kv_stitch_amd as pic
    wl = with_paged_pool(config2(), page_size=16, seed=1)
    say("config2 paged pool: generating inputs")
    pk, pv = pool_values(wl, seed=0, device="cuda:0")
    dk = sentinel_like(wl.dst_shape(), wl.dtype, "cuda:0")
    dv = sentinel_like(wl.dst_shape(), wl.dtype, "cuda:0")
    plan = pic.Plan.from_workload(wl)
    pic.stitch(plan, pk, pv, dk, dv)
    torch.cuda.synchronize()
    _layer_compare_stitch(wl, pk, pv, dk, dv, [0, 19, 31])


def test_config4_mla_full(torch_cuda):
    """DeepSeek-V3 MLA rows, 61 layers in one launch; the chunk at position 0
    keeps its first 32 tokens for recompute."""
    torch = torch_cuda
    import position_independent_kv_stitch_amd as pic
    wl = config4()
    say("config4: generating inputs")
    pk, _ = pool_values(wl, seed=0, device="cuda:0")
    dk = sentinel_like(wl.dst_shape(), wl.dtype, "cuda:0")
    plan = pic.Plan.from_workload(wl)
    pic.stitch(plan, pk, None, dk, None)
    torch.cuda.synchronize()
    _layer_compare_stitch(wl, pk, None, dk, None, [0, 29, 60])
    _all_layer_properties(torch, wl, pk, None, dk, None)
    # the content latent (dims 0..511) of every written row is the pool's, on every layer
    d_rows, s_rows = _placement_rows(wl)
    di = torch.from_numpy(d_rows).to(dk.device)
    si = torch.from_numpy(s_rows).to(dk.device)
    for layer in range(wl.n_layers):
        got = dk.reshape(wl.n_layers, -1, 576)[layer].index_select(0, di)[:, :512]
        src = pk.reshape(wl.n_layers, -1, 576)[layer].index_select(0, si)[:, :512]
        assert torch.equal(got.view(torch.int16), src.view(torch.int16)), layer


def test_config5_inplace_full(torch_cuda):
    """Qwen3-8B in-place rotation of a 131,072-token prompt, 36 layers, shifts
    up to +-65,536."""
    torch = torch_cuda
    import position_independent_kv_stitch_amd as pic
    from pic_workloads import normal_values
    wl = config5()
    say("config5: generating inputs")
    buf = normal_values(wl.buf_shape(), wl.dtype, 0, "cuda:0")
    sample = [0, 17, 35]
    before = {layer: to_host(buf[layer:layer + 1]) for layer in sample}
    keep = torch.zeros(wl.n_tokens, dtype=torch.bool, device="cuda:0")
    for s in wl.segments:
        keep[s.token_start:s.token_start + s.recompute_k] = True
    kept = buf[:, keep].clone()
    pic.rotate_workload(wl, buf)
    torch.cuda.synchronize()
    assert torch.equal(buf[:, keep].view(torch.int16), kept.view(torch.int16))
    for layer in sample:
        ref = before[layer].copy()
        assert oracle.rotate_inplace(wl, ref, layer, layer + 1, layer_base=layer) == "ok"
        stats = compare_k(to_host(buf[layer:layer + 1]), ref, 0, 128, max_abs(before[layer]),
                          what=f"in-place layer {layer}")
        say(f"  layer {layer}: {stats}")


def _subproblem(wl, req_ids):
    """The requests `req_ids` of a paged workload as a compact problem: only
    their chunks in a packed pool, their pages renumbered 0..n-1.  Returns
    (sub-workload, pool token index per packed token, physical page per
    packed page)."""
    chunk_ids = sorted({e.chunk_id for r in req_ids for e in wl.requests[r].entries})
    new_id, chunks, src_tok, at = {}, [], [], 0
    for c in chunk_ids:
        ch = wl.chunks[c]
        new_id[c] = len(chunks)
        chunks.append(Chunk(at, ch.length, ch.base_pos))
        src_tok.append(np.arange(ch.token_start, ch.token_start + ch.length))
        at += ch.length
    pages = np.concatenate([wl.requests[r].page_table for r in req_ids])
    requests, base = [], 0
    for r in req_ids:
        rq = wl.requests[r]
        n = len(rq.page_table)
        requests.append(Request([Entry(new_id[e.chunk_id], e.dst_offset, e.length,
                                       e.recompute_k) for e in rq.entries],
                                np.arange(base, base + n, dtype=np.int32)))
        base += n
    sub = Workload(wl.name + " (sample)", wl.dtype, wl.n_layers, wl.n_heads, wl.row_dim,
                   wl.rope_offset, wl.rope_dim, wl.style, wl.theta, wl.has_v, pool_tokens=at,
                   chunks=chunks, requests=requests, page_size=wl.page_size,
                   n_phys_pages=len(pages))
    return sub, np.concatenate(src_tok), pages


@pytest.mark.parametrize("tp", [1, 2, 4])
def test_config3_full_in_layer_groups(torch_cuda, tp):
    """Batched RAG: 64 requests over a 256-chunk pool, all 32 layers, in the
    benchmark's launch configuration: the pool holds every layer and each
    launch stitches one layer group of all requests into a destination
    holding that group, the group as large as the free HBM allows (all 32
    layers in one launch on a 288 GiB GPU).  Every group: on every layer,
    unwritten rows keep the sentinel, no row is written twice and every
    written V row is its pool row; 4 sampled requests on 2 layers are
    compared with the oracle.  tp = 4: one GPU's share under 4-way tensor
    parallelism (2 of the 8 KV heads), the shape its stitch has there; tp = 2
    the share under 2-way parallelism (two waves per tile instead of one)."""
    torch = torch_cuda
    import position_independent_kv_stitch_amd as pic
    from pic_workloads import layers_per_launch, tp_share
    wl = tp_share(config3(), tp)
    torch.cuda.empty_cache()
    group = layers_per_launch(wl, torch.cuda.mem_get_info()[0])
    assert group > 0, "HBM too small for the batched-RAG pool"
    say(f"config3 (tp share 1/{tp}): {group} layers per launch")
    gw = wl.with_layers(group)
    say("config3: generating the 32-layer pool")
    pk, pv = pool_values(wl, seed=0, device="cuda:0")
    plan = pic.Plan.from_workload(wl)
    rng = np.random.default_rng(0)
    dk = sentinel_like(gw.dst_shape(), wl.dtype, "cuda:0")
    dv = sentinel_like(gw.dst_shape(), wl.dtype, "cuda:0")
    for g in range(wl.n_layers // group):
        lo = g * group
        say(f"config3: layer group {g} (layers {lo}..{lo + group - 1})")
        if g:
            sent = sentinel_like((1,), wl.dtype, "cuda:0")
            dk.copy_(sent.expand_as(dk))
            dv.copy_(sent.expand_as(dv))
        gk, gv = pk[lo:lo + group], pv[lo:lo + group]
        pic.stitch(plan, gk, gv, dk, dv, 0, group)
        torch.cuda.synchronize()
        _all_layer_properties(torch, gw, gk, gv, dk, dv)
        for layer in sorted(rng.choice(group, size=2, replace=False).tolist()):
            req_ids = sorted(rng.choice(len(wl.requests), size=4, replace=False).tolist())
            sub, src_tok, pages = _subproblem(gw, req_ids)
            st = torch.from_numpy(src_tok).to("cuda:0")
            pg = torch.from_numpy(pages.astype(np.int64)).to("cuda:0")
            hk = to_host(gk[layer:layer + 1].index_select(1, st))
            hv = to_host(gv[layer:layer + 1].index_select(1, st))
            rk = to_host(sentinel_like((1,) + tuple(sub.dst_shape()[1:]), wl.dtype, "cpu"))
            rv = rk.copy()
            assert oracle.stitch(sub, hk, hv, rk, rv, layer, layer + 1, layer_base=layer) == "ok"
            stats = compare_k(to_host(dk[layer:layer + 1].index_select(1, pg)), rk, 0, 128,
                              max_abs(hk), what=f"K layer {lo + layer}")
            compare_bits(to_host(dv[layer:layer + 1].index_select(1, pg)), rv,
                         f"V layer {lo + layer}")
            say(f"  layer {lo + layer}, requests {req_ids}: {stats}")
    plan.destroy()
    del pk, pv, dk, dv
    torch.cuda.empty_cache()


def test_inplace_back_to_back_calls(torch_cuda):
    """Six pic_rotate_inplace calls enqueued without waiting, on separate
    buffers with different segment sets (the per-call staging slots are
    reused while earlier calls are still queued), each against the oracle."""
    torch = torch_cuda
    import position_independent_kv_stitch_amd as pic
    from pic_workloads import Segment, Workload, normal_values
    rng = np.random.default_rng(90)
    cases = []
    for i in range(6):
        n_seg = 2 + 3 * i
        lens = [int(x) for x in rng.integers(1, 400, size=n_seg)]
        segs, at = [], 0
        for n in lens:
            segs.append(Segment(at, n, int(rng.integers(-65536, 65537)), int(rng.integers(0, min(n, 20) + 1))))
            at += n + int(rng.integers(0, 5))
        wl = Workload(f"in-place back to back {i}", "bf16", 2, 8, 128, 0, 128, "half", 1e6, False,
                      inplace=True, n_tokens=at, segments=segs)
        buf = normal_values(wl.buf_shape(), "bf16", 100 + i, "cuda:0")
        cases.append((wl, buf, to_host(buf)))
    torch.cuda.synchronize()
    for wl, buf, _ in cases:
        pic.rotate_workload(wl, buf)
    torch.cuda.synchronize()
    for i, (wl, buf, ref) in enumerate(cases):
        want = ref.copy()
        assert oracle.rotate_inplace(wl, want) == "ok"
        stats = compare_k(to_host(buf), want, 0, 128, max_abs(ref), what=f"call {i}")
        say(f"  call {i}: {len(wl.segments)} segments, {stats}")
