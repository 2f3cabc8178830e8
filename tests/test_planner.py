"""Host logic of the library (no GPU): the planner's verdict on valid and
invalid placement tables equals the oracle's, its counts and ranges equal
the definitions, and in-place segment validation matches the oracle."""
import copy
import ctypes as C

import numpy as np
import pytest

import oracle
import position_independent_kv_stitch_amd as pic
from position_independent_kv_stitch_amd import _binding as B
from pic_workloads import (CONFIGS, Chunk, Entry, Request, Segment, Workload, config2,
                           config3, decode_batch, layers_per_launch, random_small,
                           tp_share, with_paged_pool)

ORACLE_TO_LIB = {"ok": "ok", "bad_arg": "invalid_arg", "range": "range", "overlap": "overlap"}


def plan_status(wl):
    try:
        p = pic.Plan.from_workload(wl)
    except pic.PicError as e:
        return e.name
    p.destroy()
    return "ok"


def pool_fits(wl):
    return all(c.token_start + c.length <= wl.pool_tokens for c in wl.chunks)


@pytest.mark.parametrize("seed", range(40))
def test_valid_random_problems_agree(seed):
    wl = random_small(seed, dtype=["f32", "bf16"][seed % 2], paged=seed % 3 == 0,
                      mla=seed % 5 == 4, n_requests=1 + seed % 4,
                      style=["half", "interleaved"][seed % 2])
    assert oracle.validate_stitch(wl) == "ok"
    assert plan_status(wl) == "ok"


def _mutations(wl, rng):
    """One random defect (or a harmless change) applied to a copy of wl."""
    w = copy.deepcopy(wl)
    r = int(rng.integers(0, len(w.requests)))
    req = w.requests[r]
    if not req.entries:
        return w
    j = int(rng.integers(0, len(req.entries)))
    e = req.entries[j]
    kind = int(rng.integers(0, 17))
    if kind == 0:
        req.entries[j] = Entry(int(rng.choice([-1, len(w.chunks), 10 ** 6])), e.dst_offset,
                               e.length, e.recompute_k)
    elif kind == 1:
        req.entries[j] = Entry(e.chunk_id, e.dst_offset, int(rng.choice([0, -3])), 0)
    elif kind == 2:
        req.entries[j] = Entry(e.chunk_id, e.dst_offset, w.chunks[e.chunk_id].length + 1,
                               e.recompute_k)
    elif kind == 3:
        req.entries[j] = Entry(e.chunk_id, e.dst_offset, e.length,
                               int(rng.choice([-1, e.length + 1])))
    elif kind == 4:
        req.entries[j] = Entry(e.chunk_id, -int(rng.integers(1, 5)), e.length, e.recompute_k)
    elif kind == 5:
        span = len(req.page_table) * w.page_size if w.page_size else w.capacity
        req.entries[j] = Entry(e.chunk_id, span - e.length + int(rng.integers(1, 4)), e.length,
                               e.recompute_k)
    elif kind == 6 and len(req.entries) > 1:
        o = req.entries[(j + 1) % len(req.entries)]
        shift = int(rng.integers(0, max(1, o.length)))
        req.entries[j] = Entry(e.chunk_id, o.dst_offset + shift, min(e.length, 3),
                               e.recompute_k if e.recompute_k <= 3 else 0)
    elif kind == 7 and w.page_size:
        i = int(rng.integers(0, len(req.page_table)))
        req.page_table[i] = int(rng.choice([-1, w.n_phys_pages, w.n_phys_pages + 9]))
    elif kind == 8 and w.page_size and len(w.requests) > 1:
        other = w.requests[(r + 1) % len(w.requests)]
        i = int(rng.integers(0, len(req.page_table)))
        req.page_table[i] = other.page_table[int(rng.integers(0, len(other.page_table)))]
    elif kind == 9:
        c = int(rng.integers(0, len(w.chunks)))
        ch = w.chunks[c]
        w.chunks[c] = Chunk(int(rng.choice([-1, ch.token_start])), int(rng.choice([0, ch.length])),
                            ch.base_pos, ch.page_table)
    elif kind == 10:
        w.rope_dim = int(rng.choice([0, 7, w.row_dim + 8]))
    elif kind == 11:
        w.n_heads = 0
    elif kind == 12:
        w.theta = float(rng.choice([0.0, -1.0]))
    elif kind == 13:
        w.rope_offset = w.row_dim  # slice outside the row
    elif kind == 15 and w.src_page_size:
        c = e.chunk_id
        if 0 <= c < len(w.chunks):
            ch = w.chunks[c]
            pt = ch.page_table.copy()
            choice = int(rng.integers(0, 3))
            if choice == 0:
                pt[int(rng.integers(0, len(pt)))] = int(rng.choice([-1, w.src_n_pages]))
            elif choice == 1:
                pt = pt[:-1]  # one page short
            w.chunks[c] = Chunk(ch.token_start + (choice == 2) * w.src_page_size, ch.length,
                                ch.base_pos, pt)
    elif kind == 14:  # harmless: duplicate an entry's chunk id into a new tail entry
        last = max(e.dst_offset + e.length for e in req.entries)
        req.entries.append(Entry(e.chunk_id, last, 1, 0))
        if w.page_size:
            need = -(-(last + 1) // w.page_size)
            if need > len(req.page_table):
                return wl
        elif last + 1 > w.capacity:
            return wl
    return w


@pytest.mark.parametrize("seed", range(300))
def test_invalid_problems_agree_with_oracle(seed):
    rng = np.random.default_rng(1000 + seed)
    base = random_small(seed, dtype="bf16", paged=seed % 2 == 0, mla=seed % 7 == 3,
                        n_requests=1 + seed % 3)
    if seed % 3 == 1:
        base = with_paged_pool(base, page_size=[4, 16][seed % 2], seed=seed,
                               first_offsets=True, spare_pages=seed % 4)
    w = _mutations(base, rng)
    if seed % 5 == 0:
        w = _mutations(w, rng)  # two defects: both sides must report the first one
    want = oracle.validate_stitch(w)
    if want == "ok" and not w.src_page_size and not pool_fits(w):
        pytest.skip("defect only visible against the pool tensor")
    got = plan_status(w)
    if got == "align" and want == "ok":
        pytest.skip("shape the kernels cannot vectorise")
    assert got == ORACLE_TO_LIB[want]


def test_alignment_limits():
    wl = random_small(1, dtype="bf16")
    wl.rope_dim, wl.row_dim = 96, 128  # 6 units of 16 bytes: not a power of two
    assert oracle.validate_stitch(wl) == "ok"
    assert plan_status(wl) == "align"
    wl.rope_dim, wl.rope_offset = 64, 4  # rotary slice starts mid-vector
    assert plan_status(wl) == "align"


@pytest.mark.parametrize("cfg", [1, 2, 4])
def test_info_and_ranges_match_definitions(cfg):
    wl = CONFIGS[cfg]()
    p = pic.Plan.from_workload(wl)
    ents = [e for r in wl.requests for e in r.entries]
    written = sum(e.length - e.recompute_k for e in ents)
    assert p.info["tokens_written"] == written
    assert p.info["tokens_masked"] == sum(e.recompute_k for e in ents)
    row_bytes = wl.n_heads * wl.row_dim * wl.esize * (2 if wl.has_v else 1)
    assert p.info["bytes_read_per_layer"] == written * row_bytes
    assert p.info["bytes_written_per_layer"] == written * row_bytes
    tiles = 0  # tiles of at most tile_tokens tokens that never cross a destination page
    tt = p.info["tile_tokens"]
    assert tt >= 1
    for e in ents:
        pos, end = e.dst_offset + e.recompute_k, e.dst_offset + e.length
        while pos < end:
            n = min(tt, end - pos)
            if wl.page_size:
                n = min(n, wl.page_size - pos % wl.page_size)
            pos += n
            tiles += 1
    assert p.info["n_tiles"] == tiles
    assert p.info["pool_tokens_required"] == max(c.token_start + c.length for c in wl.chunks)
    bounds, rec = p.ranges()
    want_b = [(r, e.dst_offset, e.dst_offset + e.length)
              for r, rq in enumerate(wl.requests) for e in rq.entries]
    assert [tuple(x) for x in bounds] == want_b
    got_rec = [tuple(x) for x in rec if x[2] > x[1]]
    assert got_rec == oracle.recompute_ranges(wl)
    p.destroy()
    with pytest.raises(pic.PicError):
        p.ranges()


def test_config_byte_totals():
    """Per-step algorithmic bytes of the Llama-3-8B paged workload: 16,128
    stitched tokens x 32 layers x 8 KiB (K and V read and written)."""
    wl = config2()
    p = pic.Plan.from_workload(wl)
    total = (p.info["bytes_read_per_layer"] + p.info["bytes_written_per_layer"]) * wl.n_layers
    assert p.info["tokens_written"] == 8 * (2048 - 32)
    assert total == 16128 * 32 * 8192


def test_batched_rag_plan_scales():
    wl = config3()
    p = pic.Plan.from_workload(wl)
    assert p.info["n_requests"] == 64
    assert oracle.validate_stitch(wl) == "ok"
    # every physical page is written by exactly one request (global permutation)
    pages = np.concatenate([r.page_table for r in wl.requests])
    assert len(np.unique(pages)) == len(pages) == wl.n_phys_pages



def test_tensor_parallel_share():
    """One GPU's share under tensor parallelism keeps every chunk, request and
    page and divides the KV heads; the plan's bytes divide with them and
    every token is still written once."""
    wl = config3()
    share = tp_share(wl, 4)
    assert share.n_heads == 2 and wl.n_heads == 8
    assert share.requests is wl.requests and share.chunks is wl.chunks
    assert share.pool_shape() == (32, wl.pool_tokens, 2, 128)
    assert share.dst_shape() == (32, wl.n_phys_pages, 16, 2, 128)
    full, part = pic.Plan.from_workload(wl), pic.Plan.from_workload(share)
    assert part.info["tokens_written"] == full.info["tokens_written"]
    for key in ("bytes_read_per_layer", "bytes_written_per_layer"):
        assert 4 * part.info[key] == full.info[key]
    assert oracle.validate_stitch(share) == "ok"
    full.destroy()
    part.destroy()
    for tp in (3, 16, 0):
        with pytest.raises(ValueError):
            tp_share(wl, tp)


def test_batched_rag_layers_per_launch():
    """The layer group of the batched-RAG stitch: the pool (32 layers of K
    and V over 562,245 tokens of 8 x 128 bf16 rows) stays resident and the
    destination of g layers (96,341 pages of 16 tokens for K and V)
    must fit beside it with 6 GiB to spare, g a divisor of 32."""
    wl = config3()
    row = 2 * 8 * 128 * 2
    pool = 32 * wl.pool_tokens * row
    dst = wl.n_phys_pages * 16 * row
    gib = 1 << 30
    assert layers_per_launch(wl, pool + 32 * dst + 6 * gib) == 32  # all layers, one launch
    assert layers_per_launch(wl, pool + 32 * dst + 6 * gib - 1) == 16
    assert layers_per_launch(wl, pool + 8 * dst + 6 * gib) == 8
    assert layers_per_launch(wl, pool + 7 * dst + 6 * gib) == 4  # 7 does not divide 32
    assert layers_per_launch(wl, pool + dst + 6 * gib - 1) == 0
    # a 288 GiB GPU with the runtime's share taken holds all 32 layers
    assert layers_per_launch(wl, int(286.6 * gib)) == 32


# ------------------------------------------------------------- in-place

def _inplace_status(wl):
    lib = B.load_library()
    shape, rope, keep = B._shape_and_rope(wl.dtype, wl.n_layers, wl.n_heads, wl.row_dim,
                                          wl.rope_offset, wl.rope_dim, wl.style, wl.theta,
                                          False, None)
    segs = (B.SegmentC * max(1, len(wl.segments)))()
    for i, s in enumerate(wl.segments):
        segs[i] = B.SegmentC(s.token_start, s.delta, s.length, s.recompute_k)
    view = B.KvView(None, None, 0, 0, 0, 0, 0)
    st = lib.pic_rotate_inplace(C.byref(shape), C.byref(rope), C.byref(view), wl.n_tokens, segs,
                                len(wl.segments), 0, wl.n_layers, None)
    return B.STATUS_NAMES[st]


@pytest.mark.parametrize("segs,want", [
    ([Segment(0, 5, 1), Segment(4, 3, 1)], "overlap"),
    ([Segment(0, 5, 1), Segment(5, 6, 1)], "range"),
    ([Segment(-1, 5, 1)], "range"),
    ([Segment(0, 0, 1)], "range"),
    ([Segment(0, 5, 1, 6)], "range"),
    ([Segment(0, 5, 1, -1)], "range"),
])
def test_inplace_validation_agrees(segs, want):
    wl = Workload("ip", "bf16", 2, 8, 128, 0, 128, "half", 1e6, False, inplace=True,
                  n_tokens=10, segments=segs)
    assert oracle.validate_inplace(wl) == want
    assert _inplace_status(wl) == want


def test_inplace_valid_reaches_the_view_check():
    """A valid segment table passes the planner; the NULL view is then refused
    (invalid_arg) before any device call."""
    wl = Workload("ip", "bf16", 2, 8, 128, 0, 128, "half", 1e6, False, inplace=True,
                  n_tokens=10, segments=[Segment(0, 5, 3), Segment(5, 5, -2, 1)])
    assert oracle.validate_inplace(wl) == "ok"
    assert _inplace_status(wl) == "invalid_arg"


@pytest.mark.parametrize("seed", range(20))
def test_paged_pool_plans(seed):
    """Paged pools: tiles never cross a pool page or a destination page, and
    the planner agrees with the oracle on valid tables."""
    wl = with_paged_pool(random_small(seed, dtype="bf16", paged=seed % 2 == 0, n_requests=2),
                         page_size=[4, 8, 16][seed % 3], seed=seed, first_offsets=True)
    assert oracle.validate_stitch(wl) == "ok"
    p = pic.Plan.from_workload(wl)
    ents = [e for r in wl.requests for e in r.entries]
    tt = p.info["tile_tokens"]
    tiles = 0
    for e in ents:
        ch = wl.chunks[e.chunk_id]
        t = e.recompute_k
        while t < e.length:
            n = min(tt, e.length - t)
            if wl.page_size:
                n = min(n, wl.page_size - (e.dst_offset + t) % wl.page_size)
            n = min(n, wl.src_page_size - (ch.token_start + t) % wl.src_page_size)
            t += n
            tiles += 1
    assert p.info["n_tiles"] == tiles
    assert p.info["pool_tokens_required"] == wl.src_n_pages * wl.src_page_size


def test_attention_map_counts_and_validation():
    """The pic_attend map covers every context position once, in blocks of at
    most 256 positions, shortened (to 128, then 64) while fewer than 1024
    (block, KV head) items would result; a context beyond the request's span
    is refused."""
    wl = config2()
    wl.requests[0].context_len = 128 + 8 * 2048
    p = pic.Plan.from_workload(wl)
    assert p.info["context_tokens"] == 16512
    # 65 blocks of 256 x 8 heads = 520 < 1024 -> 128-position blocks
    assert p.info["attend_block_tokens"] == 128
    assert p.info["attend_blocks"] >= -(-16512 // 128)
    wide = decode_batch(n_requests=16)
    assert pic.Plan.from_workload(wide).info["attend_block_tokens"] == 256
    small = random_small(3, n_requests=1)
    assert pic.Plan.from_workload(small).info["attend_block_tokens"] == 64
    wl.requests[0].context_len = 16513
    assert plan_status(wl) == "range"
    wl.requests[0].context_len = 0  # default: up to the last entry
    p = pic.Plan.from_workload(wl)
    assert p.info["context_tokens"] == max(e.dst_offset + e.length for e in wl.requests[0].entries)


def test_attend_refuses_unmapped_context_pages():
    """A prefix page no stitch writes may be unmapped for pic_stitch, but
    pic_attend reads it: refused before any device work."""
    lib = B.load_library()
    wl = config2()
    wl.requests[0].page_table = wl.requests[0].page_table.copy()
    wl.requests[0].page_table[0] = -1  # the 128-token prefix's first page
    p = pic.Plan.from_workload(wl)  # the stitch never touches it
    view = B.KvView(16, 16, 0, 1024, 128, 16384, 0)
    args = B.AttendArgs(16, 4096, 128, 16, 4096, 128, 32, 0, 0.1, 0, 0.0, 0)
    st = lib.pic_attend(p.handle, C.byref(view), C.byref(view), C.byref(args), None)
    assert B.STATUS_NAMES[st] == "range" and b"context page" in lib.pic_last_error()


def test_attend_refuses_rows_too_narrow_for_the_group():
    """Query heads per KV head are reduced over the lanes of one row: a
    16-dim bf16 row (2 lanes) cannot carry 8 query heads."""
    lib = B.load_library()
    wl = random_small(2, dtype="bf16", dims=(2, 16, 0, 16))
    p = pic.Plan.from_workload(wl)
    view = B.KvView(16, 16, 0, 32, 16, 0, 0)
    args = B.AttendArgs(16, 256, 16, 16, 256, 16, 16, 0, 0.25, 0, 0.0, 0)
    st = lib.pic_attend(p.handle, C.byref(view), C.byref(view), C.byref(args), None)
    assert B.STATUS_NAMES[st] == "align" and b"row_dim" in lib.pic_last_error()


@pytest.mark.parametrize("base,dst,want", [
    (2 ** 62, 5, "ok"),                        # |base_pos| up to 2^62
    (-(2 ** 62), 5, "ok"),
    (2 ** 62 + 1, 5, "range"),                 # past it delta could overflow int64
    (-(2 ** 62) - 1, 5, "range"),
    (0, 2 ** 31 - 1 - 10, "ok"),               # the last positions below 2^31
    (0, 2 ** 31 - 10, "range"),                # a position reaches 2^31
])
def test_extreme_bases_and_positions(base, dst, want):
    """The library and the oracle agree at the bounds of base_pos and of
    logical positions (contiguous destination wide enough for both)."""
    wl = Workload("edge", "bf16", 1, 2, 128, 0, 128, "half", 5e5, True, pool_tokens=20,
                  chunks=[Chunk(0, 10, base)], capacity=2 ** 31 + 64,
                  requests=[Request([Entry(0, dst, 10, 2)])])
    assert oracle.validate_stitch(wl) == want
    assert ORACLE_TO_LIB[want] == plan_status(wl)
