"""Pins of the fp64 oracle to what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: values
printed on the pages (tests/golden), closed forms of plane rotations, the
group law and orthogonality of RoPE, an independent library (numpy complex
arithmetic, torch's bf16 conversion), brute-force enumeration, and
brute-force attention on tiny inputs.  A dropped term, a wrong sign, a
swapped pair member or a wrong frequency index fails at least one of them.
"""
import copy
import json
import math
import os

import numpy as np
import pytest

import oracle
from pic_workloads import (Chunk, Entry, Request, Segment, Workload, random_small,
                           with_paged_pool)

SENT_F64 = np.float64(-12345.5)


def gqa(rope_dim=8, n_heads=2, style="half", theta=10000.0, row_dim=None, rope_offset=0,
        has_v=True, n_layers=1, inv=None):
    return Workload("pin", "f64", n_layers, n_heads, row_dim or rope_dim, rope_offset,
                    rope_dim, style, theta, has_v, inv_freq=inv)


def place(wl, pool_k, pool_v, chunks, entries, capacity, dtype="f64", page_size=0,
          page_table=None, n_phys=0, fill=None):
    """Stitch one request with the oracle; returns (status, dst_k, dst_v)."""
    wl.chunks = chunks
    wl.pool_tokens = pool_k.shape[1]
    wl.requests = [Request(entries, page_table)]
    wl.capacity = capacity
    wl.page_size = page_size
    wl.n_phys_pages = n_phys
    shape = wl.dst_shape() if page_size else (wl.n_layers, 1, capacity, wl.n_heads, wl.row_dim)
    npdt = oracle.ref.NUMPY_STORAGE[dtype]
    f = SENT_F64 if fill is None else fill
    dk = np.full(shape, f, dtype=npdt)
    dv = np.full(shape, f, dtype=npdt) if wl.has_v else None
    st = oracle.stitch(wl, pool_k, pool_v, dk, dv, dtype=dtype)
    return st, dk, dv


def rope_at(raw, positions, wl):
    """Keys of `raw` [1][T][H][D] rotated to the given absolute positions, one
    in-place segment of length 1 per token (the oracle's own rotation)."""
    buf = raw.copy()
    w = Workload("seg", "f64", 1, wl.n_heads, wl.row_dim, wl.rope_offset, wl.rope_dim,
                 wl.style, wl.theta, False, inplace=True, n_tokens=raw.shape[1],
                 inv_freq=wl.inv_freq,
                 segments=[Segment(t, 1, int(p), 0) for t, p in enumerate(positions)])
    assert oracle.rotate_inplace(w, buf, dtype="f64") == "ok"
    return buf


def pair_index(style, rope_dim, i):
    """The two members of plane i, as the pages pair coordinates: interleaved
    (2i, 2i+1) as written in the RoPE section; half (i, i + d/2) as in
    rotate-half implementations."""
    return (2 * i, 2 * i + 1) if style == "interleaved" else (i, i + rope_dim // 2)


# --------------------------------------------------------------- rounding

def test_bf16_rounding_matches_torch_on_float_values():
    """For doubles that are exact binary32 values, one RNE to bf16 must equal
    torch's float32 -> bfloat16 conversion (an independent library)."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(200000).astype(np.float32),
                        (rng.standard_normal(20000) * 1e-39).astype(np.float32),
                        (rng.standard_normal(20000) * 1e37).astype(np.float32)])
    # exact ties: bf16 value plus half a bf16 quantum
    base = (rng.integers(0, 0x7F00, 5000).astype(np.uint32) << 16)
    ties = (base | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, -ties])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.round_bf16(x.astype(np.float64))
    assert np.array_equal(got, want)


def test_bf16_rounding_brute_force_on_doubles():
    """Doubles between bf16 neighbours round to the nearer one, ties to the even
    pattern: checked against an enumeration of every finite positive bf16."""
    pats = np.arange(0, 0x7F80, dtype=np.uint32)
    vals = (pats << 16).view(np.float32).astype(np.float64)
    rng = np.random.default_rng(2)
    idx = rng.integers(1, len(vals) - 1, 30000)
    lo, hi = vals[idx], vals[idx + 1]
    frac = rng.random(30000)
    frac[:300] = 0.5  # exact midpoints in double
    x = lo + (hi - lo) * frac
    got = oracle.round_bf16(x)
    d_lo, d_hi = x - lo, hi - x
    want = np.where(d_lo < d_hi, idx, np.where(d_hi < d_lo, idx + 1,
                                               np.where(idx % 2 == 0, idx, idx + 1)))
    assert np.array_equal(got, want.astype(np.uint16))
    # sign symmetry and specials
    assert np.array_equal(oracle.round_bf16(-x), got | 0x8000)
    assert oracle.round_bf16([0.0])[0] == 0 and oracle.round_bf16([-0.0])[0] == 0x8000
    assert oracle.round_bf16([3.5e38])[0] == 0x7F80  # beyond bf16 range
    assert oracle.round_bf16([2.0 ** -134])[0] == 0  # half the subnormal quantum: tie to 0
    assert oracle.round_bf16([1.5 * 2.0 ** -133])[0] == 2  # tie to even


# ------------------------------------------------------------- frequencies

def test_plane_frequencies_page_values(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "rope_frequencies.json")))
    for case in g["cases"]:
        got = oracle.inv_freq(case["base"], case["d"])
        assert np.allclose(got, case["theta"], rtol=1e-15, atol=0)
    # theta_0 = b^0 = 1 exactly, for any base
    for b in (10000.0, 500000.0, 1e6):
        assert oracle.inv_freq(b, 128)[0] == 1.0


def test_caller_table_equals_formula():
    """Giving theta_i as a table reproduces the formula bit for bit."""
    rng = np.random.default_rng(3)
    wl = gqa(rope_dim=16, theta=500000.0)
    pool = rng.standard_normal((1, 5, 2, 16))
    chunks = [Chunk(0, 5)]
    a = place(wl, pool, pool.copy(), chunks, [Entry(0, 9, 5)], 20)[1]
    wl2 = gqa(rope_dim=16, theta=500000.0, inv=oracle.inv_freq(500000.0, 16))
    b = place(wl2, pool, pool.copy(), chunks, [Entry(0, 9, 5)], 20)[1]
    assert np.array_equal(a, b)


# ----------------------------------------------------------- plane rotation

@pytest.mark.parametrize("style", ["half", "interleaved"])
def test_quarter_and_half_turns(style):
    """With theta_i = pi/2 a shift of 1 is a quarter turn: by the page's matrix
    [[cos, -sin], [sin, cos]] the pair (x, y) becomes (-y, x); with pi it
    becomes (-x, -y)."""
    D = 8
    inv = np.array([math.pi / 2, math.pi, math.pi / 2, math.pi])
    wl = gqa(rope_dim=D, n_heads=1, style=style, inv=inv)
    rng = np.random.default_rng(4)
    pool = rng.standard_normal((1, 3, 1, D))
    st, dk, _ = place(wl, pool, pool.copy(), [Chunk(0, 3)], [Entry(0, 1, 3)], 4)
    assert st == "ok"
    out = dk[0, 0, 1:4, 0]
    for i in range(D // 2):
        a, b = pair_index(style, D, i)
        x, y = pool[0, :, 0, a], pool[0, :, 0, b]
        if inv[i] == math.pi / 2:
            want_a, want_b = -y, x
        else:
            want_a, want_b = -x, -y
        assert np.allclose(out[:, a], want_a, atol=1e-15)
        assert np.allclose(out[:, b], want_b, atol=1e-15)


@pytest.mark.parametrize("style", ["half", "interleaved"])
def test_rotation_is_complex_multiplication(style):
    """Each plane rotated by phi equals (x + iy) * exp(i phi) in numpy complex
    arithmetic, with phi = delta * theta_i and theta_i = 10^-i (b = 1e4, d = 8)."""
    D, H = 8, 3
    wl = gqa(rope_dim=D, n_heads=H, style=style)
    rng = np.random.default_rng(5)
    pool = rng.standard_normal((1, 6, H, D))
    theta = np.array([1.0, 0.1, 0.01, 0.001])
    for delta in (1, -1, 7, 123456, -65536):
        st, dk, _ = place(wl, pool, pool.copy(), [Chunk(0, 6, 70000)],
                          [Entry(0, 70000 + delta, 6)], 70000 + delta + 6)
        assert st == "ok"
        out = dk[0, 0, 70000 + delta:70000 + delta + 6]
        for i in range(D // 2):
            a, b = pair_index(style, D, i)
            z = (pool[0, :, :, a] + 1j * pool[0, :, :, b]) * np.exp(1j * delta * theta[i])
            tol = 1e-15 * (1 + abs(delta * theta[i]))
            assert np.allclose(out[:, :, a], z.real, atol=tol, rtol=0)
            assert np.allclose(out[:, :, b], z.imag, atol=tol, rtol=0)


def test_pair_zero_turns_by_delta_radians():
    """theta_0 = 1, so plane 0 turns by exactly delta radians (libm cos/sin)."""
    wl = gqa(rope_dim=128, n_heads=1, theta=500000.0)
    e = np.zeros((1, 1, 1, 128))
    e[0, 0, 0, 0] = 1.0  # unit vector on the first member of plane 0
    for delta in (1, 3, 1000, 65536):
        st, dk, _ = place(wl, e, e.copy(), [Chunk(0, 1)], [Entry(0, delta, 1)], delta + 1)
        assert st == "ok"
        row = dk[0, 0, delta, 0]
        assert row[0] == pytest.approx(math.cos(delta), abs=1e-15)
        assert row[64] == pytest.approx(math.sin(delta), abs=1e-15)
        assert np.all(row[np.r_[1:64, 65:128]] == 0.0)


# --------------------------------------------------------------- group law

@pytest.mark.parametrize("style", ["half", "interleaved"])
def test_group_law_and_inverse(style):
    """R(d) R(p) = R(p + d); R(-d) R(d) = I; R(0) = I exactly; plane norms kept."""
    D, H = 16, 2
    wl = gqa(rope_dim=D, n_heads=H, style=style, theta=1e6)
    rng = np.random.default_rng(6)
    raw = rng.standard_normal((1, 4, H, D))
    for p, d in [(5, 9), (1000, -999), (65536, 65536), (3, -3), (70000, -65536)]:
        at_p = rope_at(raw, [p] * 4, wl)
        # a chunk cached at p, placed at p + d
        st, moved, _ = place(wl, at_p, at_p.copy(), [Chunk(0, 4, p)], [Entry(0, p + d, 4)],
                             p + d + 4)
        assert st == "ok"
        direct = rope_at(raw, [p + d] * 4, wl)
        scale = 1e-12 * (1 + abs(p + d))
        assert np.allclose(moved[0, 0, p + d:p + d + 4], direct[0], atol=scale, rtol=0)
        # inverse
        st, back, _ = place(wl, moved[:, 0, p + d:p + d + 4].copy(),
                            moved[:, 0, p + d:p + d + 4].copy(), [Chunk(0, 4, p + d)],
                            [Entry(0, p, 4)], p + 4)
        assert np.allclose(back[0, 0, p:p + 4], at_p[0], atol=scale, rtol=0)
        # norms of every plane preserved
        for i in range(D // 2):
            a, b = pair_index(style, D, i)
            n0 = np.hypot(at_p[0, :, :, a], at_p[0, :, :, b])
            n1 = np.hypot(moved[0, 0, p + d:p + d + 4, :, a], moved[0, 0, p + d:p + d + 4, :, b])
            assert np.allclose(n0, n1, atol=1e-13, rtol=0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_zero_shift_is_bit_exact(dtype):
    """A chunk placed where it was cached is copied bit for bit, signed zeros
    and all (R(0) is the identity)."""
    import torch
    rng = np.random.default_rng(7)
    x = rng.standard_normal((2, 9, 2, 128)).astype(np.float32)
    x[0, 0, 0, :8] = -0.0
    x[0, 0, 0, 64:72] = np.array([-1, 2, -3, 4, -0.0, 0.0, 5, -6], dtype=np.float32)
    if dtype == "bf16":
        pk = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        fill = np.uint16(0x7FC5)
    else:
        pk = x
        fill = np.float32(7.0)
    wl = Workload("z", dtype, 2, 2, 128, 0, 128, "half", 5e5, True)
    st, dk, dv = place(wl, pk, pk.copy(), [Chunk(0, 9, 40)], [Entry(0, 40, 9)], 60, dtype=dtype,
                       fill=fill)
    assert st == "ok"
    assert np.array_equal(dk[:, 0, 40:49].view(np.uint8), pk.view(np.uint8))
    assert np.array_equal(dv[:, 0, 40:49].view(np.uint8), pk.view(np.uint8))


# ------------------------------------------------ attention-level invariance

def test_relative_position_invariance_of_scores():
    """q.k after RoPE depends only on the distance n - m: shifting both by the
    same delta leaves every score unchanged (EPIC Guide, RoPE barrier)."""
    D = 32
    wl = gqa(rope_dim=D, n_heads=1, theta=500000.0)
    rng = np.random.default_rng(8)
    q = rng.standard_normal((1, 6, 1, D))
    k = rng.standard_normal((1, 6, 1, D))
    m = np.array([0, 3, 10, 100, 4000, 70000])
    n = np.array([5, 1, 10, 2000, 0, 65536])
    base = np.einsum("td,td->t", rope_at(q, m, wl)[0, :, 0], rope_at(k, n, wl)[0, :, 0])
    for delta in (1, 777, 65536):
        shifted = np.einsum("td,td->t", rope_at(q, m + delta, wl)[0, :, 0],
                            rope_at(k, n + delta, wl)[0, :, 0])
        assert np.allclose(shifted, base, atol=1e-10, rtol=0)
    # and the score does change when only one side moves (position matters)
    moved = np.einsum("td,td->t", rope_at(q, m, wl)[0, :, 0], rope_at(k, n + 1, wl)[0, :, 0])
    assert np.max(np.abs(moved - base)) > 1e-3


def _attention(q, k, v):
    """softmax(q k^T / sqrt(d)) v per head; q [Tq][H][D], k/v [Tk][H][D]."""
    s = np.einsum("qhd,khd->hqk", q, k) / math.sqrt(q.shape[-1])
    s -= s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=-1, keepdims=True)
    return np.einsum("hqk,khd->qhd", p, v)


@pytest.mark.parametrize("style", ["half", "interleaved"])
def test_brute_force_attention_on_stitched_cache(style):
    """Chunks of 3, 5 and 4 tokens, each prefilled alone at positions 0..L-1,
    stitched after a 2-token prefix: attention of later queries over the
    stitched cache equals attention over keys RoPE'd directly at their
    absolute positions; reusing the cached keys without the shift does not."""
    H, D = 2, 8
    wl = gqa(rope_dim=D, n_heads=H, style=style, theta=10000.0)
    rng = np.random.default_rng(9)
    lens, prefix = [3, 5, 4], 2
    raw_k = rng.standard_normal((1, sum(lens), H, D))
    vals = rng.standard_normal((1, sum(lens), H, D))
    local = np.concatenate([np.arange(n) for n in lens])  # positions at caching time
    cached = rope_at(raw_k, local, wl)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]])
    chunks = [Chunk(int(s), n) for s, n in zip(starts, lens)]
    order = [2, 0, 1]
    entries, pos = [], prefix
    for c in order:
        entries.append(Entry(c, pos, lens[c]))
        pos += lens[c]
    total = pos
    st, dk, dv = place(wl, cached, vals, chunks, entries, total)
    assert st == "ok"
    # ground truth: the same raw keys RoPE'd at their absolute positions
    src = np.concatenate([np.arange(starts[c], starts[c] + lens[c]) for c in order])
    absolute = np.arange(prefix, total)
    truth_k = rope_at(raw_k[:, src], absolute, wl)[0]
    truth_v = vals[0, src]
    qraw = rng.standard_normal((1, 4, H, D))
    q = rope_at(qraw, [total + i for i in range(4)], wl)[0]
    got = _attention(q, dk[0, 0, prefix:], dv[0, 0, prefix:])
    want = _attention(q, truth_k, truth_v)
    assert np.allclose(got, want, atol=1e-12, rtol=0)
    naive = _attention(q, cached[0, src], truth_v)
    assert np.max(np.abs(naive - want)) > 1e-3


# ----------------------------------------------- placement, copy and masking

@pytest.mark.parametrize("seed", range(16))
def test_placement_copy_mask_brute_force(seed):
    """Every destination row is, by brute force over (request, entry, token):
    the source row (V and non-rotary K bits unchanged, the rotary slice equal
    to the complex-multiplication rotation), or untouched when masked or not
    covered.  Random ragged problems, contiguous and paged destinations,
    contiguous and paged pools, GQA and MLA rows."""
    paged = seed % 2 == 1
    mla = seed % 3 == 2
    style = "interleaved" if seed % 4 == 3 else "half"
    wl = random_small(seed, dtype="f32", style=style, paged=paged, mla=mla, n_requests=3,
                      n_layers=2)
    paged_pool = seed >= 8
    if paged_pool:
        wl = with_paged_pool(wl, page_size=[4, 16, 8][seed % 3], seed=seed,
                             first_offsets=seed % 2 == 0, spare_pages=3)
    wl.dtype = "f64"
    rng = np.random.default_rng(100 + seed)
    pk = rng.standard_normal(wl.pool_shape())
    pv = rng.standard_normal(wl.pool_shape()) if wl.has_v else None
    dk = np.full(wl.dst_shape(), SENT_F64)
    dv = np.full(wl.dst_shape(), SENT_F64) if wl.has_v else None
    assert oracle.stitch(wl, pk, pv, dk, dv) == "ok"

    theta = oracle.inv_freq(wl.theta, wl.rope_dim)
    rot = np.arange(wl.rope_offset, wl.rope_offset + wl.rope_dim)
    plain = np.setdiff1d(np.arange(wl.row_dim), rot)
    written = np.zeros(wl.dst_shape()[:-2], dtype=bool)
    for r, req in enumerate(wl.requests):
        for e in req.entries:
            ch = wl.chunks[e.chunk_id]
            delta = e.dst_offset - ch.base_pos
            for t in range(e.recompute_k, e.length):
                pos = e.dst_offset + t
                if paged:
                    at = (slice(None), int(req.page_table[pos // wl.page_size]),
                          pos % wl.page_size)
                else:
                    at = (slice(None), r, pos)
                if paged_pool:  # the chunk's token t through its page table
                    off = ch.token_start + t
                    src = (slice(None), int(ch.page_table[off // wl.src_page_size]),
                           off % wl.src_page_size)
                else:
                    src = (slice(None), ch.token_start + t)
                got_k, src_k = dk[at], pk[src]
                written[at] = True
                assert np.array_equal(got_k[..., plain], src_k[..., plain])
                if wl.has_v:
                    assert np.array_equal(dv[at], pv[src])
                for i in range(wl.rope_dim // 2):
                    a, b = pair_index(style, wl.rope_dim, i)
                    a, b = a + wl.rope_offset, b + wl.rope_offset
                    z = (src_k[..., a] + 1j * src_k[..., b]) * np.exp(1j * delta * theta[i])
                    tol = 1e-14 * (1 + abs(delta))
                    assert np.allclose(got_k[..., a], z.real, atol=tol, rtol=0)
                    assert np.allclose(got_k[..., b], z.imag, atol=tol, rtol=0)
    assert np.all(dk[~written] == SENT_F64)
    if wl.has_v:
        assert np.all(dv[~written] == SENT_F64)


# ------------------------------------------------------ the pages' examples

def test_epic_block_composition(golden_dir):
    """Blocks A(128), B(8192), C(1024) cached at offset 0 and composed as
    A + B + C: the page's offsets are the prefix sums of the lengths, and the
    keys of every stitched block equal the keys RoPE'd at the absolute
    position (checked on a 1-head 8-dim row)."""
    g = json.load(open(os.path.join(golden_dir, "epic_block_composition.json")))
    blocks = g["blocks"]
    lens = [b["length"] for b in blocks]
    assert [b["offset"] for b in blocks] == [0] + list(np.cumsum(lens)[:-1])
    wl = gqa(rope_dim=8, n_heads=1, theta=500000.0)
    rng = np.random.default_rng(10)
    raw = rng.standard_normal((1, sum(lens), 1, 8))
    local = np.concatenate([np.arange(n) for n in lens])
    cached = rope_at(raw, local, wl)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]])
    chunks = [Chunk(int(s), n) for s, n in zip(starts, lens)]
    entries = [Entry(i, b["offset"], b["length"]) for i, b in enumerate(blocks)]
    total = sum(lens)
    st, dk, _ = place(wl, cached, cached.copy(), chunks, entries, total)
    assert st == "ok"
    truth = rope_at(raw, np.arange(total), wl)  # composed order == pool order here
    assert np.allclose(dk[0, 0], truth[0], atol=1e-12 * total, rtol=0)
    # block C's first token sits at 8320 and was turned by 8320 * theta_i
    assert entries[2].dst_offset == 8320


def test_epic_doc_d_placement(golden_dir):
    """Document D (10,000 tokens) cached at 0 and reused behind prompt A lands
    on [100, 10100); the whole chunk is shifted by 100."""
    g = json.load(open(os.path.join(golden_dir, "epic_doc_d.json")))
    n, first, end = g["length"], g["first"], g["end"]
    assert end - first == n
    wl = gqa(rope_dim=4, n_heads=1, theta=10000.0)
    rng = np.random.default_rng(11)
    raw = rng.standard_normal((1, n, 1, 4))
    cached = rope_at(raw, np.arange(n), wl)
    st, dk, dv = place(wl, cached, raw.copy(), [Chunk(0, n)], [Entry(0, first, n)], end + 7)
    assert st == "ok"
    assert np.all(dk[0, 0, :first] == SENT_F64) and np.all(dk[0, 0, end:] == SENT_F64)
    truth = rope_at(raw, np.arange(first, end), wl)
    assert np.allclose(dk[0, 0, first:end], truth[0], atol=1e-12 * end, rtol=0)
    assert np.array_equal(dv[0, 0, first:end], raw[0])


def test_epic_chunk_references(golden_dir):
    """Two client chunk references at offsets 128 and 4224: placed adjacent,
    the first spans 4096 tokens; overlapping them by one token is refused."""
    g = json.load(open(os.path.join(golden_dir, "epic_chunk_references.json")))
    o1, o2 = [r["offset"] for r in g["references"]]
    n1 = o2 - o1
    assert n1 == 4096
    wl = gqa(rope_dim=4, n_heads=1)
    pool = np.random.default_rng(12).standard_normal((1, n1 + 64, 1, 4))
    chunks = [Chunk(0, n1), Chunk(n1, 64)]
    st, dk, _ = place(wl, pool, pool.copy(), chunks, [Entry(0, o1, n1), Entry(1, o2, 64)],
                      o2 + 64)
    assert st == "ok"
    st, _, _ = place(wl, pool, pool.copy(), chunks, [Entry(0, o1, n1), Entry(1, o2 - 1, 64)],
                     o2 + 64)
    assert st == "overlap"


def test_mla_rotary_slice_only(golden_dir):
    """In the MLA row (512 content dims + 64 rotary dims) only the rotary slice
    moves; the content latent is reused verbatim."""
    g = json.load(open(os.path.join(golden_dir, "mla_row.json")))
    ckv, kr = g["cKV"], g["k_r"]
    assert ckv / (ckv + kr) == pytest.approx(g["content_share_approx"], abs=0.005)
    wl = Workload("mla", "f64", 1, 1, ckv + kr, ckv, kr, "half", 10000.0, False)
    rng = np.random.default_rng(13)
    pool = rng.standard_normal((1, 10, 1, ckv + kr))
    st, dk, _ = place(wl, pool, None, [Chunk(0, 10)], [Entry(0, 300, 10)], 310)
    assert st == "ok"
    out = dk[0, 0, 300:310, 0]
    assert np.array_equal(out[:, :ckv], pool[0, :, 0, :ckv])
    assert not np.allclose(out[:, ckv:], pool[0, :, 0, ckv:])
    theta = 10000.0 ** (-2.0 * np.arange(kr // 2) / kr)
    z = (pool[0, :, 0, ckv:ckv + kr // 2] + 1j * pool[0, :, 0, ckv + kr // 2:]) * \
        np.exp(1j * 300 * theta)
    assert np.allclose(out[:, ckv:ckv + kr // 2], z.real, atol=1e-13)
    assert np.allclose(out[:, ckv + kr // 2:], z.imag, atol=1e-13)


def test_bf16_error_below_irminsul_bound(golden_dir):
    """The oracle's bf16 result (one rounding of the exact rotation) has a
    relative L2 error far below the 4.7e-3 the Irminsul page reports."""
    import torch
    bound = json.load(open(os.path.join(golden_dir, "irminsul_bf16_error.json")))["rel_l2_bf16"]
    rng = np.random.default_rng(14)
    x = rng.standard_normal((1, 2000, 1, 64)).astype(np.float32)
    xb = torch.from_numpy(x).to(torch.bfloat16)
    xbits = xb.view(torch.int16).numpy().view(np.uint16)
    xf64 = xb.to(torch.float64).numpy()
    wl_b = Workload("e", "bf16", 1, 1, 64, 0, 64, "half", 10000.0, False)
    wl_f = Workload("e", "f64", 1, 1, 64, 0, 64, "half", 10000.0, False)
    _, kb, _ = place(wl_b, xbits, None, [Chunk(0, 2000)], [Entry(0, 5000, 2000)], 7000,
                     dtype="bf16", fill=np.uint16(0))
    _, kf, _ = place(wl_f, xf64, None, [Chunk(0, 2000)], [Entry(0, 5000, 2000)], 7000)
    got = torch.from_numpy(kb[0, 0, 5000:].view(np.int16)).view(torch.bfloat16).double().numpy()
    exact = kf[0, 0, 5000:]
    rel = np.linalg.norm(got - exact) / np.linalg.norm(exact)
    assert rel < bound / 2
    assert rel > 1e-4  # bf16 storage does round


# ------------------------------------------------------------- in-place mode

def test_inplace_matches_copy_mode_and_leaves_the_rest():
    """Rotating segments in place equals placing them by copy at a position
    delta away from their cached one; tokens [0, k), other dims and other
    tokens stay untouched."""
    rng = np.random.default_rng(15)
    D, H, T = 16, 2, 40
    buf = rng.standard_normal((2, T, H, D + 8))
    segs = [Segment(0, 10, 5, 3), Segment(10, 12, -70000, 0), Segment(25, 15, 0, 2),
            Segment(22, 3, 1, 3)]
    wl = Workload("ip", "f64", 2, H, D + 8, 8, D, "half", 1e6, False, inplace=True,
                  n_tokens=T, segments=segs)
    out = buf.copy()
    assert oracle.rotate_inplace(wl, out) == "ok"
    for s in segs:
        sl = slice(s.token_start, s.token_start + s.recompute_k)
        assert np.array_equal(out[:, sl], buf[:, sl])
        ts = slice(s.token_start + s.recompute_k, s.token_start + s.length)
        assert np.array_equal(out[:, ts, :, :8], buf[:, ts, :, :8])
        cw = Workload("cp", "f64", 2, H, D + 8, 8, D, "half", 1e6, False)
        n = s.length - s.recompute_k
        if n == 0:
            continue
        src = buf[:, ts].copy()
        st, dk, _ = place(cw, src, None, [Chunk(0, n, 80000)], [Entry(0, 80000 + s.delta, n)],
                          80000 + s.delta + n)
        assert st == "ok"
        assert np.array_equal(out[:, ts], dk[:, 0, 80000 + s.delta:])


# ------------------------------------------------------------- validation

def _valid_problem():
    wl = random_small(3, dtype="f32", paged=True, n_requests=2)
    assert oracle.validate_stitch(wl) == "ok"
    return wl


@pytest.mark.parametrize("mutate,expect", [
    (lambda w: setattr(w, "rope_dim", 7), "bad_arg"),
    (lambda w: setattr(w, "rope_offset", w.row_dim - w.rope_dim + 1), "bad_arg"),
    (lambda w: setattr(w, "n_heads", 0), "bad_arg"),
    (lambda w: setattr(w, "theta", 0.0), "bad_arg"),
    (lambda w: w.chunks.__setitem__(0, Chunk(w.pool_tokens - 1, 5)), "range"),
    (lambda w: w.requests[0].entries.__setitem__(0, Entry(99, 0, 1)), "range"),
    (lambda w: w.requests[0].entries.__setitem__(
        0, Entry(w.requests[0].entries[0].chunk_id, w.requests[0].entries[0].dst_offset,
                 w.requests[0].entries[0].length, w.requests[0].entries[0].length + 1)),
     "range"),
    (lambda w: w.requests[0].page_table.__setitem__(0, w.n_phys_pages), "range"),
])
def test_validation_single_defects(mutate, expect):
    wl = _valid_problem()
    wl.chunks = list(wl.chunks)
    wl.requests[0].entries = list(wl.requests[0].entries)
    e0 = wl.requests[0].entries[0]
    # make sure the mutated page is one the first entry writes
    if e0.recompute_k >= e0.length:
        wl.requests[0].entries[0] = Entry(e0.chunk_id, e0.dst_offset, e0.length, 0)
        e0 = wl.requests[0].entries[0]
    first_page = (e0.dst_offset + e0.recompute_k) // wl.page_size
    pt = wl.requests[0].page_table
    pt[[0, first_page]] = pt[[first_page, 0]]
    assert oracle.validate_stitch(wl) == "ok"
    mutate(wl)
    assert oracle.validate_stitch(wl) == expect


def test_validation_overlaps_and_no_write_on_error():
    wl = Workload("ov", "f32", 1, 1, 8, 0, 8, "half", 1e4, True, pool_tokens=20,
                  chunks=[Chunk(0, 10), Chunk(10, 10)], capacity=40,
                  requests=[Request([Entry(0, 0, 10), Entry(1, 9, 10)])])
    assert oracle.validate_stitch(wl) == "overlap"
    pk = np.ones((1, 20, 1, 8), np.float32)
    dk = np.zeros((1, 1, 40, 1, 8), np.float32)
    dv = np.zeros_like(dk)
    assert oracle.stitch(wl, pk, pk.copy(), dk, dv) == "overlap"
    assert not dk.any() and not dv.any()
    # two requests writing the same physical row of a paged pool
    wl2 = Workload("ov2", "f32", 1, 1, 8, 0, 8, "half", 1e4, True, pool_tokens=20,
                   chunks=[Chunk(0, 10)], page_size=4, n_phys_pages=6,
                   requests=[Request([Entry(0, 0, 4)], np.array([5], np.int32)),
                             Request([Entry(0, 2, 2)], np.array([5], np.int32))])
    assert oracle.validate_stitch(wl2) == "overlap"
    # ... but disjoint rows of one shared page are fine, and masked rows do not count
    wl2.requests[1] = Request([Entry(0, 0, 4, 4)], np.array([5], np.int32))
    assert oracle.validate_stitch(wl2) == "ok"
    # duplicate chunk ids and negative shifts are allowed
    wl3 = Workload("dup", "f32", 1, 1, 8, 0, 8, "half", 1e4, True, pool_tokens=20,
                   chunks=[Chunk(0, 10, 500)], capacity=40,
                   requests=[Request([Entry(0, 0, 10), Entry(0, 20, 10)])])
    assert oracle.validate_stitch(wl3) == "ok"
    # layer range
    assert oracle.validate_stitch(wl3, 0, 2) == "bad_arg"
    # in-place segments overlapping
    ip = Workload("ip", "f32", 1, 1, 8, 0, 8, "half", 1e4, False, inplace=True, n_tokens=10,
                  segments=[Segment(0, 5, 1), Segment(4, 3, 1)])
    assert oracle.validate_inplace(ip) == "overlap"
    ip.segments = [Segment(0, 5, 1), Segment(5, 6, 1)]
    assert oracle.validate_inplace(ip) == "range"


def test_validation_paged_pool():
    """Paged pool: chunks must fit their page tables, pages read must exist;
    pages of masked tokens are not read."""
    base = Workload("pp", "f32", 1, 1, 8, 0, 8, "half", 1e4, True, capacity=40,
                    chunks=[Chunk(2, 10, 0, np.array([5, 1, 3], np.int32))],
                    requests=[Request([Entry(0, 0, 10, 0)])], src_page_size=4, src_n_pages=6)
    assert oracle.validate_stitch(base) == "ok"
    w = copy.deepcopy(base)
    w.chunks = [Chunk(3, 10, 0, np.array([5, 1, 3], np.int32))]  # 3 + 10 > 3 pages x 4
    assert oracle.validate_stitch(w) == "range"
    w = copy.deepcopy(base)
    w.chunks = [Chunk(2, 10, 0, np.array([5, 6, 3], np.int32))]  # page 6 of 6
    assert oracle.validate_stitch(w) == "range"
    w.requests = [Request([Entry(0, 0, 10, 6)])]  # page 6 holds tokens 2..5 only: masked
    assert oracle.validate_stitch(w) == "ok"


# ------------------------------------------------------------ decode attention

def _attend_case(H=2, D=8, G=2, L=20, entries=(), chunks=(), seed=20, same_keys=False):
    """A one-request problem whose own cache holds every context position
    (contiguous destination), pool of the given chunks, f64 storage."""
    rng = np.random.default_rng(seed)
    pool_tokens = max([c.token_start + c.length for c in chunks] + [1])
    wl = Workload("att", "f64", 1, H, D, 0, D, "half", 10000.0, True, pool_tokens=pool_tokens,
                  chunks=list(chunks), requests=[Request(list(entries), None, L)], capacity=L)
    pk = rng.standard_normal((1, pool_tokens, H, D))
    pv = rng.standard_normal((1, pool_tokens, H, D))
    ck = rng.standard_normal((1, 1, L, H, D))
    if same_keys:
        ck[:] = ck[0, 0, 0]
    cv = rng.standard_normal((1, 1, L, H, D))
    q = rng.standard_normal((1, H * G, D))
    return wl, pk, pv, ck, cv, q


def test_attend_uniform_keys_average_values():
    """Equal keys give equal weights: the output is the mean value row."""
    wl, pk, pv, ck, cv, q = _attend_case(same_keys=True)
    out = oracle.attend(wl, pk, pv, ck, cv, q, 0)
    for j in range(q.shape[1]):
        assert np.allclose(out[0, j], cv[0, 0, :, j // 2].mean(axis=0), atol=1e-13)


def test_attend_sink_bias_closed_form():
    """With equal keys, a logit bias b on the first sink_tokens positions of a
    chunk placed after 0 weights them by e^b against 1 for the rest."""
    ch = [Chunk(0, 6)]
    wl, pk, pv, ck, cv, q = _attend_case(L=20, entries=[Entry(0, 8, 6, 6)], chunks=ch,
                                         same_keys=True)
    for b in (-15.0, -2.0, 3.0):
        out = oracle.attend(wl, pk, pv, ck, cv, q, 0, sink_tokens=4, sink_bias=b)
        wts = np.ones(20)
        wts[8:12] = np.exp(b)
        for j in range(q.shape[1]):
            want = (wts[:, None] * cv[0, 0, :, j // 2]).sum(0) / wts.sum()
            assert np.allclose(out[0, j], want, atol=1e-13)
    # an entry at position 0 carries no pseudo-sink (the global sink is real)
    wl.requests[0].entries = [Entry(0, 0, 6, 6)]
    out0 = oracle.attend(wl, pk, pv, ck, cv, q, 0, sink_tokens=4, sink_bias=-15.0)
    assert np.allclose(out0[0, 0], cv[0, 0, :, 0].mean(0), atol=1e-13)


def test_attend_single_position_and_gqa_heads():
    """A one-position context returns that value row; query head j reads KV
    head j // G."""
    wl, pk, pv, ck, cv, q = _attend_case(H=3, G=2, L=1)
    out = oracle.attend(wl, pk, pv, ck, cv, q, 0)
    for j in range(6):
        assert np.array_equal(out[0, j], cv[0, 0, 0, j // 2])


@pytest.mark.parametrize("style", ["half", "interleaved"])
def test_attend_rotated_chunks_equal_direct_rope(style):
    """Chunks cached at positions 0..L-1 and placed (rotated on the way in)
    attend exactly like keys RoPE'd directly at their absolute positions
    sitting in the cache; reusing the cached keys unturned does not."""
    H, D, G = 2, 8, 2
    lens, starts = [5, 7], [0, 5]
    rng = np.random.default_rng(21)
    raw = rng.standard_normal((1, 12, H, D))
    wl0 = gqa(rope_dim=D, n_heads=H, style=style)
    cached = rope_at(raw, np.concatenate([np.arange(5), np.arange(7)]), wl0)
    vals = rng.standard_normal((1, 12, H, D))
    chunks = [Chunk(starts[0], lens[0]), Chunk(starts[1], lens[1])]
    entries = [Entry(1, 3, 7), Entry(0, 12, 5, 2)]  # chunk 1 at 3, chunk 0 at 12 (2 recomputed)
    L = 18
    wl = Workload("att", "f64", 1, H, D, 0, D, style, 10000.0, True, pool_tokens=12,
                  chunks=chunks, requests=[Request(entries, None, L)], capacity=L)
    ck = rng.standard_normal((1, 1, L, H, D))
    cv = rng.standard_normal((1, 1, L, H, D))
    q = rng.standard_normal((1, H * G, D))
    got = oracle.attend(wl, cached, vals, ck, cv, q, 0)
    # the same context written out: direct RoPE at absolute positions
    dk, dv = ck.copy(), cv.copy()
    dk[0, 0, 3:10] = rope_at(raw[:, 5:12], np.arange(3, 10), wl0)[0]
    dv[0, 0, 3:10] = vals[0, 5:12]
    dk[0, 0, 14:17] = rope_at(raw[:, 2:5], np.arange(14, 17), wl0)[0]
    dv[0, 0, 14:17] = vals[0, 2:5]
    plain = Workload("att", "f64", 1, H, D, 0, D, style, 10000.0, True, pool_tokens=12,
                     chunks=chunks, requests=[Request([], None, L)], capacity=L)
    want = oracle.attend(plain, cached, vals, dk, dv, q, 0)
    assert np.allclose(got, want, atol=1e-12)
    naive_k = dk.copy()
    naive_k[0, 0, 3:10] = cached[0, 5:12]
    naive = oracle.attend(plain, cached, vals, naive_k, dv, q, 0)
    assert np.max(np.abs(naive - want)) > 1e-3


# ------------------------------------------------------ latent (MLA) attention

def _latent_case(L=20, entries=(), chunks=(), Hq=3, D=12, ro=8, seed=30, same_rows=False,
                 style="half"):
    """One request, MLA-shaped rows (content [0, ro), rotary [ro, D)), f64."""
    rng = np.random.default_rng(seed)
    pool_tokens = max([c.token_start + c.length for c in chunks] + [1])
    wl = Workload("lat", "f64", 1, 1, D, ro, D - ro, style, 10000.0, False,
                  pool_tokens=pool_tokens, chunks=list(chunks),
                  requests=[Request(list(entries), None, L)], capacity=L)
    pk = rng.standard_normal((1, pool_tokens, 1, D))
    ck = rng.standard_normal((1, 1, L, 1, D))
    if same_rows:
        ck[:] = ck[0, 0, 0]
    q = rng.standard_normal((1, Hq, D))
    return wl, pk, ck, q


def test_latent_attend_equal_rows_and_sink_bias():
    """Equal rows give equal weights: every head returns the content latent;
    a bias b on the first sink_tokens of a chunk after 0 weights them e^b."""
    wl, pk, ck, q = _latent_case(same_rows=True)
    out = oracle.attend_latent(wl, pk, ck, q, 0)
    for j in range(3):
        assert np.allclose(out[0, j], ck[0, 0, 0, 0, :8], atol=1e-13)
    # the chunk at 8 is all recompute tokens (read from the cache); equal
    # rotary keys and a query with no content part make every logit equal,
    # while the content latents (the values) differ
    wl, pk, ck, q = _latent_case(L=20, entries=[Entry(0, 8, 6, 6)], chunks=[Chunk(0, 6)])
    ck[0, 0, :, 0, 8:] = ck[0, 0, 0, 0, 8:]
    q[0, :, :8] = 0.0
    for b in (-15.0, 2.5):
        out = oracle.attend_latent(wl, pk, ck, q, 0, sink_tokens=4, sink_bias=b)
        wts = np.ones(20)
        wts[8:12] = np.exp(b)
        want = (wts[:, None] * ck[0, 0, :, 0, :8]).sum(0) / wts.sum()
        for j in range(3):
            assert np.allclose(out[0, j], want, atol=1e-13)


def test_latent_attend_single_position():
    wl, pk, ck, q = _latent_case(L=1)
    out = oracle.attend_latent(wl, pk, ck, q, 0)
    for j in range(3):
        assert np.array_equal(out[0, j], ck[0, 0, 0, 0, :8])


@pytest.mark.parametrize("style", ["half", "interleaved"])
def test_latent_attend_rotated_chunks_equal_direct_rope(style):
    """MLA chunks whose rotary keys were RoPE'd at 0..L-1, placed and turned
    (in fp64), attend exactly like rows RoPE'd directly at their absolute
    positions; unturned reuse differs."""
    D, ro = 12, 8
    rng = np.random.default_rng(32)
    raw = rng.standard_normal((1, 12, 1, D))
    wl0 = gqa(rope_dim=D - ro, n_heads=1, style=style, row_dim=D, rope_offset=ro, has_v=False)
    cached = rope_at(raw, np.concatenate([np.arange(5), np.arange(7)]), wl0)
    chunks = [Chunk(0, 5), Chunk(5, 7)]
    entries = [Entry(1, 3, 7), Entry(0, 12, 5, 2)]
    L = 18
    wl = Workload("lat", "f64", 1, 1, D, ro, D - ro, style, 10000.0, False, pool_tokens=12,
                  chunks=chunks, requests=[Request(entries, None, L)], capacity=L)
    ck = rng.standard_normal((1, 1, L, 1, D))
    q = rng.standard_normal((1, 4, D))
    got = oracle.attend_latent(wl, cached, ck, q, 0, dtype="f64")
    dk = ck.copy()
    dk[0, 0, 3:10] = rope_at(raw[:, 5:12], np.arange(3, 10), wl0)[0]
    dk[0, 0, 14:17] = rope_at(raw[:, 2:5], np.arange(14, 17), wl0)[0]
    plain = Workload("lat", "f64", 1, 1, D, ro, D - ro, style, 10000.0, False, pool_tokens=12,
                     chunks=chunks, requests=[Request([], None, L)], capacity=L)
    want = oracle.attend_latent(plain, cached, dk, q, 0, dtype="f64")
    assert np.allclose(got, want, atol=1e-12)
    naive_k = dk.copy()
    naive_k[0, 0, 3:10] = cached[0, 5:12]
    assert np.max(np.abs(oracle.attend_latent(plain, cached, naive_k, q, 0) - want)) > 1e-3


def test_latent_attend_matches_library_attention_over_stitched_bf16_rows():
    """bf16 storage: the oracle's latent attention equals torch's scaled dot
    product attention (fp64, CPU) over the rows its stitch stores (rotary
    keys rounded to bf16), with the content latent as the values."""
    import torch
    from parity_util import to_host
    from pic_workloads import normal_values
    D, ro = 576, 512
    chunks = [Chunk(0, 40), Chunk(40, 30)]
    entries = [Entry(1, 10, 30, 4), Entry(0, 45, 40)]
    L = 90
    wl = Workload("lat", "bf16", 1, 1, D, ro, 64, "half", 10000.0, False, pool_tokens=70,
                  chunks=chunks, requests=[Request(entries, None, L)], capacity=L)
    pk = to_host(normal_values((1, 70, 1, D), "bf16", 1))
    ck = to_host(normal_values((1, 1, L, 1, D), "bf16", 2))
    q = to_host(normal_values((1, 16, D), "bf16", 3))
    sc = 192 ** -0.5
    got = oracle.attend_latent(wl, pk, ck, q, 0, scale=sc, sink_tokens=4, sink_bias=-15.0)
    rows = ck.copy()
    assert oracle.stitch(wl, pk, None, rows, None) == "ok"
    k = torch.from_numpy(oracle.ref._to_f64(rows[0, 0, :, 0]))
    bias = torch.zeros(L, dtype=torch.float64)
    bias[45:49] = -15.0  # the chunk placed at 45 (the one at 10 starts with recompute tokens)
    bias[10:14] = -15.0
    qq = torch.from_numpy(oracle.ref._to_f64(q[0]))
    want = torch.nn.functional.scaled_dot_product_attention(
        qq[None], k[None].contiguous(), k[None, :, :ro].contiguous(),
        attn_mask=bias[None, None, :].expand(1, 16, L), scale=sc)[0].numpy()
    assert np.allclose(got[0], want, rtol=0, atol=1e-12)


# -------------------------------------------- LegoLink boundary reconnection

def test_boundary_rows_enumerate_relocated_entries():
    wl = Workload("b", "f64", 1, 1, 8, 0, 8, "half", 1e4, True, pool_tokens=30,
                  chunks=[Chunk(0, 10), Chunk(10, 20)], capacity=60,
                  requests=[Request([Entry(0, 0, 10), Entry(1, 12, 3), Entry(1, 20, 20)])])
    rows = oracle.boundary_rows(wl, 4)
    assert rows == [(0, 1, 0, 12), (0, 1, 1, 13), (0, 1, 2, 14),
                    (0, 2, 0, 20), (0, 2, 1, 21), (0, 2, 2, 22), (0, 2, 3, 23)]


@pytest.mark.parametrize("style", ["half", "interleaved"])
def test_boundary_attention_equals_decode_attention_at_each_position(style):
    """Boundary token j of an entry at d attends exactly like a decode step
    whose context ends at d + j (the decode oracle, an independent path),
    damping included."""
    H, D, G, L = 2, 8, 2, 40
    rng = np.random.default_rng(40)
    chunks = [Chunk(0, 9), Chunk(9, 12)]
    entries = [Entry(1, 3, 12, 2), Entry(0, 20, 9)]
    wl = Workload("b", "f64", 1, H, D, 0, D, style, 1e4, True, pool_tokens=21, chunks=chunks,
                  requests=[Request(entries, None, L)], capacity=L)
    pk = rng.standard_normal((1, 21, H, D))
    pv = rng.standard_normal((1, 21, H, D))
    ck = rng.standard_normal((1, 1, L, H, D))
    cv = rng.standard_normal((1, 1, L, H, D))
    rows = oracle.boundary_rows(wl, 5)
    q = rng.standard_normal((len(rows), H * G, D))
    got = oracle.attend_boundary(wl, pk, pv, ck, cv, q, 0, 5, sink_tokens=3, sink_bias=-4.0,
                                 dtype="f64")
    for b, (_, _, _, p) in enumerate(rows):
        dec = Workload("b", "f64", 1, H, D, 0, D, style, 1e4, True, pool_tokens=21,
                       chunks=chunks, requests=[Request(entries, None, p + 1)], capacity=L)
        want = oracle.attend(dec, pk, pv, ck, cv, q[b:b + 1], 0, sink_tokens=3, sink_bias=-4.0)
        assert np.allclose(got[b], want[0], atol=1e-12)


def test_boundary_rows_given_by_the_caller():
    """Caller rows (entry, token), entries numbered in plan order: the
    positions follow from each entry's offset; a token outside its entry is
    refused."""
    wl = Workload("b", "f64", 1, 1, 8, 0, 8, "half", 1e4, True, pool_tokens=30,
                  chunks=[Chunk(0, 10), Chunk(10, 20)], capacity=60,
                  requests=[Request([Entry(0, 0, 10), Entry(1, 12, 3)]), Request([Entry(1, 20, 20)])])
    assert oracle.boundary_rows(wl, 0, rows=[(1, 2), (0, 9), (2, 17), (2, 0)]) == \
        [(0, 1, 2, 14), (0, 0, 9, 9), (1, 0, 17, 37), (1, 0, 0, 20)]
    with pytest.raises(ValueError):
        oracle.boundary_rows(wl, 0, rows=[(1, 3)])


@pytest.mark.parametrize("style", ["half", "interleaved"])
def test_caller_boundary_rows_equal_decode_attention_at_their_positions(style):
    """Caller rows anywhere in an entry (past the first k tokens, in the entry
    at position 0, repeated, out of order within the request) each attend
    exactly like a decode step whose context ends at the row's position
    (the decode oracle)."""
    H, D, G, L = 2, 8, 2, 40
    rng = np.random.default_rng(41)
    chunks = [Chunk(0, 9), Chunk(9, 12)]
    entries = [Entry(1, 3, 12, 2), Entry(0, 20, 9), Entry(0, 0, 3)]
    wl = Workload("b", "f64", 1, H, D, 0, D, style, 1e4, True, pool_tokens=21, chunks=chunks,
                  requests=[Request(entries, None, L)], capacity=L)
    pk = rng.standard_normal((1, 21, H, D))
    pv = rng.standard_normal((1, 21, H, D))
    ck = rng.standard_normal((1, 1, L, H, D))
    cv = rng.standard_normal((1, 1, L, H, D))
    given = [(1, 8), (0, 11), (2, 0), (2, 2), (0, 0), (1, 8), (0, 5)]
    rows = oracle.boundary_rows(wl, 0, rows=given)
    q = rng.standard_normal((len(rows), H * G, D))
    got = oracle.attend_boundary(wl, pk, pv, ck, cv, q, 0, 0, sink_tokens=3, sink_bias=-4.0,
                                 dtype="f64", rows=given)
    for b, (_, _, _, p) in enumerate(rows):
        dec = Workload("b", "f64", 1, H, D, 0, D, style, 1e4, True, pool_tokens=21,
                       chunks=chunks, requests=[Request(entries, None, p + 1)], capacity=L)
        want = oracle.attend(dec, pk, pv, ck, cv, q[b:b + 1], 0, sink_tokens=3, sink_bias=-4.0)
        assert np.allclose(got[b], want[0], atol=1e-12)


def test_boundary_attention_matches_library_sdpa_bf16():
    """bf16 storage: equals torch's scaled dot product attention (fp64, CPU)
    over the rows the oracle's stitch stores, with a causal limit per row."""
    import torch
    from parity_util import to_host
    from pic_workloads import normal_values
    H, D, G, L = 2, 128, 4, 96
    chunks = [Chunk(0, 30), Chunk(30, 40)]
    entries = [Entry(0, 0, 30), Entry(1, 40, 40, 3)]
    wl = Workload("b", "bf16", 1, H, D, 0, D, "half", 5e5, True, pool_tokens=70, chunks=chunks,
                  requests=[Request(entries, None, L)], capacity=L)
    pk = to_host(normal_values((1, 70, H, D), "bf16", 1))
    pv = to_host(normal_values((1, 70, H, D), "bf16", 2))
    ck = to_host(normal_values((1, 1, L, H, D), "bf16", 3))
    cv = to_host(normal_values((1, 1, L, H, D), "bf16", 4))
    rows = oracle.boundary_rows(wl, 16)
    q = to_host(normal_values((len(rows), H * G, D), "bf16", 5))
    got = oracle.attend_boundary(wl, pk, pv, ck, cv, q, 0, 16, scale=0.09)
    sk, sv = ck.copy(), cv.copy()
    assert oracle.stitch(wl, pk, pv, sk, sv) == "ok"
    K = torch.from_numpy(oracle.ref._to_f64(sk[0, 0]))  # [L][H][D]
    V = torch.from_numpy(oracle.ref._to_f64(sv[0, 0]))
    for b, (_, _, _, p) in enumerate(rows):
        qq = torch.from_numpy(oracle.ref._to_f64(q[b])).view(H, G, 1, D)
        mask = torch.full((1, 1, 1, L), float("-inf"), dtype=torch.float64)
        mask[..., :p + 1] = 0.0
        want = torch.nn.functional.scaled_dot_product_attention(
            qq, K.permute(1, 0, 2)[:, None].expand(H, G, L, D).contiguous(),
            V.permute(1, 0, 2)[:, None].expand(H, G, L, D).contiguous(),
            attn_mask=mask, scale=0.09).reshape(H * G, D).numpy()
        assert np.allclose(got[b], want, rtol=0, atol=1e-12), b


# ------------------------------------------------------- recompute ranges

def test_recompute_ranges_irminsul_carveout(golden_dir):
    """The MLA workload places its first chunk at absolute position 0, the
    only chunk the carve-out applies to: exactly one range, its first 32
    tokens (the page's figure), and none for the chunks placed after it."""
    from pic_workloads import config4
    g = json.load(open(os.path.join(golden_dir, "irminsul_carveout.json")))
    wl = config4()
    at_zero = [e for e in wl.requests[0].entries if e.dst_offset == g["applies_at_position"]]
    assert len(at_zero) == 1
    assert oracle.recompute_ranges(wl) == [(0, 0, g["recompute_tokens"])]


def test_recompute_ranges_llama_paged_workload():
    """The Llama-3-8B paged workload: 8 chunks of 2048 tokens behind a
    128-token prefix, each with its first 32 tokens left for recompute, give
    the eight ranges [128 + 2048 j, 160 + 2048 j)."""
    from pic_workloads import config2
    want = [(0, 128 + 2048 * j, 160 + 2048 * j) for j in range(8)]
    assert oracle.recompute_ranges(config2()) == want


@pytest.mark.parametrize("seed", range(10))
def test_recompute_ranges_are_the_rows_the_stitch_leaves(seed):
    """Brute force over every position of every request: after the oracle's
    stitch onto a sentinel-filled destination, the positions inside an
    entry whose K row still holds the sentinel form a prefix of that entry,
    and those prefixes are exactly the ranges recompute_ranges lists (entry
    by entry, empty ones omitted)."""
    paged = seed % 2 == 1
    wl = random_small(200 + seed, dtype="f32", paged=paged, mla=seed % 3 == 2, n_requests=3,
                      n_layers=1)
    wl.dtype = "f64"
    rng = np.random.default_rng(seed)
    pk = rng.standard_normal(wl.pool_shape())
    pv = rng.standard_normal(wl.pool_shape()) if wl.has_v else None
    dk = np.full(wl.dst_shape(), SENT_F64)
    dv = np.full(wl.dst_shape(), SENT_F64) if wl.has_v else None
    assert oracle.stitch(wl, pk, pv, dk, dv) == "ok"

    def untouched(r, pos):
        if paged:
            row = dk[0, int(wl.requests[r].page_table[pos // wl.page_size]), pos % wl.page_size]
        else:
            row = dk[0, r, pos]
        return bool(np.all(row == SENT_F64))

    want = []
    for r, req in enumerate(wl.requests):
        for e in req.entries:
            kept = [untouched(r, p) for p in range(e.dst_offset, e.dst_offset + e.length)]
            n = kept.index(False) if False in kept else len(kept)
            assert not any(kept[n:])  # the untouched positions are a prefix
            if n:
                want.append((r, e.dst_offset, e.dst_offset + n))
    assert oracle.recompute_ranges(wl) == want
