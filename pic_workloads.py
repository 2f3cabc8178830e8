"""Seeded synthetic inputs for position-independent KV stitching.

This module only builds inputs: chunk pools, per-request placement tables,
page tables, in-place segments and the random key/value contents.  It holds
none of the stitching arithmetic (no rotation, no shift, no address
translation), so both the HIP library and the oracle can be fed from it.

Structure (lengths, orders, offsets, page permutations, shifts) is drawn
with ``numpy.random.default_rng(seed)``; values are N(0, 1) drawn with
torch's generator (on the CPU or the device) and rounded to the storage
type by torch.

The five named workloads follow the shapes of the pages' workloads:
multi-document RAG with re-ordered documents after a system prompt (EPIC
Guide, "Prefix Caching Failure in Real-World RAG" and the benchmark section),
agentic shifted chunks on an MLA model (Irminsul, Technical Summary sections
2.1, 2.2 and 4) and 128k-token composed prompts (EPIC Guide,
needle-in-a-haystack up to 128k).  No benchmark data is used.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import List, Optional

import numpy as np

DTYPE_BYTES = {"f32": 4, "bf16": 2}

# Destination fill before a stitch: quiet-NaN patterns with a payload, so an
# untouched row is recognisable bit for bit.
SENTINEL_BITS = {"f32": 0x7FC5A5A5, "bf16": 0x7FC5}


@dataclass(frozen=True, eq=False)
class Chunk:
    token_start: int  # contiguous pool: first row; paged pool: offset in the first page
    length: int
    base_pos: int = 0  # position its keys were cached at (virtual offset 0)
    page_table: Optional[np.ndarray] = None  # paged pool: physical pages of the chunk


@dataclass(frozen=True)
class Entry:
    chunk_id: int
    dst_offset: int  # logical position of the chunk's first token
    length: int
    recompute_k: int = 0


@dataclass
class Request:
    entries: List[Entry]
    page_table: Optional[np.ndarray] = None  # int32 physical page per logical page
    context_len: int = 0  # attention context [0, context_len); 0 = up to the last entry


@dataclass(frozen=True)
class Segment:
    token_start: int
    length: int
    delta: int
    recompute_k: int = 0


@dataclass(frozen=True)
class PageSegment:
    """A segment of a paged buffer (pic_rotate_paged): tokens [0, length) at
    logical positions first + t of the block table `pages`; cow[i] >= 0 is
    the page a shared page i is copied to, -1 a page the caller owns."""
    pages: tuple
    cow: Optional[tuple]
    delta: int
    first: int
    length: int
    recompute_k: int = 0


@dataclass
class Workload:
    name: str
    dtype: str  # "f32" | "bf16"
    n_layers: int
    n_heads: int
    row_dim: int
    rope_offset: int
    rope_dim: int
    style: str  # "half" | "interleaved"
    theta: float
    has_v: bool
    pool_tokens: int = 0
    chunks: List[Chunk] = field(default_factory=list)
    requests: List[Request] = field(default_factory=list)
    page_size: int = 0  # 0 = contiguous destination
    capacity: int = 0  # contiguous: positions per request
    n_phys_pages: int = 0
    src_page_size: int = 0  # 0 = contiguous pool
    src_n_pages: int = 0
    inplace: bool = False
    n_tokens: int = 0  # in-place buffer length
    segments: List[Segment] = field(default_factory=list)
    inv_freq: Optional[np.ndarray] = None

    @property
    def esize(self) -> int:
        return DTYPE_BYTES[self.dtype]

    @property
    def row_elems(self) -> int:
        return self.n_heads * self.row_dim

    def pool_shape(self):
        if self.src_page_size:
            return (self.n_layers, self.src_n_pages, self.src_page_size, self.n_heads,
                    self.row_dim)
        return (self.n_layers, self.pool_tokens, self.n_heads, self.row_dim)

    def dst_shape(self):
        if self.page_size:
            return (self.n_layers, self.n_phys_pages, self.page_size, self.n_heads, self.row_dim)
        return (self.n_layers, len(self.requests), self.capacity, self.n_heads, self.row_dim)

    def buf_shape(self):
        return (self.n_layers, self.n_tokens, self.n_heads, self.row_dim)

    def with_layers(self, n_layers: int) -> "Workload":
        return replace(self, n_layers=n_layers)


def tp_share(wl: Workload, tp: int) -> Workload:
    """One GPU's share of `wl` under tensor parallelism of degree tp: the same
    chunks, requests and pages with n_heads / tp KV heads (each GPU stitches
    its own heads with the same plan; no data crosses GPUs)."""
    if tp < 1 or wl.n_heads % tp:
        raise ValueError(f"{wl.n_heads} KV heads do not split {tp} ways")
    return replace(wl, name=f"{wl.name}, 1/{tp} of the KV heads", n_heads=wl.n_heads // tp)


# ---------------------------------------------------------------- workloads

def config1() -> Workload:
    """One layer, 8 KV heads x 128, fp32, three chunks of 512/1024/256 tokens
    cached at offset 0, stitched at 64, 576 and 1600 behind a 64-token
    prefix, nothing recomputed, contiguous destination."""
    lens = [512, 1024, 256]
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]])
    chunks = [Chunk(int(s), int(n)) for s, n in zip(starts, lens)]
    entries = [Entry(0, 64, 512), Entry(1, 576, 1024), Entry(2, 1600, 256)]
    return Workload("single-layer fp32 3-chunk", "f32", 1, 8, 128, 0, 128, "half", 500000.0,
                    True, pool_tokens=int(sum(lens)), chunks=chunks,
                    requests=[Request(entries)], capacity=1856)


def config2(seed: int = 0, n_layers: int = 32) -> Workload:
    """Llama-3-8B-shaped cache: 32 layers, 8 KV heads x 128, bf16; one request
    of 8 chunks x 2048 tokens in a seeded random order behind a 128-token
    prefix; paged destination (16-token pages, physical pages a random
    permutation); the first 32 tokens of every chunk left for recompute."""
    rng = np.random.default_rng(seed)
    n, length, prefix, ps = 8, 2048, 128, 16
    chunks = [Chunk(i * length, length) for i in range(n)]
    order = rng.permutation(n)
    entries = [Entry(int(c), prefix + j * length, length, 32) for j, c in enumerate(order)]
    n_pages = (prefix + n * length) // ps
    table = rng.permutation(n_pages).astype(np.int32)
    return Workload("llama3-8b paged 8x2048", "bf16", n_layers, 8, 128, 0, 128, "half",
                    500000.0, True, pool_tokens=n * length, chunks=chunks,
                    requests=[Request(entries, table)], page_size=ps, n_phys_pages=n_pages)


def config3(seed: int = 0, n_layers: int = 32, n_requests: int = 64,
            n_chunks: int = 256) -> Workload:
    """Batched RAG: a pool of 256 chunks of 128..4096 tokens, bf16, 32 layers,
    8 KV heads x 128; 64 requests stitching 4..16 pool chunks each, drawn with
    replacement in random order, behind prefixes of 32..512 tokens; paged
    destination (16-token pages from one global random permutation)."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(128, 4096, size=n_chunks, endpoint=True)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]])
    chunks = [Chunk(int(s), int(n)) for s, n in zip(starts, lens)]
    ps = 16
    reqs_entries, reqs_pages = [], []
    for _ in range(n_requests):
        k = int(rng.integers(4, 16, endpoint=True))
        ids = rng.integers(0, n_chunks, size=k)
        pos = int(rng.integers(32, 512, endpoint=True))
        entries = []
        for c in ids:
            entries.append(Entry(int(c), pos, int(lens[c]), 0))
            pos += int(lens[c])
        reqs_entries.append(entries)
        reqs_pages.append(-(-pos // ps))
    total_pages = int(sum(reqs_pages))
    perm = rng.permutation(total_pages).astype(np.int32)
    requests, at = [], 0
    for entries, npg in zip(reqs_entries, reqs_pages):
        requests.append(Request(entries, perm[at:at + npg].copy()))
        at += npg
    return Workload("batched RAG paged", "bf16", n_layers, 8, 128, 0, 128, "half", 500000.0,
                    True, pool_tokens=int(lens.sum()), chunks=chunks, requests=requests,
                    page_size=ps, n_phys_pages=total_pages)


def repeat_heavy(seed: int, dtype: str = "bf16", style: str = "half", n_layers: int = 2,
                 n_chunks: int = 24, n_requests: int = 20, max_len: int = 300,
                 page_size: int = 16) -> Workload:
    """Batched RAG in small: a pool of n_chunks chunks of ragged length
    (1..max_len), n_requests requests each placing 3..8 of them drawn with
    replacement (so every chunk is placed several times, at offsets with every
    residue modulo the page), behind ragged prefixes, with recompute_k of 0,
    1 or a random part of the entry and entries that place only a prefix of
    their chunk; paged destination from one global random permutation."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, max_len, size=n_chunks, endpoint=True)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]])
    chunks = [Chunk(int(s), int(n)) for s, n in zip(starts, lens)]
    reqs_entries, reqs_pages = [], []
    for _ in range(n_requests):
        k = int(rng.integers(3, 8, endpoint=True))
        ids = rng.integers(0, n_chunks, size=k)
        pos = int(rng.integers(0, 40))
        entries = []
        for c in ids:
            ln = int(lens[c]) if rng.random() < 0.8 else int(rng.integers(1, lens[c], endpoint=True))
            rk = int(rng.choice([0, 0, 1, int(rng.integers(0, ln + 1))]))
            entries.append(Entry(int(c), pos, ln, rk))
            pos += ln + int(rng.integers(0, 5))
        reqs_entries.append(entries)
        reqs_pages.append(-(-pos // page_size))
    total_pages = int(sum(reqs_pages))
    perm = rng.permutation(total_pages).astype(np.int32)
    requests, at = [], 0
    for entries, npg in zip(reqs_entries, reqs_pages):
        requests.append(Request(entries, perm[at:at + npg].copy()))
        at += npg
    return Workload(f"repeat heavy {seed}", dtype, n_layers, 2, 128, 0, 128, style, 500000.0,
                    True, pool_tokens=int(lens.sum()), chunks=chunks, requests=requests,
                    page_size=page_size, n_phys_pages=total_pages)


def config4(seed: int = 0, n_layers: int = 61) -> Workload:
    """MLA (DeepSeek-V3 shape): 61 layers, one 576-wide latent row per token
    (512 content dims copied, 64 rotary dims rotated, theta 1e4), bf16;
    16 chunks x 4096 tokens in random order at random offsets (the first at
    position 0 with its first 32 tokens left for recompute, the others
    separated by gaps of 0..512 inline tokens); contiguous destination."""
    rng = np.random.default_rng(seed)
    n, length = 16, 4096
    chunks = [Chunk(i * length, length) for i in range(n)]
    order = rng.permutation(n)
    gaps = rng.integers(0, 512, size=n - 1, endpoint=True)
    entries, pos = [], 0
    for j, c in enumerate(order):
        entries.append(Entry(int(c), pos, length, 32 if j == 0 else 0))
        pos += length + (int(gaps[j]) if j < n - 1 else 0)
    return Workload("deepseek-v3 MLA 16x4096", "bf16", n_layers, 1, 576, 512, 64, "half",
                    10000.0, False, pool_tokens=n * length, chunks=chunks,
                    requests=[Request(entries)], capacity=pos)


def config5(seed: int = 0, n_layers: int = 36) -> Workload:
    """Long-context in-place mode, Qwen3-8B shape: 36 layers, 8 KV heads x 128,
    theta 1e6, bf16; 64 chunks x 2048 tokens forming one 131072-token
    prompt, keys rotated in place by per-chunk shifts drawn from
    [-65536, 65536]; the first 16 tokens of each chunk left alone."""
    rng = np.random.default_rng(seed)
    n, length = 64, 2048
    deltas = rng.integers(-65536, 65536, size=n, endpoint=True)
    segs = [Segment(i * length, length, int(d), 16) for i, d in enumerate(deltas)]
    return Workload("qwen3-8b in-place 131072", "bf16", n_layers, 8, 128, 0, 128, "half",
                    1000000.0, False, inplace=True, n_tokens=n * length, segments=segs)


CONFIGS = {1: config1, 2: config2, 3: config3, 4: config4, 5: config5}


def config5_paged_cow(seed: int = 0, n_layers: int = 36, n_shared: int = 16):
    """The long-context in-place workload on a paged pool: Qwen3-8B shape
    (36 layers, 8 KV heads x 128, theta 1e6, bf16), 64 chunks x 2048 tokens
    in 16-token pages placed by a random permutation of the pool, each
    chunk one segment shifted by a draw from [-65536, 65536] with the first
    16 tokens left alone.  n_shared chunks (a random subset) are shared with
    other requests: their pages are copied to fresh pages and turned there;
    the other chunks are turned in place.  Returns (workload fields,
    n_phys_pages, segments)."""
    rng = np.random.default_rng(seed)
    n, length, ps = 64, 2048, 16
    npg = length // ps
    deltas = rng.integers(-65536, 65536, size=n, endpoint=True)
    shared = set(int(c) for c in rng.choice(n, size=n_shared, replace=False))
    n_phys = n * npg + n_shared * npg
    perm = [int(x) for x in rng.permutation(n_phys)]
    take = iter(perm)
    segs = []
    for c in range(n):
        pages = tuple(next(take) for _ in range(npg))
        cow = tuple(next(take) for _ in range(npg)) if c in shared else None
        segs.append(PageSegment(pages, cow, int(deltas[c]), 0, length, 16))
    wl = Workload("qwen3-8b paged in-place 131072", "bf16", n_layers, 8, 128, 0, 128, "half",
                  1000000.0, True, page_size=ps, n_phys_pages=n_phys)
    return wl, n_phys, segs


def paged_cow_case(seed: int, dtype: str = "bf16", style: str = "half", mla: bool = False,
                   n_layers: int = 2, page_size: int = 16, n_chunks: int = 4, max_len: int = 70,
                   share: float = 0.5, delta_range: int = 5000):
    """A small seeded pic_rotate_paged problem: chunks of ragged length sit
    in physical pages of a pool (a random permutation), starting at a random
    slot of their first page.  A chunk is shared with probability `share`:
    then 2..3 segments (requests) map it, each copying every page to fresh
    target pages with its own shift; a private chunk has one segment that
    copies each page with probability 0.3 (a block some other request holds)
    and turns the rest in place.  Returns (workload fields for the shape,
    n_phys_pages, segments)."""
    rng = np.random.default_rng(seed)
    if mla:
        heads, row, roff, rdim, has_v, theta = 1, 576, 512, 64, False, 10000.0
    else:
        heads, row, roff, rdim, has_v, theta = 2, 128, 0, 128, True, 500000.0
    chunks = []
    for _ in range(n_chunks):
        first = int(rng.integers(0, page_size))
        length = int(rng.integers(1, max_len + 1))
        chunks.append((first, length, -(-(first + length) // page_size)))
    shared = [bool(rng.random() < share) for _ in chunks]
    n_refs = [int(rng.integers(2, 4)) if sh else 1 for sh in shared]
    n_pages = sum(c[2] for c in chunks)
    n_targets = sum(c[2] * k for c, k in zip(chunks, n_refs))
    n_phys = n_pages + n_targets + int(rng.integers(0, 5))
    perm = [int(x) for x in rng.permutation(n_phys)]
    take = iter(perm)
    segs = []
    for (first, length, npg), sh, k in zip(chunks, shared, n_refs):
        pages = tuple(next(take) for _ in range(npg))
        for _ in range(k):
            if sh:
                cow = tuple(next(take) for _ in range(npg))
            else:
                cow = tuple(next(take) if rng.random() < 0.3 else -1 for _ in range(npg))
                if all(c < 0 for c in cow) and rng.random() < 0.5:
                    cow = None
            delta = 0 if rng.random() < 0.1 else int(rng.integers(-delta_range, delta_range + 1))
            rk = int(rng.choice([0, 0, 1, length, int(rng.integers(0, length + 1))]))
            segs.append(PageSegment(pages, cow, delta, first, length, rk))
    order = [int(i) for i in rng.permutation(len(segs))]
    segs = [segs[i] for i in order]
    wl = Workload(f"paged cow {seed}", dtype, n_layers, heads, row, roff, rdim, style, theta,
                  has_v, page_size=page_size, n_phys_pages=n_phys)
    return wl, n_phys, segs


def decode_batch(seed: int = 0, n_requests: int = 16, n_layers: int = 32) -> Workload:
    """A decode batch over stitched contexts, Llama-3-8B shape: n_requests
    requests, each built like the 8 x 2048 paged request (its own 8 chunks
    in a seeded random order behind a 128-token prefix, the first 32 tokens
    of every chunk left for recompute), whose whole 16,512-position context
    is attended; 16-token pages from one global random permutation.  The
    chunks are distinct per request, so no pool row is read twice."""
    rng = np.random.default_rng(seed)
    n, length, prefix, ps = 8, 2048, 128, 16
    chunks = [Chunk(i * length, length) for i in range(n * n_requests)]
    per = (prefix + n * length) // ps
    perm = rng.permutation(per * n_requests).astype(np.int32)
    requests = []
    for r in range(n_requests):
        order = rng.permutation(n) + n * r
        entries = [Entry(int(c), prefix + j * length, length, 32) for j, c in enumerate(order)]
        requests.append(Request(entries, perm[r * per:(r + 1) * per].copy(),
                                prefix + n * length))
    return Workload("llama3-8b decode batch", "bf16", n_layers, 8, 128, 0, 128, "half",
                    500000.0, True, pool_tokens=n * length * n_requests, chunks=chunks,
                    requests=requests, page_size=ps, n_phys_pages=per * n_requests)


def mla_decode_batch(seed: int = 0, n_requests: int = 16, n_layers: int = 61,
                     page_size: int = 64) -> Workload:
    """A decode batch over stitched MLA contexts, DeepSeek-V3 shape (576-wide
    latent rows: 512 content + 64 rotary dims, theta 1e4): each request
    places its own 8 chunks x 2048 tokens in a seeded random order behind a
    128-token prefix, the first 32 tokens of every chunk left for recompute,
    and attends its whole 16,512-position context; pages of 64 tokens from
    one global random permutation."""
    rng = np.random.default_rng(seed)
    n, length, prefix, ps = 8, 2048, 128, page_size
    chunks = [Chunk(i * length, length) for i in range(n * n_requests)]
    per = -(-(prefix + n * length) // ps)
    perm = rng.permutation(per * n_requests).astype(np.int32)
    requests = []
    for r in range(n_requests):
        order = rng.permutation(n) + n * r
        entries = [Entry(int(c), prefix + j * length, length, 32) for j, c in enumerate(order)]
        requests.append(Request(entries, perm[r * per:(r + 1) * per].copy(),
                                prefix + n * length))
    return Workload("deepseek-v3 MLA decode batch", "bf16", n_layers, 1, 576, 512, 64, "half",
                    10000.0, False, pool_tokens=n * length * n_requests, chunks=chunks,
                    requests=requests, page_size=ps, n_phys_pages=per * n_requests)


def with_paged_pool(wl: Workload, page_size: int = 16, seed: int = 0,
                    first_offsets: bool = False, spare_pages: int = 0) -> Workload:
    """The same placements with the chunks kept in a paged pool (the block
    pool of a PagedAttention runtime): every chunk gets its own pages, drawn
    from one random permutation of the pool's pages.  With first_offsets a
    chunk may start part-way into its first page."""
    rng = np.random.default_rng(seed + 7919)
    offs = [int(rng.integers(0, page_size)) if first_offsets else 0 for _ in wl.chunks]
    need = [-(-(o + c.length) // page_size) for o, c in zip(offs, wl.chunks)]
    total = int(sum(need)) + spare_pages
    perm = rng.permutation(total).astype(np.int32)
    chunks, at = [], 0
    for o, n, c in zip(offs, need, wl.chunks):
        chunks.append(Chunk(o, c.length, c.base_pos, perm[at:at + n].copy()))
        at += n
    return replace(wl, name=wl.name + " (paged pool)", chunks=chunks, pool_tokens=0,
                   src_page_size=page_size, src_n_pages=total)


def random_small(seed: int, dtype: str = "bf16", style: str = "half", paged: bool = False,
                 mla: bool = False, n_requests: int = 2, n_layers: int = 2,
                 max_len: int = 150, deltas=None, dims=None) -> Workload:
    """A small random stitch problem with ragged chunk lengths, gaps, shared
    and partial chunks, several requests and varied recompute_k.  dims =
    (heads, row_dim, rope_offset, rope_dim) overrides the GQA row shape."""
    rng = np.random.default_rng(seed)
    if mla:
        heads, row, roff, rdim, has_v, theta = 1, 576, 512, 64, False, 10000.0
    else:
        heads, row, roff, rdim, has_v, theta = 2, 128, 0, 128, True, 500000.0
    if dims is not None:
        heads, row, roff, rdim = dims
    n_chunks = int(rng.integers(2, 6))
    lens = rng.integers(1, max_len, size=n_chunks, endpoint=True)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]])
    bases = rng.integers(0, 3, size=n_chunks) * rng.integers(0, 50, size=n_chunks)
    chunks = [Chunk(int(s), int(n), int(b)) for s, n, b in zip(starts, lens, bases)]
    ps = int(rng.choice([4, 16])) if paged else 0
    reqs_entries, spans = [], []
    for _ in range(n_requests):
        k = int(rng.integers(1, 5))
        pos = int(rng.integers(0, 40))
        entries = []
        for _ in range(k):
            c = int(rng.integers(0, n_chunks))
            ln = int(rng.integers(1, lens[c], endpoint=True))
            rk = int(rng.choice([0, 0, 1, ln, int(rng.integers(0, ln + 1))]))
            if deltas is not None:
                # a chunk record of its own, cached where this shift is wanted
                d = int(rng.choice(deltas))
                chunks.append(Chunk(chunks[c].token_start, chunks[c].length, pos - d))
                c = len(chunks) - 1
            entries.append(Entry(c, pos, ln, rk))
            pos += ln + int(rng.integers(0, 9))
        reqs_entries.append(entries)
        spans.append(pos + int(rng.integers(0, 5)))
    if paged:
        pages = [-(-s // ps) for s in spans]
        total = int(sum(pages)) + int(rng.integers(0, 4))
        perm = rng.permutation(total).astype(np.int32)
        requests, at = [], 0
        for entries, npg in zip(reqs_entries, pages):
            requests.append(Request(entries, perm[at:at + npg].copy()))
            at += npg
        return Workload(f"random{seed}", dtype, n_layers, heads, row, roff, rdim, style, theta,
                        has_v, pool_tokens=int(lens.sum()), chunks=chunks, requests=requests,
                        page_size=ps, n_phys_pages=total)
    return Workload(f"random{seed}", dtype, n_layers, heads, row, roff, rdim, style, theta,
                    has_v, pool_tokens=int(lens.sum()), chunks=chunks,
                    requests=[Request(e) for e in reqs_entries], capacity=int(max(spans)))


def layers_per_launch(wl: Workload, free_bytes: int, margin: int = 6 << 30) -> int:
    """The most layers (a divisor of wl.n_layers) whose destination fits in
    free_bytes beside the whole pool (K and V, all layers) and a margin: the
    layer-group size of a stitch whose pool stays resident and whose
    destination is reused by each group's launch."""
    row = wl.n_heads * wl.row_dim * wl.esize * (2 if wl.has_v else 1)
    pool = wl.n_layers * (wl.pool_tokens if not wl.src_page_size else
                          wl.src_n_pages * wl.src_page_size) * row
    dst_layer = (wl.n_phys_pages * wl.page_size if wl.page_size else
                 len(wl.requests) * wl.capacity) * row
    for g in range(wl.n_layers, 0, -1):
        if wl.n_layers % g == 0 and pool + g * dst_layer + margin <= free_bytes:
            return g
    return 0


# ------------------------------------------------------------ token streams

# Mean content-defined chunk length of the chunking workloads: a boundary
# wherever the rolling hash falls below 2^64 / 256 (the pages give no value).
CDC_THRESHOLD = 1 << 56
LLAMA3_VOCAB = 128256


@dataclass
class TokenStream:
    tokens: np.ndarray          # int32: every request's prompt, back to back
    docs: List[np.ndarray]      # the document pool (int32 token ids)
    request_starts: np.ndarray  # first token of each request in `tokens`
    placements: List[tuple]     # (doc id, first token in `tokens`, edited position or -1)


def rag_token_stream(seed: int = 0, n_docs: int = 256, doc_len=(128, 4096), n_requests: int = 64,
                     per_request=(4, 16), prefix=(32, 512), vocab: int = LLAMA3_VOCAB,
                     edit_prob: float = 0.0) -> TokenStream:
    """Prompts of batched RAG requests as one token stream: a pool of
    documents with lengths uniform in doc_len, and per request a fresh
    prefix (system prompt and query) of U{prefix} tokens followed by U{per_request}
    documents drawn with replacement in random order (the shape of the
    batched-RAG stitch workload).  With edit_prob > 0 a placed document has,
    with that probability, one token replaced (the uncontrolled traffic the
    fixed-window fallback recovers from).  Token ids are uniform in [0, vocab)."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(doc_len[0], doc_len[1], n_docs, endpoint=True)
    docs = [rng.integers(0, vocab, int(n)).astype(np.int32) for n in lens]
    parts, starts, placements, at = [], [], [], 0
    for _ in range(n_requests):
        starts.append(at)
        pre = rng.integers(0, vocab, int(rng.integers(prefix[0], prefix[1], endpoint=True)))
        parts.append(pre.astype(np.int32))
        at += len(pre)
        for d in rng.integers(0, n_docs, int(rng.integers(per_request[0], per_request[1],
                                                           endpoint=True))):
            doc = docs[int(d)]
            edit = -1
            if edit_prob > 0 and rng.random() < edit_prob:
                doc = doc.copy()
                edit = int(rng.integers(0, len(doc)))
                doc[edit] = (int(doc[edit]) + 1 + int(rng.integers(0, vocab - 1))) % vocab
            placements.append((int(d), at, edit))
            parts.append(doc)
            at += len(doc)
    tokens = np.concatenate(parts).astype(np.int32) if parts else np.zeros(0, np.int32)
    return TokenStream(tokens, docs, np.asarray(starts, np.int64), placements)


def random_tokens(n: int, seed: int, vocab: int = LLAMA3_VOCAB, signed: bool = False) -> np.ndarray:
    """n uniform token ids (or, signed, uniform over all int32 values)."""
    rng = np.random.default_rng(seed)
    if signed:
        return rng.integers(-2 ** 31, 2 ** 31, n, dtype=np.int64).astype(np.int32)
    return rng.integers(0, vocab, n).astype(np.int32)


# ------------------------------------------------------------------- values

def _torch():
    import torch
    return torch


def storage_torch_dtype(dtype: str):
    torch = _torch()
    return {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]


def normal_values(shape, dtype: str, seed: int, device="cpu"):
    """N(0, 1) values of `shape` rounded to the storage type (a torch tensor),
    drawn one leading slice at a time so large tensors need no fp32 copy."""
    torch = _torch()
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    out = torch.empty(shape, dtype=storage_torch_dtype(dtype), device=device)
    for i in range(shape[0]):
        out[i].copy_(torch.randn(shape[1:], generator=gen, device=device, dtype=torch.float32))
    return out


def pool_values(wl: Workload, seed: int = 0, device="cpu"):
    """(pool_k, pool_v) for a copy-mode workload; pool_v is None without V."""
    k = normal_values(wl.pool_shape(), wl.dtype, seed, device)
    v = normal_values(wl.pool_shape(), wl.dtype, seed + 1, device) if wl.has_v else None
    return k, v


def sentinel_like(shape, dtype: str, device="cpu"):
    """A destination tensor filled with the sentinel bit pattern."""
    torch = _torch()
    if dtype == "f32":
        bits = torch.full(shape, SENTINEL_BITS["f32"] - (1 << 32), dtype=torch.int32,
                          device=device) if SENTINEL_BITS["f32"] >= (1 << 31) else \
            torch.full(shape, SENTINEL_BITS["f32"], dtype=torch.int32, device=device)
        return bits.view(torch.float32)
    bits = torch.full(shape, SENTINEL_BITS["bf16"], dtype=torch.int16, device=device)
    return bits.view(torch.bfloat16)


def to_host(t) -> np.ndarray:
    """A torch tensor's storage as numpy: float32 values, or bf16 as uint16
    bit patterns (no arithmetic; the layout the oracle reads)."""
    torch = _torch()
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()
