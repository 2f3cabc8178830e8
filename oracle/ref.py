"""ctypes wrapper around the fp64 C oracle (test infrastructure only).

Only the test suite, the package smoke check and the benchmark's CPU
baseline may import this module.  It does not import the HIP library or
its binding, and the HIP library does not import it.

Inputs are numpy arrays in the oracle's dense layouts (see pic_oracle.c):
f32 storage as float32, bf16 storage as uint16 bit patterns, and the
oracle-only f64 storage as float64.  Workload descriptions are read by
attribute (dtype, n_layers, n_heads, row_dim, rope_offset, rope_dim, style,
theta, inv_freq, has_v, pool_tokens, chunks, requests, page_size, capacity,
n_phys_pages, n_tokens, segments) so any object with those fields works.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(HERE, "liboracle.so")

DTYPES = {"f32": 0, "bf16": 1, "f64": 2}
NUMPY_STORAGE = {"f32": np.float32, "bf16": np.uint16, "f64": np.float64}
STYLES = {"half": 0, "interleaved": 1}
STATUS = {0: "ok", 1: "bad_arg", 2: "range", 3: "overlap"}

_i32p = C.POINTER(C.c_int32)
_i64p = C.POINTER(C.c_int64)
_f64p = C.POINTER(C.c_double)


class _StitchProblem(C.Structure):
    _fields_ = [("dtype", C.c_int32), ("n_layers", C.c_int32), ("n_heads", C.c_int32),
                ("row_dim", C.c_int32), ("rope_offset", C.c_int32), ("rope_dim", C.c_int32),
                ("style", C.c_int32), ("has_v", C.c_int32), ("theta", C.c_double),
                ("inv_freq", _f64p), ("pool_tokens", C.c_int64), ("src_page_size", C.c_int32),
                ("src_num_pages", C.c_int64), ("chunk_pages", _i32p),
                ("chunk_page_table", _i32p), ("n_chunks", C.c_int32),
                ("chunk_start", _i64p), ("chunk_base", _i64p), ("chunk_len", _i32p),
                ("n_requests", C.c_int32), ("req_entries", _i32p), ("ent_chunk", _i32p),
                ("ent_dst", _i64p), ("ent_len", _i32p), ("ent_k", _i32p),
                ("page_size", C.c_int32), ("capacity", C.c_int64),
                ("n_phys_pages", C.c_int64), ("req_pages", _i32p), ("page_table", _i32p)]


class _InplaceProblem(C.Structure):
    _fields_ = [("dtype", C.c_int32), ("n_layers", C.c_int32), ("n_heads", C.c_int32),
                ("row_dim", C.c_int32), ("rope_offset", C.c_int32), ("rope_dim", C.c_int32),
                ("style", C.c_int32), ("pad_", C.c_int32), ("theta", C.c_double),
                ("inv_freq", _f64p), ("n_tokens", C.c_int64), ("n_segments", C.c_int32),
                ("pad2_", C.c_int32), ("seg_start", _i64p), ("seg_delta", _i64p),
                ("seg_len", _i32p), ("seg_k", _i32p)]


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIBRARY):
            from . import build as _build
            _build.build()
        lib = C.CDLL(LIBRARY)
        lib.orc_stitch.restype = C.c_int
        lib.orc_stitch.argtypes = [C.POINTER(_StitchProblem), C.c_void_p, C.c_void_p,
                                   C.c_void_p, C.c_void_p, C.c_int, C.c_int]
        lib.orc_validate_stitch.restype = C.c_int
        lib.orc_validate_stitch.argtypes = [C.POINTER(_StitchProblem), C.c_int, C.c_int]
        lib.orc_rotate_inplace.restype = C.c_int
        lib.orc_rotate_inplace.argtypes = [C.POINTER(_InplaceProblem), C.c_void_p, C.c_int,
                                           C.c_int]
        lib.orc_validate_inplace.restype = C.c_int
        lib.orc_validate_inplace.argtypes = [C.POINTER(_InplaceProblem), C.c_int, C.c_int]
        lib.orc_round_bf16.restype = C.c_uint16
        lib.orc_round_bf16.argtypes = [C.c_double]
        lib.orc_round_bf16_array.restype = None
        lib.orc_round_bf16_array.argtypes = [_f64p, C.POINTER(C.c_uint16), C.c_int64]
        lib.orc_inv_freq.restype = C.c_double
        lib.orc_inv_freq.argtypes = [C.c_double, C.c_int, C.c_int]
        _lib = lib
    return _lib


def _ptr(a, ctype):
    return a.ctypes.data_as(C.POINTER(ctype)) if a is not None else None


def _stitch_problem(wl, dtype=None):
    """Build the C problem struct; returns (struct, keep-alive arrays)."""
    dt = dtype or wl.dtype
    keep = []

    def arr(values, npdt):
        a = np.ascontiguousarray(np.asarray(values, dtype=npdt))
        if a.size == 0:
            a = np.zeros(1, dtype=npdt)
        keep.append(a)
        return a

    src_ps = getattr(wl, "src_page_size", 0)
    tables = [np.asarray(c.page_table if c.page_table is not None else [], dtype=np.int32)
              for c in wl.chunks] if src_ps else []
    chunk_pages = arr([len(t) for t in tables] if src_ps else [0] * len(wl.chunks), np.int32)
    chunk_page_table = arr(np.concatenate(tables) if tables else [], np.int32)
    chunk_start = arr([c.token_start for c in wl.chunks], np.int64)
    chunk_base = arr([c.base_pos for c in wl.chunks], np.int64)
    chunk_len = arr([c.length for c in wl.chunks], np.int32)
    req_entries = arr([len(r.entries) for r in wl.requests], np.int32)
    ents = [e for r in wl.requests for e in r.entries]
    ent_chunk = arr([e.chunk_id for e in ents], np.int32)
    ent_dst = arr([e.dst_offset for e in ents], np.int64)
    ent_len = arr([e.length for e in ents], np.int32)
    ent_k = arr([e.recompute_k for e in ents], np.int32)
    paged = wl.page_size > 0
    req_pages = arr([len(r.page_table) if paged else 0 for r in wl.requests], np.int32)
    page_table = arr(np.concatenate([np.asarray(r.page_table, dtype=np.int32)
                                     for r in wl.requests]) if paged and wl.requests else [],
                     np.int32)
    inv = arr(wl.inv_freq, np.float64) if getattr(wl, "inv_freq", None) is not None else None
    p = _StitchProblem(DTYPES[dt], wl.n_layers, wl.n_heads, wl.row_dim, wl.rope_offset,
                       wl.rope_dim, STYLES[wl.style], int(bool(wl.has_v)), float(wl.theta),
                       _ptr(inv, C.c_double), wl.pool_tokens, src_ps,
                       getattr(wl, "src_n_pages", 0), _ptr(chunk_pages, C.c_int32),
                       _ptr(chunk_page_table, C.c_int32), len(wl.chunks),
                       _ptr(chunk_start, C.c_int64), _ptr(chunk_base, C.c_int64),
                       _ptr(chunk_len, C.c_int32), len(wl.requests),
                       _ptr(req_entries, C.c_int32), _ptr(ent_chunk, C.c_int32),
                       _ptr(ent_dst, C.c_int64), _ptr(ent_len, C.c_int32),
                       _ptr(ent_k, C.c_int32), wl.page_size, wl.capacity, wl.n_phys_pages,
                       _ptr(req_pages, C.c_int32), _ptr(page_table, C.c_int32))
    return p, keep


def _inplace_problem(wl, dtype=None):
    dt = dtype or wl.dtype
    keep = []

    def arr(values, npdt):
        a = np.ascontiguousarray(np.asarray(values, dtype=npdt))
        if a.size == 0:
            a = np.zeros(1, dtype=npdt)
        keep.append(a)
        return a

    seg_start = arr([s.token_start for s in wl.segments], np.int64)
    seg_delta = arr([s.delta for s in wl.segments], np.int64)
    seg_len = arr([s.length for s in wl.segments], np.int32)
    seg_k = arr([s.recompute_k for s in wl.segments], np.int32)
    inv = arr(wl.inv_freq, np.float64) if getattr(wl, "inv_freq", None) is not None else None
    p = _InplaceProblem(DTYPES[dt], wl.n_layers, wl.n_heads, wl.row_dim, wl.rope_offset,
                        wl.rope_dim, STYLES[wl.style], 0, float(wl.theta),
                        _ptr(inv, C.c_double), wl.n_tokens, len(wl.segments), 0,
                        _ptr(seg_start, C.c_int64), _ptr(seg_delta, C.c_int64),
                        _ptr(seg_len, C.c_int32), _ptr(seg_k, C.c_int32))
    return p, keep


def _check_array(a, dt, shape, name):
    if a is None:
        return
    if a.dtype != NUMPY_STORAGE[dt] or not a.flags.c_contiguous:
        raise TypeError(f"{name}: expected C-contiguous {NUMPY_STORAGE[dt].__name__}")
    if tuple(a.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {a.shape}, expected {shape}")


def validate_stitch(wl, layer_begin=0, layer_end=None) -> str:
    """The oracle's verdict on a copy-mode problem: 'ok', 'bad_arg', 'range'
    or 'overlap'."""
    p, keep = _stitch_problem(wl)
    le = wl.n_layers if layer_end is None else layer_end
    return STATUS[_load().orc_validate_stitch(C.byref(p), layer_begin, le)]


def validate_inplace(wl, layer_begin=0, layer_end=None) -> str:
    p, keep = _inplace_problem(wl)
    le = wl.n_layers if layer_end is None else layer_end
    return STATUS[_load().orc_validate_inplace(C.byref(p), layer_begin, le)]


def stitch(wl, pool_k, pool_v, dst_k, dst_v, layer_begin=0, layer_end=None, dtype=None,
           layer_base=0) -> str:
    """Stitch layers [layer_begin, layer_end) into dst_k / dst_v (modified in
    place).  The arrays hold layers [layer_base, layer_base + n) of the
    workload, so a caller can pass one layer at a time.  Returns the
    oracle's status string; nothing is written unless it is 'ok'."""
    dt = dtype or wl.dtype
    le = wl.n_layers if layer_end is None else layer_end
    n = pool_k.shape[0]
    if not (layer_base <= layer_begin <= le <= layer_base + n):
        raise ValueError("layer range outside the arrays given")
    sub = _Layers(wl, n)
    p, keep = _stitch_problem(sub, dt)
    if getattr(wl, "src_page_size", 0):
        pshape = (n, wl.src_n_pages, wl.src_page_size, wl.n_heads, wl.row_dim)
    else:
        pshape = (n, wl.pool_tokens, wl.n_heads, wl.row_dim)
    _check_array(pool_k, dt, pshape, "pool_k")
    dshape = ((n, wl.n_phys_pages, wl.page_size, wl.n_heads, wl.row_dim) if wl.page_size
              else (n, len(wl.requests), wl.capacity, wl.n_heads, wl.row_dim))
    _check_array(dst_k, dt, dshape, "dst_k")
    if wl.has_v:
        _check_array(pool_v, dt, pool_k.shape, "pool_v")
        _check_array(dst_v, dt, dshape, "dst_v")
    st = _load().orc_stitch(C.byref(p), pool_k.ctypes.data,
                            pool_v.ctypes.data if wl.has_v else None, dst_k.ctypes.data,
                            dst_v.ctypes.data if wl.has_v else None,
                            layer_begin - layer_base, le - layer_base)
    return STATUS[st]


def rotate_inplace(wl, buf_k, layer_begin=0, layer_end=None, dtype=None, layer_base=0) -> str:
    """Rotate, in place, the segments of buf_k (layers [layer_base, ...))."""
    dt = dtype or wl.dtype
    le = wl.n_layers if layer_end is None else layer_end
    n = buf_k.shape[0]
    if not (layer_base <= layer_begin <= le <= layer_base + n):
        raise ValueError("layer range outside the array given")
    p, keep = _inplace_problem(_Layers(wl, n), dt)
    _check_array(buf_k, dt, (n, wl.n_tokens, wl.n_heads, wl.row_dim), "buf_k")
    st = _load().orc_rotate_inplace(C.byref(p), buf_k.ctypes.data, layer_begin - layer_base,
                                    le - layer_base)
    return STATUS[st]


def validate_rotate_paged(page_size, n_phys_pages, segments) -> str:
    """The status pic_rotate_paged gives a set of paged segments, checked
    here from its stated rules (after the shape checks): first every
    segment's counts (bad_arg) and positions and page ids (range; the
    logical positions its pages span must stay below 2^31), then the clashes
    between segments (overlap)."""
    if page_size < 1 or n_phys_pages < 1:
        return "bad_arg"
    for sg in segments:
        if not (0 <= sg.first < page_size) or sg.length < 1:
            return "range"
        if -(-(sg.first + sg.length) // page_size) * page_size > 2 ** 31 - 1:
            return "range"  # the pages' logical positions must fit int32
        if not (0 <= sg.recompute_k <= sg.length):
            return "range"
        n_pages = -(-(sg.first + sg.length) // page_size)
        cow = sg.cow if sg.cow is not None else [-1] * len(sg.pages)
        if len(sg.pages) != n_pages or len(cow) != n_pages:
            return "bad_arg"
        for pg, cw in zip(sg.pages, cow):
            if not (0 <= pg < n_phys_pages) or not (-1 <= cw < n_phys_pages):
                return "range"
    turned_slots, targets, sources, turned_pages, all_pages = set(), [], set(), set(), set()
    clash = False
    for sg in segments:
        cow = sg.cow if sg.cow is not None else [-1] * len(sg.pages)
        for i, (pg, cw) in enumerate(zip(sg.pages, cow)):
            all_pages.add(pg)
            if cw >= 0:
                clash |= cw in targets
                targets.append(cw)
                sources.add(pg)
                continue
            # logical positions of the page's turned tokens
            lo = max(sg.first + sg.recompute_k, i * page_size)
            hi = min(sg.first + sg.length, (i + 1) * page_size)
            if sg.delta == 0 or lo >= hi:
                continue
            turned_pages.add(pg)
            for q in range(lo, hi):
                key = (pg, q - i * page_size)
                clash |= key in turned_slots
                turned_slots.add(key)
    if clash or any(t in all_pages for t in targets) or sources & turned_pages:
        return "overlap"
    return "ok"


def rotate_paged(shape, buf_k, buf_v, page_size, segments, layer_begin=0, layer_end=None,
                 dtype=None) -> str:
    """fp64 oracle of pic_rotate_paged on numpy buffers [L][pages][page][H][D]
    (buf_v may be None): every shared page (cow[i] >= 0) is copied whole,
    K and V, to its target page, then every segment's tokens t in
    [recompute_k, length) have their K rotary slice turned by the segment's
    delta where they now live (the copy for a shared page, the page itself
    otherwise), by this oracle's in-place turn.  shape: an object with
    n_layers, n_heads, row_dim, rope_offset, rope_dim, style, theta,
    inv_freq; segments: objects with pages, cow, delta, first, length,
    recompute_k.  Returns the status."""
    from types import SimpleNamespace as NS
    dt = dtype or shape.dtype
    le = shape.n_layers if layer_end is None else layer_end
    st = validate_rotate_paged(page_size, buf_k.shape[1], segments)
    if st != "ok":
        return st
    L = slice(layer_begin, le)
    for sg in segments:  # copies first: no copy source is turned, no target is read
        for pg, cw in zip(sg.pages, sg.cow if sg.cow is not None else [-1] * len(sg.pages)):
            if cw >= 0:
                buf_k[L, cw] = buf_k[L, pg]
                if buf_v is not None:
                    buf_v[L, cw] = buf_v[L, pg]
    for sg in segments:
        if sg.delta == 0:
            continue
        cow = sg.cow if sg.cow is not None else [-1] * len(sg.pages)
        home = [cw if cw >= 0 else pg for pg, cw in zip(sg.pages, cow)]
        where = [(home[(sg.first + t) // page_size], (sg.first + t) % page_size)
                 for t in range(sg.length)]
        rows = np.stack([buf_k[L, p, s] for p, s in where], axis=1)  # [L'][length][H][D]
        sub = NS(dtype=dt, n_layers=rows.shape[0], n_heads=shape.n_heads, row_dim=shape.row_dim,
                 rope_offset=shape.rope_offset, rope_dim=shape.rope_dim, style=shape.style,
                 theta=shape.theta, inv_freq=getattr(shape, "inv_freq", None), n_tokens=sg.length,
                 segments=[NS(token_start=0, length=sg.length, delta=sg.delta,
                              recompute_k=sg.recompute_k)])
        rows = np.ascontiguousarray(rows)
        res = rotate_inplace(sub, rows, 0, rows.shape[0], dtype=dt)
        if res != "ok":
            return res
        for t, (p, s) in enumerate(where):
            buf_k[L, p, s] = rows[:, t]
    return "ok"


def round_bf16(x) -> np.ndarray:
    """bf16 bit patterns of fp64 values, one round-to-nearest-even each."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    out = np.empty(x.shape, dtype=np.uint16)
    _load().orc_round_bf16_array(_ptr(x, C.c_double), _ptr(out, C.c_uint16), x.size)
    return out


def inv_freq(theta: float, rope_dim: int) -> np.ndarray:
    """The oracle's plane frequencies theta_i = theta^(-2i/rope_dim)."""
    lib = _load()
    return np.array([lib.orc_inv_freq(theta, rope_dim, i) for i in range(rope_dim // 2)])


def recompute_ranges(wl):
    """[(request, begin, end)] positions left for the recompute pass: the first
    recompute_k tokens of every entry (empty ranges omitted)."""
    out = []
    for r, req in enumerate(wl.requests):
        for e in req.entries:
            if e.recompute_k > 0:
                out.append((r, e.dst_offset, e.dst_offset + e.recompute_k))
    return out


class _Layers:
    """View of a workload whose arrays hold only `n` layers."""

    def __init__(self, wl, n):
        self._wl = wl
        self.n_layers = n

    def __getattr__(self, name):
        return getattr(self._wl, name)


def _to_f64(a):
    """Storage values (float32, or bf16 as uint16 bits) widened exactly to fp64."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def attend(wl, pool_k, pool_v, cache_k, cache_v, q, layer, scale=None, sink_tokens=0,
           sink_bias=0.0, layer_base=0):
    """Decode attention of every request at `layer`, in fp64 (returns
    [requests][q heads][row_dim] float64).

    A request's context is positions [0, context_len) (0: up to its last
    entry's end).  Positions an entry writes take the chunk's key turned by
    the entry's shift, computed exactly by this oracle's stitch in fp64
    (no rounding to storage), and the chunk's value; every other position
    takes the request's own cache row.  Query head j uses KV head
    j // (num_q_heads / n_heads).  logit_p = scale * q . K_p, plus
    sink_bias on the first sink_tokens positions of every entry placed after
    position 0 (the EPIC Guide's LegoLink listing: -15 on 4 tokens); the
    weights are softmax over the context and the output their weighted sum
    of values (the plain definition of attention).
    """
    from types import SimpleNamespace as NS
    li = layer - layer_base
    H, D = wl.n_heads, wl.row_dim
    R, Hq = q.shape[0], q.shape[1]
    G = Hq // H
    sc = D ** -0.5 if scale is None else scale
    out = np.zeros((R, Hq, D))
    pk64 = _to_f64(pool_k[li:li + 1])
    pv64 = _to_f64(pool_v[li:li + 1])
    for r, rq in enumerate(wl.requests):
        L = rq.context_len or max([e.dst_offset + e.length for e in rq.entries] + [0])
        if L == 0:
            raise ValueError(f"request {r} has an empty context")
        # the request's own cache rows
        pos = np.arange(L)
        if wl.page_size:
            pt = np.asarray(rq.page_table)
            k = _to_f64(cache_k[li][pt[pos // wl.page_size], pos % wl.page_size])
            v = _to_f64(cache_v[li][pt[pos // wl.page_size], pos % wl.page_size])
        else:
            k = _to_f64(cache_k[li][r, :L])
            v = _to_f64(cache_v[li][r, :L])
        # chunk rows, turned exactly: the stitch oracle in fp64 into a scratch request
        cap = max(L, max([e.dst_offset + e.length for e in rq.entries] + [0]))
        sub = NS(dtype="f64", n_layers=1, n_heads=H, row_dim=D, rope_offset=wl.rope_offset,
                 rope_dim=wl.rope_dim, style=wl.style, theta=wl.theta, inv_freq=wl.inv_freq,
                 has_v=True, pool_tokens=wl.pool_tokens, chunks=wl.chunks,
                 src_page_size=getattr(wl, "src_page_size", 0),
                 src_n_pages=getattr(wl, "src_n_pages", 0),
                 requests=[NS(entries=rq.entries, page_table=None)], page_size=0, capacity=cap,
                 n_phys_pages=0)
        sk = np.zeros((1, 1, cap, H, D))
        sv = np.zeros((1, 1, cap, H, D))
        st = stitch(sub, pk64, pv64, sk, sv, 0, 1, dtype="f64")
        if st != "ok":
            raise ValueError(f"request {r}: {st}")
        bias = np.zeros(L)
        for e in rq.entries:
            lo, hi = e.dst_offset + e.recompute_k, min(e.dst_offset + e.length, L)
            if lo < hi:
                k[lo:hi] = sk[0, 0, lo:hi]
                v[lo:hi] = sv[0, 0, lo:hi]
            if e.dst_offset > 0 and sink_tokens > 0:
                bias[e.dst_offset:min(e.dst_offset + sink_tokens, L)] = sink_bias
        qq = _to_f64(q[r])
        for j in range(Hq):
            h = j // G
            logits = sc * (k[:, h, :] @ qq[j]) + bias
            w = np.exp(logits - logits.max())
            out[r, j] = (w @ v[:, h, :]) / w.sum()
    return out


def attend_latent(wl, pool_k, cache_k, q, layer, scale=None, sink_tokens=0, sink_bias=0.0,
                  layer_base=0, dtype=None):
    """Decode attention over MLA latent rows, in fp64 (returns
    [requests][q heads][rope_offset] float64).

    Irminsul (Technical Summary sections 2.1, 2.2 and 4): a latent row is the
    content latent [0, rope_offset) followed by the rotary key; in the
    absorbed form every query head j has a full-width query row, its logit
    at position p is scale * q_j . row_p, and the value of position p is
    the content latent.  row_p is the row this oracle's stitch leaves at p:
    for positions an entry writes, the chunk's row with its rotary key
    turned by the entry's shift and rounded to the storage type (dtype
    'f64': not rounded); for every other position the request's own cache
    row.  Damping as in attend().  The weights are softmax over the context
    and the output their weighted sum of content latents (the plain
    definition of attention).
    """
    from types import SimpleNamespace as NS
    li = layer - layer_base
    D, V = wl.row_dim, wl.rope_offset
    R, Hq = q.shape[0], q.shape[1]
    sc = D ** -0.5 if scale is None else scale
    dt = dtype or wl.dtype
    out = np.zeros((R, Hq, V))
    pk = pool_k[li:li + 1]
    if dt == "f64":
        pk = _to_f64(pk)
    for r, rq in enumerate(wl.requests):
        L = rq.context_len or max([e.dst_offset + e.length for e in rq.entries] + [0])
        if L == 0:
            raise ValueError(f"request {r} has an empty context")
        pos = np.arange(L)
        if wl.page_size:
            pt = np.asarray(rq.page_table)
            k = _to_f64(cache_k[li][pt[pos // wl.page_size], pos % wl.page_size])
        else:
            k = _to_f64(cache_k[li][r, :L])
        cap = max(L, max([e.dst_offset + e.length for e in rq.entries] + [0]))
        sub = NS(dtype=dt, n_layers=1, n_heads=1, row_dim=D, rope_offset=wl.rope_offset,
                 rope_dim=wl.rope_dim, style=wl.style, theta=wl.theta, inv_freq=wl.inv_freq,
                 has_v=False, pool_tokens=wl.pool_tokens, chunks=wl.chunks,
                 src_page_size=getattr(wl, "src_page_size", 0),
                 src_n_pages=getattr(wl, "src_n_pages", 0),
                 requests=[NS(entries=rq.entries, page_table=None)], page_size=0, capacity=cap,
                 n_phys_pages=0)
        sk = np.zeros((1, 1, cap, 1, D), dtype=pk.dtype)
        st = stitch(sub, pk, None, sk, None, 0, 1, dtype=dt)
        if st != "ok":
            raise ValueError(f"request {r}: {st}")
        sk = _to_f64(sk)
        bias = np.zeros(L)
        for e in rq.entries:
            lo, hi = e.dst_offset + e.recompute_k, min(e.dst_offset + e.length, L)
            if lo < hi:
                k[lo:hi] = sk[0, 0, lo:hi]
            if e.dst_offset > 0 and sink_tokens > 0:
                bias[e.dst_offset:min(e.dst_offset + sink_tokens, L)] = sink_bias
        rows = k[:, 0, :]
        qq = _to_f64(q[r])
        for j in range(Hq):
            logits = sc * (rows @ qq[j]) + bias
            w = np.exp(logits - logits.max())
            out[r, j] = (w @ rows[:, :V]) / w.sum()
    return out


def boundary_rows(wl, boundary_k, rows=None):
    """The boundary rows of a plan, in order: (request, entry index, token j,
    position).  Without `rows`: every entry placed after position 0 and
    j < min(k, length), requests in order, each request's entries in the
    order given.  With `rows`: the given (entry, token) pairs, entries
    numbered across the requests in plan order (request by request), in the
    order given; a token outside its entry raises ValueError."""
    if rows is not None:
        flat = [(r, i, e) for r, rq in enumerate(wl.requests) for i, e in enumerate(rq.entries)]
        out = []
        for ent, j in rows:
            r, i, e = flat[int(ent)]
            if not 0 <= int(j) < e.length:
                raise ValueError(f"token {j} outside entry {ent} of length {e.length}")
            out.append((r, i, int(j), e.dst_offset + int(j)))
        return out
    out = []
    for r, rq in enumerate(wl.requests):
        for i, e in enumerate(rq.entries):
            if e.dst_offset > 0:
                for j in range(min(boundary_k, e.length)):
                    out.append((r, i, j, e.dst_offset + j))
    return out


def attend_boundary(wl, pool_k, pool_v, cache_k, cache_v, q, layer, boundary_k, scale=None,
                    sink_tokens=0, sink_bias=0.0, layer_base=0, dtype=None, rows=None):
    """LegoLink's boundary reconnection (EPIC Guide, "2. Sparse Cross-Block
    Reconnection"), in fp64: boundary token j of every entry placed after
    position 0 (its first boundary_k tokens) attends causally to every
    position of its request up to and including its own, p = dst_offset + j:
    the preceding chunks and prefix (the cross-chunk part) and its own
    chunk's earlier tokens.  With `rows`, the given (entry, token) pairs
    instead (any token of any entry, each attending causally up to its own
    position).  q: [boundary rows][q heads][row_dim] in boundary_rows()
    order; returns [boundary rows][q heads][row_dim].

    The context rows are those this oracle's stitch leaves (chunk keys turned
    by the entry's shift and rounded to the storage type; dtype 'f64': not
    rounded), every other position the request's own cache row; query head
    j reads KV head j // (num_q_heads / n_heads); damping as in attend()."""
    from types import SimpleNamespace as NS
    li = layer - layer_base
    H, D = wl.n_heads, wl.row_dim
    Hq = q.shape[1]
    G = Hq // H
    sc = D ** -0.5 if scale is None else scale
    dt = dtype or wl.dtype
    rows = boundary_rows(wl, boundary_k, rows)
    out = np.zeros((len(rows), Hq, D))
    pk, pv = pool_k[li:li + 1], pool_v[li:li + 1]
    if dt == "f64":
        pk, pv = _to_f64(pk), _to_f64(pv)
    ctx = {}
    for r in sorted({row[0] for row in rows}):
        rq = wl.requests[r]
        L = max(e.dst_offset + e.length for e in rq.entries)
        pos = np.arange(L)
        if wl.page_size:
            pt = np.asarray(rq.page_table)
            k = _to_f64(cache_k[li][pt[pos // wl.page_size], pos % wl.page_size])
            v = _to_f64(cache_v[li][pt[pos // wl.page_size], pos % wl.page_size])
        else:
            k = _to_f64(cache_k[li][r, :L])
            v = _to_f64(cache_v[li][r, :L])
        sub = NS(dtype=dt, n_layers=1, n_heads=H, row_dim=D, rope_offset=wl.rope_offset,
                 rope_dim=wl.rope_dim, style=wl.style, theta=wl.theta, inv_freq=wl.inv_freq,
                 has_v=True, pool_tokens=wl.pool_tokens, chunks=wl.chunks,
                 src_page_size=getattr(wl, "src_page_size", 0),
                 src_n_pages=getattr(wl, "src_n_pages", 0),
                 requests=[NS(entries=rq.entries, page_table=None)], page_size=0, capacity=L,
                 n_phys_pages=0)
        sk = np.zeros((1, 1, L, H, D), dtype=pk.dtype)
        sv = np.zeros((1, 1, L, H, D), dtype=pk.dtype)
        st = stitch(sub, pk, pv, sk, sv, 0, 1, dtype=dt)
        if st != "ok":
            raise ValueError(f"request {r}: {st}")
        sk, sv = _to_f64(sk), _to_f64(sv)
        bias = np.zeros(L)
        for e in rq.entries:
            lo, hi = e.dst_offset + e.recompute_k, e.dst_offset + e.length
            if lo < hi:
                k[lo:hi] = sk[0, 0, lo:hi]
                v[lo:hi] = sv[0, 0, lo:hi]
            if e.dst_offset > 0 and sink_tokens > 0:
                bias[e.dst_offset:min(e.dst_offset + sink_tokens, L)] = sink_bias
        ctx[r] = (k, v, bias)
    for b, (r, _, _, p) in enumerate(rows):
        k, v, bias = ctx[r]
        qq = _to_f64(q[b])
        for h in range(H):  # the G query heads of KV head h at once
            logits = sc * (qq[h * G:(h + 1) * G] @ k[:p + 1, h, :].T) + bias[:p + 1]
            w = np.exp(logits - logits.max(axis=1, keepdims=True))
            out[b, h * G:(h + 1) * G] = (w @ v[:p + 1, h, :]) / w.sum(axis=1, keepdims=True)
    return out
