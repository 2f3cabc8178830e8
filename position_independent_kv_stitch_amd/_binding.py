"""ctypes binding of libpic_stitch.so (argument marshalling only).

Every step of the path runs in the HIP library; this module turns torch
tensors into views (pointer + element strides), Python placement tables
into the C structs of ``include/pic_stitch.h``, and torch's current stream
into the stream argument.  There is no fallback: if the library is missing
or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes as C
import os
import time
from typing import Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# PIC_STITCH_LIBRARY selects another build of the same library (same ABI).
LIBRARY = os.environ.get("PIC_STITCH_LIBRARY") or os.path.join(HERE, "libpic_stitch.so")

PIC_OK, PIC_ERR_INVALID_ARG, PIC_ERR_RANGE, PIC_ERR_OVERLAP = 0, 1, 2, 3
PIC_ERR_ALIGN, PIC_ERR_DEVICE, PIC_ERR_NOMEM, PIC_ERR_STATE = 4, 5, 6, 7
STATUS_NAMES = {0: "ok", 1: "invalid_arg", 2: "range", 3: "overlap", 4: "align", 5: "device",
                6: "nomem", 7: "state"}
DTYPES = {"f32": 0, "bf16": 1}
STYLES = {"half": 0, "interleaved": 1}

# every entry point the header declares
EXPORTS = ("pic_plan", "pic_stitch", "pic_rotate_inplace", "pic_rotate_paged", "pic_attend",
           "pic_attend_latent",
           "pic_attend_boundary", "pic_plan_info",
           "pic_plan_ranges", "pic_plan_destroy", "pic_registry_create", "pic_registry_add",
           "pic_registry_destroy", "pic_match", "pic_stream_copy", "pic_rotate_inplace_noalloc",
           "pic_last_error")
FP_KINDS = {"xxh64": 0, "sha256": 1}


class PicError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status
        self.name = STATUS_NAMES.get(status, str(status))


class RopeConfig(C.Structure):
    _fields_ = [("rope_dim", C.c_int32), ("style", C.c_int32), ("theta", C.c_double),
                ("inv_freq", C.POINTER(C.c_double))]


class KvShape(C.Structure):
    _fields_ = [("dtype", C.c_int32), ("num_layers", C.c_int32), ("num_heads", C.c_int32),
                ("row_dim", C.c_int32), ("rope_offset", C.c_int32), ("has_v", C.c_int32)]


class ChunkC(C.Structure):
    _fields_ = [("token_start", C.c_int64), ("base_pos", C.c_int64), ("length", C.c_int32),
                ("n_pages", C.c_int32), ("page_table", C.POINTER(C.c_int32))]


class EntryC(C.Structure):
    _fields_ = [("dst_offset", C.c_int64), ("chunk_id", C.c_int32), ("length", C.c_int32),
                ("recompute_k", C.c_int32), ("reserved", C.c_int32)]


class RequestC(C.Structure):
    _fields_ = [("entries", C.POINTER(EntryC)), ("page_table", C.POINTER(C.c_int32)),
                ("n_entries", C.c_int32), ("n_pages", C.c_int32), ("context_len", C.c_int64)]


class AttendArgs(C.Structure):
    _fields_ = [("q", C.c_void_p), ("q_request_stride", C.c_int64),
                ("q_head_stride", C.c_int64), ("out", C.c_void_p),
                ("out_request_stride", C.c_int64), ("out_head_stride", C.c_int64),
                ("num_q_heads", C.c_int32), ("layer", C.c_int32), ("scale", C.c_float),
                ("sink_tokens", C.c_int32), ("sink_bias", C.c_float), ("reserved", C.c_int32)]


class LatentArgs(C.Structure):
    _fields_ = [("q", C.c_void_p), ("q_request_stride", C.c_int64),
                ("q_head_stride", C.c_int64), ("out", C.c_void_p),
                ("out_request_stride", C.c_int64), ("out_head_stride", C.c_int64),
                ("num_q_heads", C.c_int32), ("layer", C.c_int32), ("scale", C.c_float),
                ("sink_tokens", C.c_int32), ("sink_bias", C.c_float), ("reserved", C.c_int32)]


class BoundaryArgs(C.Structure):
    _fields_ = [("q", C.c_void_p), ("q_row_stride", C.c_int64), ("q_head_stride", C.c_int64),
                ("out", C.c_void_p), ("out_row_stride", C.c_int64),
                ("out_head_stride", C.c_int64), ("num_q_heads", C.c_int32),
                ("layer", C.c_int32), ("scale", C.c_float), ("boundary_k", C.c_int32),
                ("sink_tokens", C.c_int32), ("sink_bias", C.c_float),
                ("rows", C.POINTER(C.c_int32)), ("n_rows", C.c_int32), ("reserved", C.c_int32)]


class Geom(C.Structure):
    _fields_ = [("dst_page_size", C.c_int32), ("src_page_size", C.c_int32),
                ("dst_capacity", C.c_int64), ("dst_num_pages", C.c_int64),
                ("src_num_pages", C.c_int64)]


class KvView(C.Structure):
    _fields_ = [("k", C.c_void_p), ("v", C.c_void_p), ("layer_stride", C.c_int64),
                ("token_stride", C.c_int64), ("head_stride", C.c_int64),
                ("page_stride", C.c_int64), ("request_stride", C.c_int64)]


class SegmentC(C.Structure):
    _fields_ = [("token_start", C.c_int64), ("delta", C.c_int64), ("length", C.c_int32),
                ("recompute_k", C.c_int32)]


class PageSegmentC(C.Structure):
    _fields_ = [("pages", C.POINTER(C.c_int32)), ("cow", C.POINTER(C.c_int32)),
                ("delta", C.c_int64), ("n_pages", C.c_int32), ("first", C.c_int32),
                ("length", C.c_int32), ("recompute_k", C.c_int32)]


class CdcConfig(C.Structure):
    _fields_ = [("threshold", C.c_uint64), ("gear_seed", C.c_uint64), ("fp_seed", C.c_uint64),
                ("fingerprint", C.c_int32), ("window", C.c_int32)]


class MatchRecord(C.Structure):
    _fields_ = [("start", C.c_int64), ("length", C.c_int32), ("level", C.c_int32),
                ("chunk_id", C.c_int32), ("reserved", C.c_int32), ("fp", C.c_uint8 * 32)]


# numpy view of pic_match_t records
MATCH_DTYPE = np.dtype([("start", "<i8"), ("length", "<i4"), ("level", "<i4"),
                        ("chunk_id", "<i4"), ("reserved", "<i4"), ("fp", "u1", (32,))])


class PlanInfo(C.Structure):
    _fields_ = [(n, C.c_int64) for n in (
        "n_requests", "n_entries", "n_tiles", "tokens_written", "tokens_masked",
        "pool_tokens_required", "bytes_read_per_layer", "bytes_written_per_layer",
        "tile_tokens", "context_tokens", "attend_blocks",
        "attend_block_tokens")]

    def as_dict(self):
        return {n: int(getattr(self, n)) for n, _ in self._fields_}


_lib = None
_runtime_checked = False


def hip_runtimes(maps_lines=None, resolve=os.path.realpath):
    """Distinct HIP runtime files in a /proc/<pid>/maps listing (by default
    this process's own): the path column of every mapping of a
    libamdhip64 file, with symlinks resolved."""
    if maps_lines is None:
        try:
            with open("/proc/self/maps") as f:
                maps_lines = f.readlines()
        except OSError:
            maps_lines = []
    paths = set()
    for line in maps_lines:
        fields = line.split()
        if len(fields) >= 6 and "libamdhip64" in fields[-1]:
            paths.add(resolve(fields[-1]))
    return paths


def check_single_runtime(maps_lines=None, resolve=os.path.realpath):
    """torch ships its own HIP runtime under the same soname as the system's.
    Tensors and streams handed to the library must belong to the runtime it
    calls, so exactly one may be mapped; raise ImportError otherwise."""
    paths = hip_runtimes(maps_lines, resolve)
    if len(paths) > 1:
        raise ImportError("two HIP runtimes are loaded (" + ", ".join(sorted(paths)) +
                          "): import torch before position_independent_kv_stitch_amd")


def _check_single_runtime():
    global _runtime_checked
    if _runtime_checked:
        return
    check_single_runtime()
    _runtime_checked = True


def _configure(lib):
    P = C.POINTER
    lib.pic_plan.restype = C.c_int
    lib.pic_plan.argtypes = [P(KvShape), P(RopeConfig), P(ChunkC), C.c_int32, P(RequestC),
                             C.c_int32, P(Geom), P(C.c_void_p)]
    lib.pic_stitch.restype = C.c_int
    lib.pic_stitch.argtypes = [C.c_void_p, P(KvView), P(KvView), C.c_int32, C.c_int32,
                               C.c_void_p]
    lib.pic_rotate_inplace.restype = C.c_int
    lib.pic_rotate_inplace.argtypes = [P(KvShape), P(RopeConfig), P(KvView), C.c_int64,
                                       P(SegmentC), C.c_int32, C.c_int32, C.c_int32,
                                       C.c_void_p]
    lib.pic_rotate_inplace_noalloc.restype = C.c_int
    lib.pic_rotate_inplace_noalloc.argtypes = lib.pic_rotate_inplace.argtypes
    lib.pic_rotate_paged.restype = C.c_int
    lib.pic_rotate_paged.argtypes = [P(KvShape), P(RopeConfig), P(KvView), C.c_int32, C.c_int64,
                                     P(PageSegmentC), C.c_int32, C.c_int32, C.c_int32,
                                     C.c_void_p]
    lib.pic_attend.restype = C.c_int
    lib.pic_attend.argtypes = [C.c_void_p, P(KvView), P(KvView), P(AttendArgs), C.c_void_p]
    lib.pic_attend_latent.restype = C.c_int
    lib.pic_attend_latent.argtypes = [C.c_void_p, P(KvView), P(KvView), P(LatentArgs),
                                      C.c_void_p]
    lib.pic_attend_boundary.restype = C.c_int
    lib.pic_attend_boundary.argtypes = [C.c_void_p, P(KvView), P(KvView), P(BoundaryArgs),
                                        C.c_void_p]
    lib.pic_plan_info.restype = C.c_int
    lib.pic_plan_info.argtypes = [C.c_void_p, P(PlanInfo)]
    lib.pic_plan_ranges.restype = C.c_int
    lib.pic_plan_ranges.argtypes = [C.c_void_p, P(C.c_int64), P(C.c_int64)]
    lib.pic_plan_destroy.restype = None
    lib.pic_plan_destroy.argtypes = [C.c_void_p]
    lib.pic_registry_create.restype = C.c_int
    lib.pic_registry_create.argtypes = [C.c_int32, P(C.c_void_p)]
    lib.pic_registry_add.restype = C.c_int
    lib.pic_registry_add.argtypes = [C.c_void_p, P(C.c_uint8), C.c_int32, C.c_int32]
    lib.pic_registry_destroy.restype = None
    lib.pic_registry_destroy.argtypes = [C.c_void_p]
    lib.pic_match.restype = C.c_int
    lib.pic_match.argtypes = [C.c_void_p, P(CdcConfig), C.c_void_p, C.c_int64, C.c_void_p,
                              C.c_int64, C.c_void_p, C.c_void_p]
    lib.pic_stream_copy.restype = C.c_int
    lib.pic_stream_copy.argtypes = [C.c_void_p, C.c_void_p, C.c_int64, C.c_void_p]
    lib.pic_last_error.restype = C.c_char_p
    lib.pic_last_error.argtypes = []
    return lib


_other_builds = {}


def load_library(path: Optional[str] = None):
    """Load libpic_stitch.so (or, with `path`, another build of the same ABI);
    raise if it has not been built.

    torch is imported first when it is installed, so that the library binds
    to torch's HIP runtime (the one that owns the tensors and streams it is
    given) rather than loading a second copy."""
    global _lib
    if path is None and _lib is not None:
        return _lib
    if path is not None and path in _other_builds:
        return _other_builds[path]
    target = LIBRARY if path is None else path
    if not os.path.exists(target):
        raise ImportError(f"{target} is missing: build it with "
                          "`python -c 'import __graft_entry__ as g; g.build()'`")
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = _configure(C.CDLL(target))
    _check_single_runtime()
    if path is None:
        _lib = lib
    else:
        _other_builds[path] = lib
    return lib


def _check(status: int, lib=None):
    if status != PIC_OK:
        raise PicError(status, (lib or load_library()).pic_last_error().decode())


def _get(obj, name, idx):
    """Field `name` of an attribute object, or position `idx` of a tuple."""
    return getattr(obj, name) if hasattr(obj, name) else obj[idx]


def _shape_and_rope(dtype, n_layers, n_heads, row_dim, rope_offset, rope_dim, style, theta,
                    has_v, inv_freq):
    keep = []
    inv_ptr = None
    if inv_freq is not None:
        arr = np.ascontiguousarray(np.asarray(inv_freq, dtype=np.float64))
        keep.append(arr)
        inv_ptr = arr.ctypes.data_as(C.POINTER(C.c_double))
    shape = KvShape(DTYPES[dtype], n_layers, n_heads, row_dim, rope_offset, int(bool(has_v)))
    rope = RopeConfig(rope_dim, STYLES[style], float(theta), inv_ptr)
    return shape, rope, keep


class Plan:
    """An execution plan of the stitch library (wraps pic_plan_t*)."""

    def __init__(self, *, dtype: str, n_layers: int, n_heads: int, row_dim: int,
                 rope_offset: int, rope_dim: int, style: str, theta: float, has_v: bool,
                 chunks: Sequence, requests: Sequence, page_size: int = 0,
                 capacity: int = 0, n_phys_pages: int = 0, inv_freq=None, library=None,
                 src_page_size: int = 0, src_n_pages: int = 0):
        lib = load_library(library)
        self._lib = lib
        self._handle = C.c_void_p()
        self.dtype, self.n_layers, self.n_heads, self.row_dim = dtype, n_layers, n_heads, row_dim
        self.has_v, self.page_size = bool(has_v), page_size
        self.capacity, self.n_phys_pages, self.n_requests = capacity, n_phys_pages, len(requests)
        self.src_page_size, self.src_n_pages = src_page_size, src_n_pages
        shape, rope, keep = _shape_and_rope(dtype, n_layers, n_heads, row_dim, rope_offset,
                                            rope_dim, style, theta, has_v, inv_freq)
        carr = (ChunkC * max(1, len(chunks)))()
        for i, c in enumerate(chunks):
            pt = getattr(c, "page_table", None) if src_page_size else None
            pt_ptr, n_pages = None, 0
            if pt is not None:
                pta = np.ascontiguousarray(np.asarray(pt, dtype=np.int32))
                keep.append(pta)
                pt_ptr, n_pages = pta.ctypes.data_as(C.POINTER(C.c_int32)), len(pta)
            carr[i] = ChunkC(int(_get(c, "token_start", 0)), int(_get(c, "base_pos", 2)),
                             int(_get(c, "length", 1)), n_pages, pt_ptr)
        rarr = (RequestC * max(1, len(requests)))()
        for r, rq in enumerate(requests):
            entries = _get(rq, "entries", 0)
            earr = (EntryC * max(1, len(entries)))()
            for j, e in enumerate(entries):
                earr[j] = EntryC(int(_get(e, "dst_offset", 1)), int(_get(e, "chunk_id", 0)),
                                 int(_get(e, "length", 2)), int(_get(e, "recompute_k", 3)), 0)
            keep.append(earr)
            pt = _get(rq, "page_table", 1) if page_size else None
            pt_ptr, n_pages = None, 0
            if pt is not None:
                pta = np.ascontiguousarray(np.asarray(pt, dtype=np.int32))
                keep.append(pta)
                pt_ptr, n_pages = pta.ctypes.data_as(C.POINTER(C.c_int32)), len(pta)
            rarr[r] = RequestC(earr, pt_ptr, len(entries), n_pages,
                               int(getattr(rq, "context_len", 0) or 0))
        geom = Geom(page_size, src_page_size, capacity, n_phys_pages, src_n_pages)
        t0 = time.perf_counter()
        st = lib.pic_plan(C.byref(shape), C.byref(rope), carr, len(chunks), rarr, len(requests),
                          C.byref(geom), C.byref(self._handle))
        self.plan_seconds = time.perf_counter() - t0  # the C call alone, no marshalling
        _check(st, lib)
        self._info_cache = None
        # what the launch wrappers check tensors against, without asking the
        # library for the full info (whose attention counts build the map)
        self.n_entries = sum(len(_get(rq, "entries", 0)) for rq in requests)
        self.pool_tokens_required = (src_n_pages * src_page_size if src_page_size else
                                     max((int(_get(c, "token_start", 0)) + int(_get(c, "length", 1))
                                          for c in chunks), default=0))

    @classmethod
    def from_workload(cls, wl, library=None) -> "Plan":
        return cls(dtype=wl.dtype, n_layers=wl.n_layers, n_heads=wl.n_heads,
                   row_dim=wl.row_dim, rope_offset=wl.rope_offset, rope_dim=wl.rope_dim,
                   style=wl.style, theta=wl.theta, has_v=wl.has_v, chunks=wl.chunks,
                   requests=wl.requests, page_size=wl.page_size, capacity=wl.capacity,
                   n_phys_pages=wl.n_phys_pages, inv_freq=wl.inv_freq, library=library,
                   src_page_size=getattr(wl, "src_page_size", 0),
                   src_n_pages=getattr(wl, "src_n_pages", 0))

    @property
    def info(self) -> dict:
        """pic_plan_info as a dict (its first call on a plan builds the
        attention map, which the attention calls would build anyway)."""
        if self._info_cache is None:
            info = PlanInfo()
            _check(self._lib.pic_plan_info(self.handle, C.byref(info)), self._lib)
            self._info_cache = info.as_dict()
        return self._info_cache

    def ranges(self):
        """(boundaries, recompute) as int64 arrays of [request, begin, end] rows."""
        n = self.n_entries
        b = np.zeros((max(n, 1), 3), dtype=np.int64)
        r = np.zeros((max(n, 1), 3), dtype=np.int64)
        _check(self._lib.pic_plan_ranges(self._handle, b.ctypes.data_as(C.POINTER(C.c_int64)),
                                         r.ctypes.data_as(C.POINTER(C.c_int64))), self._lib)
        return b[:n], r[:n]

    @property
    def handle(self):
        if not self._handle:
            raise PicError(PIC_ERR_STATE, "plan destroyed")
        return self._handle

    def destroy(self):
        if self._handle:
            self._lib.pic_plan_destroy(self._handle)
            self._handle = C.c_void_p()

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


# ------------------------------------------------------------------- views

def _torch():
    import torch
    return torch


def _dtype_name(t) -> str:
    torch = _torch()
    if t.dtype == torch.float32:
        return "f32"
    if t.dtype == torch.bfloat16:
        return "bf16"
    raise TypeError(f"unsupported tensor dtype {t.dtype}")


def _view(k, v, kind: str) -> KvView:
    """A view of 4-D [L][T][H][D] (pool, in-place buffer), 5-D [L][R][S][H][D]
    (contiguous destination) or 5-D [L][P][page][H][D] (paged destination)."""
    for t in (k, v):
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{kind}: tensors must be on a GPU")
        if t.stride(-1) != 1:
            raise ValueError(f"{kind}: the last (dim) axis must be contiguous")
    if v is not None:
        if v.shape != k.shape or v.stride() != k.stride() or v.dtype != k.dtype:
            raise ValueError(f"{kind}: K and V must share shape, strides and dtype")
    st = k.stride()
    if kind in ("pool", "buf"):
        if k.dim() != 4:
            raise ValueError(f"{kind}: expected [layers][tokens][heads][dim]")
        return KvView(k.data_ptr(), v.data_ptr() if v is not None else None, st[0], st[1],
                      st[2], 0, 0)
    if kind == "paged-pool":
        if k.dim() != 5:
            raise ValueError("paged pool: expected [layers][pages][page][heads][dim]")
        return KvView(k.data_ptr(), v.data_ptr() if v is not None else None, st[0], st[2],
                      st[3], st[1], 0)
    if k.dim() != 5:
        raise ValueError(f"{kind}: expected a 5-D destination")
    if kind == "paged":
        return KvView(k.data_ptr(), v.data_ptr() if v is not None else None, st[0], st[2],
                      st[3], st[1], 0)
    return KvView(k.data_ptr(), v.data_ptr() if v is not None else None, st[0], st[2], st[3],
                  0, st[1])


def _stream_of(t, stream):
    torch = _torch()
    _check_single_runtime()
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return C.c_void_p(stream.cuda_stream)


def stitch(plan: Plan, pool_k, pool_v, dst_k, dst_v, layer_begin: int = 0,
           layer_end: Optional[int] = None, stream=None):
    """Enqueue pic_stitch for layers [layer_begin, layer_end) of the tensors.

    pool_*: contiguous [L][T][H][D] or paged [L][P][page][H][D]; dst_*:
    contiguous [L][R][S][H][D] or paged [L][P][page][H][D].  V tensors are
    None when the plan has no V."""
    le = dst_k.shape[0] if layer_end is None else layer_end
    if _dtype_name(pool_k) != plan.dtype or _dtype_name(dst_k) != plan.dtype:
        raise TypeError("tensor dtype does not match the plan")
    if plan.src_page_size:
        if pool_k.dim() != 5 or pool_k.shape[1] < plan.src_n_pages or \
                pool_k.shape[2] != plan.src_page_size:
            raise PicError(PIC_ERR_RANGE, "paged pool tensor smaller than the plan's pages")
    elif pool_k.shape[1] < plan.pool_tokens_required:
        raise PicError(PIC_ERR_RANGE, f"pool holds {pool_k.shape[1]} tokens, plan needs "
                       f"{plan.pool_tokens_required}")
    if tuple(pool_k.shape[-2:]) != (plan.n_heads, plan.row_dim) or \
            tuple(dst_k.shape[3:]) != (plan.n_heads, plan.row_dim):
        raise ValueError("head/row shape does not match the plan")
    if plan.page_size:
        if dst_k.shape[1] < plan.n_phys_pages or dst_k.shape[2] != plan.page_size:
            raise ValueError("paged destination smaller than the plan's page pool")
    else:
        if dst_k.shape[1] < plan.n_requests or dst_k.shape[2] < plan.capacity:
            raise ValueError("contiguous destination smaller than requests x capacity")
    if pool_k.shape[0] < le or dst_k.shape[0] < le:
        raise ValueError("layer range beyond the tensors")
    if pool_k.device != dst_k.device:
        raise ValueError("pool and destination on different devices")
    if plan.has_v and (pool_v is None or dst_v is None):
        raise ValueError("plan has V rows: pass pool_v and dst_v")
    pv = _view(pool_k, pool_v if plan.has_v else None,
               "paged-pool" if plan.src_page_size else "pool")
    dv = _view(dst_k, dst_v if plan.has_v else None, "paged" if plan.page_size else "contig")
    lib = plan._lib  # the build that made the plan runs it
    _check(lib.pic_stitch(plan.handle, C.byref(pv), C.byref(dv), layer_begin, le,
                          _stream_of(pool_k, stream)), lib)


def attend(plan: Plan, pool_k, pool_v, cache_k, cache_v, q, *, layer: int, out=None,
           scale: Optional[float] = None, sink_tokens: int = 0, sink_bias: float = 0.0,
           stream=None):
    """Enqueue pic_attend: decode attention of every request of the plan at
    `layer`.  q: [requests][q heads][row_dim] in the plan's dtype (post-RoPE);
    pool_* as for stitch(); cache_*: the requests' own KV in the plan's
    destination geometry.  Returns out, fp32 [requests][q heads][row_dim]."""
    torch = _torch()
    if _dtype_name(q) != plan.dtype or q.dim() != 3 or q.stride(-1) != 1:
        raise TypeError("q must be [requests][q heads][row_dim] in the plan's dtype")
    if q.shape[0] != plan.n_requests or q.shape[2] != plan.row_dim:
        raise ValueError("q shape does not match the plan")
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    if out.dtype != torch.float32 or out.shape != q.shape or out.stride(-1) != 1:
        raise TypeError("out must be fp32 with q's shape")
    if plan.src_page_size:
        if pool_k.dim() != 5 or pool_k.shape[1] < plan.src_n_pages:
            raise PicError(PIC_ERR_RANGE, "paged pool tensor smaller than the plan's pages")
        pv = _view(pool_k, pool_v, "paged-pool")
    else:
        if pool_k.shape[1] < plan.pool_tokens_required:
            raise PicError(PIC_ERR_RANGE, "pool tensor smaller than the plan needs")
        pv = _view(pool_k, pool_v, "pool")
    if plan.page_size:
        if cache_k.shape[1] < plan.n_phys_pages or cache_k.shape[2] != plan.page_size:
            raise ValueError("paged cache smaller than the plan's page pool")
        cv = _view(cache_k, cache_v, "paged")
    else:
        if cache_k.shape[1] < plan.n_requests or cache_k.shape[2] < plan.capacity:
            raise ValueError("contiguous cache smaller than requests x capacity")
        cv = _view(cache_k, cache_v, "contig")
    if not (0 <= layer < min(pool_k.shape[0], cache_k.shape[0])):
        raise ValueError("layer beyond the tensors")
    a = AttendArgs(q.data_ptr(), q.stride(0), q.stride(1), out.data_ptr(), out.stride(0),
                   out.stride(1), q.shape[1], layer,
                   float(plan.row_dim ** -0.5 if scale is None else scale), int(sink_tokens),
                   float(sink_bias), 0)
    lib = plan._lib
    _check(lib.pic_attend(plan.handle, C.byref(pv), C.byref(cv), C.byref(a),
                          _stream_of(q, stream)), lib)
    return out


def attend_latent(plan: Plan, pool_k, cache_k, q, *, layer: int, out=None,
                  scale: Optional[float] = None, sink_tokens: int = 0, sink_bias: float = 0.0,
                  stream=None):
    """Enqueue pic_attend_latent: MLA decode attention of every request of an
    MLA plan at `layer`.  q: bf16 [requests][q heads][576] (absorbed query,
    rotary part post-RoPE); pool_k as for stitch(); cache_k: the requests'
    own latent rows in the plan's destination geometry.  Returns out, fp32
    [requests][q heads][512]."""
    torch = _torch()
    if q.dtype != torch.bfloat16 or q.dim() != 3 or q.stride(-1) != 1:
        raise TypeError("q must be bf16 [requests][q heads][row_dim]")
    if q.shape[0] != plan.n_requests or q.shape[2] != plan.row_dim:
        raise ValueError("q shape does not match the plan")
    vdim = 512
    oshape = (q.shape[0], q.shape[1], vdim)
    if out is None:
        out = torch.empty(oshape, dtype=torch.float32, device=q.device)
    if out.dtype != torch.float32 or tuple(out.shape) != oshape or out.stride(-1) != 1:
        raise TypeError(f"out must be fp32 {oshape}")
    if plan.src_page_size:
        if pool_k.dim() != 5 or pool_k.shape[1] < plan.src_n_pages:
            raise PicError(PIC_ERR_RANGE, "paged pool tensor smaller than the plan's pages")
        pv = _view(pool_k, None, "paged-pool")
    else:
        if pool_k.shape[1] < plan.pool_tokens_required:
            raise PicError(PIC_ERR_RANGE, "pool tensor smaller than the plan needs")
        pv = _view(pool_k, None, "pool")
    if plan.page_size:
        if cache_k.shape[1] < plan.n_phys_pages or cache_k.shape[2] != plan.page_size:
            raise ValueError("paged cache smaller than the plan's page pool")
        cv = _view(cache_k, None, "paged")
    else:
        if cache_k.shape[1] < plan.n_requests or cache_k.shape[2] < plan.capacity:
            raise ValueError("contiguous cache smaller than requests x capacity")
        cv = _view(cache_k, None, "contig")
    if not (0 <= layer < min(pool_k.shape[0], cache_k.shape[0])):
        raise ValueError("layer beyond the tensors")
    a = LatentArgs(q.data_ptr(), q.stride(0), q.stride(1), out.data_ptr(), out.stride(0),
                   out.stride(1), q.shape[1], layer,
                   float(plan.row_dim ** -0.5 if scale is None else scale), int(sink_tokens),
                   float(sink_bias), 0)
    lib = plan._lib
    _check(lib.pic_attend_latent(plan.handle, C.byref(pv), C.byref(cv), C.byref(a),
                                 _stream_of(q, stream)), lib)
    return out


def boundary_row_count(plan: Plan, boundary_k: int) -> int:
    """Boundary rows of a plan: min(k, length) per entry placed after 0."""
    bounds, _ = plan.ranges()
    return int(sum(min(boundary_k, int(e - b)) for _, b, e in bounds if b > 0))


def attend_boundary(plan: Plan, pool_k, pool_v, cache_k, cache_v, q, *, layer: int,
                    boundary_k: int = 16, out=None, scale: Optional[float] = None,
                    sink_tokens: int = 0, sink_bias: float = 0.0, stream=None, rows=None):
    """Enqueue pic_attend_boundary (LegoLink boundary reconnection) at `layer`.
    q: bf16 [boundary rows][q heads][row_dim]: the first boundary_k tokens
    of every relocated entry (as boundary_row_count enumerates them), or,
    with `rows`, the given (entry, token) pairs (entries in plan order, the
    rows of one request together, requests ascending); tensors as for
    attend().  Returns out, fp32 with q's shape."""
    torch = _torch()
    if q.dtype != torch.bfloat16 or q.dim() != 3 or q.stride(-1) != 1:
        raise TypeError("q must be bf16 [boundary rows][q heads][row_dim]")
    row_arr = None
    if rows is not None:
        row_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 2))
        if row_arr.size and (row_arr.min() < -2 ** 31 or row_arr.max() >= 2 ** 31):
            raise PicError(PIC_ERR_RANGE, "row entries and tokens must fit int32")
        row_arr = row_arr.astype(np.int32)
        n = len(row_arr)
    else:
        n = boundary_row_count(plan, boundary_k)
    if q.shape[0] != n or q.shape[2] != plan.row_dim:
        raise ValueError(f"q must have {n} boundary rows of {plan.row_dim} dims")
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    if out.dtype != torch.float32 or out.shape != q.shape or out.stride(-1) != 1:
        raise TypeError("out must be fp32 with q's shape")
    if plan.src_page_size:
        if pool_k.dim() != 5 or pool_k.shape[1] < plan.src_n_pages:
            raise PicError(PIC_ERR_RANGE, "paged pool tensor smaller than the plan's pages")
        pv = _view(pool_k, pool_v, "paged-pool")
    else:
        if pool_k.shape[1] < plan.pool_tokens_required:
            raise PicError(PIC_ERR_RANGE, "pool tensor smaller than the plan needs")
        pv = _view(pool_k, pool_v, "pool")
    if plan.page_size:
        if cache_k.shape[1] < plan.n_phys_pages or cache_k.shape[2] != plan.page_size:
            raise ValueError("paged cache smaller than the plan's page pool")
        cv = _view(cache_k, cache_v, "paged")
    else:
        if cache_k.shape[1] < plan.n_requests or cache_k.shape[2] < plan.capacity:
            raise ValueError("contiguous cache smaller than requests x capacity")
        cv = _view(cache_k, cache_v, "contig")
    if not (0 <= layer < min(pool_k.shape[0], cache_k.shape[0])):
        raise ValueError("layer beyond the tensors")
    a = BoundaryArgs(q.data_ptr(), q.stride(0), q.stride(1), out.data_ptr(), out.stride(0),
                     out.stride(1), q.shape[1], layer,
                     float(plan.row_dim ** -0.5 if scale is None else scale), int(boundary_k),
                     int(sink_tokens), float(sink_bias),
                     row_arr.ctypes.data_as(C.POINTER(C.c_int32)) if row_arr is not None else None,
                     n if row_arr is not None else 0, 0)
    lib = plan._lib
    _check(lib.pic_attend_boundary(plan.handle, C.byref(pv), C.byref(cv), C.byref(a),
                                   _stream_of(q, stream)), lib)
    return out


def rotate_inplace(buf_k, segments: Sequence, *, rope_dim: int, theta: float,
                   style: str = "half", rope_offset: int = 0, layer_begin: int = 0,
                   layer_end: Optional[int] = None, inv_freq=None, stream=None, library=None,
                   noalloc: bool = False):
    """Enqueue pic_rotate_inplace on buf_k [L][T][H][D]; segments are
    (token_start, length, delta, recompute_k) tuples or objects.  With
    noalloc, pic_rotate_inplace_noalloc (nothing allocated; calls on one
    device that may overlap race)."""
    lib = load_library(library)
    fn = lib.pic_rotate_inplace_noalloc if noalloc else lib.pic_rotate_inplace
    L, T, H, D = buf_k.shape
    le = L if layer_end is None else layer_end
    shape, rope, keep = _shape_and_rope(_dtype_name(buf_k), L, H, D, rope_offset, rope_dim,
                                        style, theta, False, inv_freq)
    sarr = (SegmentC * max(1, len(segments)))()
    for i, s in enumerate(segments):
        sarr[i] = SegmentC(int(_get(s, "token_start", 0)), int(_get(s, "delta", 2)),
                           int(_get(s, "length", 1)), int(_get(s, "recompute_k", 3)))
    view = _view(buf_k, None, "buf")
    _check(fn(C.byref(shape), C.byref(rope), C.byref(view), T, sarr, len(segments),
              layer_begin, le, _stream_of(buf_k, stream)), lib)


def stream_copy(dst, src, stream=None, library=None):
    """Enqueue pic_stream_copy of src's bytes into dst (two contiguous device
    tensors of equal byte size): the library's 1:1 read/write bandwidth
    reference."""
    if not (dst.is_contiguous() and src.is_contiguous()):
        raise ValueError("stream_copy needs contiguous tensors")
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("dst and src differ in size")
    lib = load_library(library)
    _check(lib.pic_stream_copy(C.c_void_p(dst.data_ptr()), C.c_void_p(src.data_ptr()), nbytes,
                               _stream_of(src, stream)), lib)


def _int32_array(ids):
    """A page-id list as a C-contiguous int32 array and its length; the array
    holds at least one element, so its pointer is never NULL.  Ids outside
    int32 are refused here rather than wrapped."""
    a = np.asarray(ids)
    if a.ndim != 1:
        raise ValueError("a page list is one-dimensional")
    if a.size and a.dtype != np.int32:
        if not np.issubdtype(a.dtype, np.integer):
            raise TypeError("page ids are integers")
        if a.min() < np.iinfo(np.int32).min or a.max() > np.iinfo(np.int32).max:
            raise ValueError("page id outside int32")
    n = int(a.size)
    return (np.ascontiguousarray(a, dtype=np.int32) if n else np.zeros(1, np.int32)), n


def rotate_paged(buf_k, buf_v, segments: Sequence, *, rope_dim: int, theta: float,
                 style: str = "half", rope_offset: int = 0, layer_begin: int = 0,
                 layer_end: Optional[int] = None, inv_freq=None, stream=None, library=None):
    """Enqueue pic_rotate_paged on a paged buffer buf_k (and buf_v, or None)
    of shape [L][P][page][H][D].  segments are objects with fields pages and
    cow (sequences of physical page ids, cow -1 for a page the caller owns,
    or cow None), delta, first, length and recompute_k, or tuples in that
    order.  Page lists given as C-contiguous int32 numpy arrays are passed
    without a copy; other integer sequences are converted, and ids outside
    int32 are refused."""
    lib = load_library(library)
    L, P, S, H, D = buf_k.shape
    le = L if layer_end is None else layer_end
    shape, rope, keep = _shape_and_rope(_dtype_name(buf_k), L, H, D, rope_offset, rope_dim,
                                        style, theta, buf_v is not None, inv_freq)
    sarr = (PageSegmentC * max(1, len(segments)))()
    for i, sg in enumerate(segments):
        pa, n_pages = _int32_array(_get(sg, "pages", 0))
        keep.append(pa)
        cow = _get(sg, "cow", 1)
        if cow is not None:
            ca, n_cow = _int32_array(cow)
            if n_cow != n_pages:
                raise ValueError(f"segment {i}: {n_cow} copy targets for {n_pages} pages")
            keep.append(ca)
            cptr = ca.ctypes.data_as(C.POINTER(C.c_int32))
        else:
            cptr = C.POINTER(C.c_int32)()
        sarr[i] = PageSegmentC(pa.ctypes.data_as(C.POINTER(C.c_int32)), cptr,
                               int(_get(sg, "delta", 2)), n_pages, int(_get(sg, "first", 3)),
                               int(_get(sg, "length", 4)), int(_get(sg, "recompute_k", 5)))
    view = _view(buf_k, buf_v, "paged")
    _check(lib.pic_rotate_paged(C.byref(shape), C.byref(rope), C.byref(view), S, P, sarr,
                                len(segments), layer_begin, le, _stream_of(buf_k, stream)), lib)


def rotate_workload(wl, buf_k, layer_begin=0, layer_end=None, stream=None, library=None):
    """pic_rotate_inplace for an in-place workload description."""
    rotate_inplace(buf_k, wl.segments, rope_dim=wl.rope_dim, theta=wl.theta, style=wl.style,
                   rope_offset=wl.rope_offset, layer_begin=layer_begin, layer_end=layer_end,
                   inv_freq=wl.inv_freq, stream=stream, library=library)


# ------------------------------------------------------- chunking, registry

class Registry:
    """A chunk registry of the library (wraps pic_registry_t*): entries are
    (32-byte fingerprint, length, chunk id)."""

    def __init__(self, kind: str = "xxh64", entries: Sequence = (), library=None):
        lib = load_library(library)
        self._lib = lib
        self.kind = kind
        self._handle = C.c_void_p()
        _check(lib.pic_registry_create(FP_KINDS[kind], C.byref(self._handle)), lib)
        for fp, length, chunk_id in entries:
            self.add(fp, length, chunk_id)

    def add(self, fp: bytes, length: int, chunk_id: int):
        if len(fp) != 32:
            raise ValueError("a fingerprint is 32 bytes")
        buf = (C.c_uint8 * 32).from_buffer_copy(bytes(fp))
        _check(self._lib.pic_registry_add(self.handle, buf, int(length), int(chunk_id)),
               self._lib)

    @property
    def handle(self):
        if not self._handle:
            raise PicError(PIC_ERR_STATE, "registry destroyed")
        return self._handle

    def destroy(self):
        if self._handle:
            self._lib.pic_registry_destroy(self._handle)
            self._handle = C.c_void_p()

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def match(tokens, threshold: int, registry: Optional[Registry] = None, *, gear_seed: int = 0,
          kind: str = "xxh64", fp_seed: int = 0, window: int = 128,
          max_out: Optional[int] = None, out=None, n_out=None, stream=None, library=None):
    """Enqueue pic_match on a device int32 token tensor.  Returns (out, n_out):
    a uint8 device tensor of max_out 56-byte pic_match_t records (default
    max_out: one per token, the most a stream can produce) and a one-element
    int64 device tensor holding the segment count."""
    torch = _torch()
    if tokens.dtype != torch.int32 or tokens.dim() != 1 or not tokens.is_cuda:
        raise TypeError("tokens must be a 1-D int32 GPU tensor")
    if tokens.numel() and tokens.stride(0) != 1:
        raise ValueError("tokens must be contiguous")
    lib = registry._lib if registry is not None else load_library(library)
    n = tokens.numel()
    cap = n if max_out is None else int(max_out)
    rec = C.sizeof(MatchRecord)
    if out is None:
        out = torch.empty((max(cap, 1), rec), dtype=torch.uint8, device=tokens.device)
    elif out.dtype != torch.uint8 or out.numel() < cap * rec or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous uint8 tensor of at least {cap} records")
    if n_out is None:
        n_out = torch.empty(1, dtype=torch.int64, device=tokens.device)
    cfg = CdcConfig(int(threshold) & (2 ** 64 - 1), int(gear_seed) & (2 ** 64 - 1),
                    int(fp_seed) & (2 ** 64 - 1), FP_KINDS[kind], int(window))
    _check(lib.pic_match(registry.handle if registry is not None else None, C.byref(cfg),
                         C.c_void_p(tokens.data_ptr() if n else None), n,
                         C.c_void_p(out.data_ptr()), cap, C.c_void_p(n_out.data_ptr()),
                         _stream_of(tokens, stream)), lib)
    return out, n_out


def match_records(out, n_out) -> np.ndarray:
    """Host copy of the written records as a MATCH_DTYPE array (waits for the
    device)."""
    m = int(n_out.cpu()[0])
    raw = out.cpu().numpy().reshape(-1)
    k = min(m, raw.size // MATCH_DTYPE.itemsize)
    return raw[:k * MATCH_DTYPE.itemsize].view(MATCH_DTYPE), m
