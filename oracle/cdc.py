"""ctypes wrapper around the oracle's chunking code (cdc_oracle.c).

TEST INFRASTRUCTURE ONLY, like the rest of this package.  Token streams are
int32 numpy arrays; fingerprints are 32-byte `bytes` (SHA-256 digests, or
the xxHash64 value as 8 little-endian bytes followed by 24 zero bytes).
"""
from __future__ import annotations

import ctypes as C
from dataclasses import dataclass

import numpy as np

from .ref import _load

FP_KINDS = {"xxh64": 0, "sha256": 1}
_u8p = C.POINTER(C.c_uint8)
_i32p = C.POINTER(C.c_int32)
_i64p = C.POINTER(C.c_int64)
_u64p = C.POINTER(C.c_uint64)
_ready = False


def _lib():
    global _ready
    lib = _load()
    if not _ready:
        lib.orc_xxh64.restype = C.c_uint64
        lib.orc_xxh64.argtypes = [_u8p, C.c_int64, C.c_uint64]
        lib.orc_sha256.restype = None
        lib.orc_sha256.argtypes = [_u8p, C.c_int64, _u8p]
        lib.orc_gear_value.restype = C.c_uint64
        lib.orc_gear_value.argtypes = [C.c_int32, C.c_uint64]
        lib.orc_gear.restype = None
        lib.orc_gear.argtypes = [_i32p, C.c_int64, C.c_uint64, _u64p]
        lib.orc_cdc_ends.restype = C.c_int64
        lib.orc_cdc_ends.argtypes = [_i32p, C.c_int64, C.c_uint64, C.c_uint64, _i64p]
        lib.orc_fingerprint.restype = C.c_int
        lib.orc_fingerprint.argtypes = [_i32p, C.c_int64, C.c_int64, C.c_int, C.c_uint64, _u8p]
        lib.orc_match.restype = C.c_int64
        lib.orc_match.argtypes = [_i32p, C.c_int64, C.c_uint64, C.c_uint64, C.c_int, C.c_uint64,
                                  C.c_int32, _u8p, _i32p, _i32p, C.c_int64, _i64p, _i32p, _i32p,
                                  _i32p, _u8p, C.c_int64]
        _ready = True
    return lib


def _buf(data: bytes):
    a = np.frombuffer(bytes(data), dtype=np.uint8).copy() if data else np.zeros(1, np.uint8)
    return a, a.ctypes.data_as(_u8p)


def _tokens(t):
    a = np.ascontiguousarray(t, dtype=np.int32)
    if a.size == 0:
        a = np.zeros(1, np.int32)[:0]
    return a, a.ctypes.data_as(_i32p)


def xxh64(data: bytes, seed: int = 0) -> int:
    a, p = _buf(data)
    return int(_lib().orc_xxh64(p, len(data), seed & (2 ** 64 - 1)))


def sha256(data: bytes) -> bytes:
    a, p = _buf(data)
    out = np.zeros(32, np.uint8)
    _lib().orc_sha256(p, len(data), out.ctypes.data_as(_u8p))
    return out.tobytes()


def gear_value(token: int, gear_seed: int = 0) -> int:
    return int(_lib().orc_gear_value(int(token), gear_seed))


def gear(tokens, gear_seed: int = 0) -> np.ndarray:
    a, p = _tokens(tokens)
    h = np.zeros(max(1, a.size), np.uint64)
    _lib().orc_gear(p, a.size, gear_seed, h.ctypes.data_as(_u64p))
    return h[:a.size]


def cdc_ends(tokens, threshold: int, gear_seed: int = 0) -> np.ndarray:
    a, p = _tokens(tokens)
    ends = np.zeros(max(1, a.size), np.int64)
    n = _lib().orc_cdc_ends(p, a.size, threshold, gear_seed, ends.ctypes.data_as(_i64p))
    return ends[:n]


def fingerprint(tokens, start: int, length: int, kind: str = "xxh64", seed: int = 0) -> bytes:
    a, p = _tokens(tokens)
    out = np.zeros(32, np.uint8)
    assert _lib().orc_fingerprint(p, start, length, FP_KINDS[kind], seed,
                                  out.ctypes.data_as(_u8p)) == 0
    return out.tobytes()


@dataclass(frozen=True)
class Segment:
    start: int
    length: int
    level: int      # 0: content-defined chunk, 1: fallback window of a missed chunk
    chunk_id: int   # registry id, -1 when the registry has no such segment
    fp: bytes


def match(tokens, threshold: int, registry=(), *, gear_seed: int = 0, kind: str = "xxh64",
          fp_seed: int = 0, window: int = 128):
    """Segments of a stream against a registry of (fingerprint, length, id)."""
    a, p = _tokens(tokens)
    n_reg = len(registry)
    rfp = np.zeros((max(1, n_reg), 32), np.uint8)
    rlen = np.zeros(max(1, n_reg), np.int32)
    rid = np.zeros(max(1, n_reg), np.int32)
    for i, (fp, ln, cid) in enumerate(registry):
        rfp[i] = np.frombuffer(fp, np.uint8)
        rlen[i], rid[i] = ln, cid
    cap = max(1, 2 * a.size)
    st = np.zeros(cap, np.int64)
    ln = np.zeros(cap, np.int32)
    lv = np.zeros(cap, np.int32)
    ids = np.zeros(cap, np.int32)
    fps = np.zeros((cap, 32), np.uint8)
    m = _lib().orc_match(p, a.size, threshold, gear_seed, FP_KINDS[kind], fp_seed, window,
                         rfp.ctypes.data_as(_u8p), rlen.ctypes.data_as(_i32p),
                         rid.ctypes.data_as(_i32p), n_reg, st.ctypes.data_as(_i64p),
                         ln.ctypes.data_as(_i32p), lv.ctypes.data_as(_i32p),
                         ids.ctypes.data_as(_i32p), fps.ctypes.data_as(_u8p), cap)
    assert 0 <= m <= cap
    return [Segment(int(st[i]), int(ln[i]), int(lv[i]), int(ids[i]), fps[i].tobytes())
            for i in range(m)]
