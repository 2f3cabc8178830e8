"""Pins of the oracle's chunking code (no GPU): the two fingerprints against
independent libraries (python-xxhash, hashlib), the rolling Gear hash
against its 64-token window closed form, the content-defined property of
the boundaries, and the registry lookup on streams built to hit known
chunks and windows."""
import hashlib

import numpy as np
import pytest
import xxhash

from oracle import cdc

M64 = 2 ** 64 - 1


def le32(tokens) -> bytes:
    return np.asarray(tokens, dtype="<i4").tobytes()


@pytest.mark.parametrize("seed", [0, 1, 0x9E3779B97F4A7C15])
def test_xxh64_matches_library(seed):
    rng = np.random.default_rng(seed & 0xFFFF)
    for n in list(range(0, 100)) + [255, 256, 1000, 4099]:
        b = rng.integers(0, 256, n, dtype=np.uint8).tobytes()
        assert cdc.xxh64(b, seed) == xxhash.xxh64(b, seed=seed).intdigest(), n


def test_sha256_matches_library():
    rng = np.random.default_rng(1)
    for n in list(range(0, 140)) + [1000, 4096, 4097]:
        b = rng.integers(0, 256, n, dtype=np.uint8).tobytes()
        assert cdc.sha256(b) == hashlib.sha256(b).digest(), n


def test_gear_values_and_window_closed_form():
    """G(t) is xxHash64 of the token's 4 little-endian bytes; the rolling hash
    equals sum_{j < 64} G(t_{i-j}) * 2^j mod 2^64 (Python integers)."""
    rng = np.random.default_rng(2)
    toks = rng.integers(-2 ** 31, 2 ** 31, 300, dtype=np.int64).astype(np.int32)
    for seed in (0, 77):
        G = [xxhash.xxh64(le32([t]), seed=seed).intdigest() for t in toks]
        assert [cdc.gear_value(int(t), seed) for t in toks[:20]] == G[:20]
        h = cdc.gear(toks, seed)
        for i in range(len(toks)):
            want = sum(G[i - j] << j for j in range(min(i, 63) + 1)) & M64
            assert int(h[i]) == want, i


def test_boundaries_follow_content():
    """Inserting tokens in front moves every boundary at least 63 tokens past
    the insertion by exactly the inserted length."""
    rng = np.random.default_rng(3)
    doc = rng.integers(0, 128000, 6000).astype(np.int32)
    th = 1 << 56  # about one boundary per 256 tokens
    base = cdc.cdc_ends(doc, th)
    for k in (1, 17, 500):
        pre = rng.integers(0, 128000, k).astype(np.int32)
        moved = cdc.cdc_ends(np.concatenate([pre, doc]), th)
        want = [e + k for e in base if e - 1 >= 63]
        got = [e for e in moved if e - 1 >= k + 63]
        assert got == want
    assert 10 < len(base) < 60  # 6000 / 256 ~ 23 expected


def test_threshold_extremes():
    rng = np.random.default_rng(4)
    toks = rng.integers(0, 1000, 500).astype(np.int32)
    assert list(cdc.cdc_ends(toks, 0)) == [500]  # nothing is below 0: one chunk
    assert list(cdc.cdc_ends(toks, M64)) == list(range(1, 501))
    assert list(cdc.cdc_ends(toks[:0], 123)) == []
    assert list(cdc.cdc_ends(toks[:1], 0)) == [1]


def test_fingerprints_hash_little_endian_token_bytes():
    rng = np.random.default_rng(5)
    toks = rng.integers(-5, 200000, 1000).astype(np.int32)
    fp = cdc.fingerprint(toks, 100, 300, "xxh64", seed=9)
    v = xxhash.xxh64(le32(toks[100:400]), seed=9).intdigest()
    assert fp == v.to_bytes(8, "little") + bytes(24)
    assert cdc.fingerprint(toks, 7, 129, "sha256") == hashlib.sha256(le32(toks[7:136])).digest()


def _registry_of(doc, th, kind, window, first_id=0):
    """A document's chunks and their fallback windows, as a registry."""
    reg, seen, s, cid = [], set(), 0, first_id
    for e in cdc.cdc_ends(doc, th):
        for w, wl in [(s, e - s)] + [(w, min(window, e - w)) for w in range(s, e, window)]:
            fp = cdc.fingerprint(doc, w, wl, kind)
            if (fp, wl) not in seen:  # a chunk no longer than a window is its own window
                seen.add((fp, wl))
                reg.append((fp, wl, cid))
                cid += 1
        s = e
    return reg


@pytest.mark.parametrize("kind", ["xxh64", "sha256"])
def test_match_finds_a_registered_document(kind):
    """A registered document embedded behind unrelated tokens: every chunk
    of it that starts at least 64 tokens into it is found, at its shifted
    place, with its id; the segments tile the stream."""
    rng = np.random.default_rng(6)
    th = 1 << 56
    doc = rng.integers(0, 128000, 5000).astype(np.int32)
    reg = _registry_of(doc, th, kind, 128)
    pre = rng.integers(0, 128000, 333).astype(np.int32)
    post = rng.integers(0, 128000, 200).astype(np.int32)
    stream = np.concatenate([pre, doc, post])
    segs = cdc.match(stream, th, reg, kind=kind)
    pos = 0
    for s in segs:  # contiguous tiling of the stream
        assert s.start == pos and s.length >= 1
        pos += s.length
    assert pos == len(stream)
    ends = list(cdc.cdc_ends(doc, th))
    starts = [0] + ends[:-1]
    by_start = {s.start: s for s in segs}
    chunk_ids = {fp: cid for fp, _, cid in reg}
    found = 0
    for st, en in zip(starts, ends):
        if st < 64 or en == len(doc):
            continue  # boundaries there depend on the surrounding tokens
        s = by_start[len(pre) + st]
        assert s.level == 0 and s.length == en - st
        assert s.chunk_id == chunk_ids[cdc.fingerprint(doc, st, en - st, kind)]
        found += 1
    assert found >= 10


def test_fallback_windows_recover_an_edited_chunk():
    """One token edited inside a long registered chunk: that chunk misses,
    and its 128-token windows before the edit are found (S1)."""
    rng = np.random.default_rng(7)
    th = 1 << 54  # about one boundary per 1024 tokens
    doc = rng.integers(0, 128000, 8000).astype(np.int32)
    reg = _registry_of(doc, th, "xxh64", 128)
    ends = list(cdc.cdc_ends(doc, th))
    starts = [0] + ends[:-1]
    i = max(range(1, len(ends) - 1), key=lambda j: ends[j] - starts[j])  # longest inner chunk
    st, en = starts[i], ends[i]
    assert en - st > 600
    edit = st + 5 * 128 + 3
    stream = doc.copy()
    stream[edit] ^= 1
    segs = cdc.match(stream, th, reg)
    win = [s for s in segs if s.level == 1 and st <= s.start < en]
    assert win and win[0].start == st
    ids = {fp: cid for fp, _, cid in reg}
    for s in win:
        if s.start + s.length <= edit:
            assert s.chunk_id == ids[cdc.fingerprint(doc, s.start, s.length)]
        elif s.start <= edit:
            assert s.chunk_id == -1
    # with no fallback the edited chunk stays one missed segment
    segs0 = cdc.match(stream, th, reg, window=0)
    miss = [s for s in segs0 if s.start == st]
    assert miss and miss[0].level == 0 and miss[0].chunk_id == -1
