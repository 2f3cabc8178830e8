"""GPU parity of pic_match (content-defined chunking, fingerprints, registry
lookup, fixed-window fallback) against the oracle's chunking code.

Everything here is integer and byte work, so the bar is bit-exactness:
every record (start, length, level, registry id, 32 fingerprint bytes) and
the segment count must equal the oracle's.  Registries are built from the
oracle's own fingerprints of the documents, never from the GPU's.
"""
import sys

import numpy as np
import pytest

from oracle import cdc
from pic_workloads import CDC_THRESHOLD, rag_token_stream, random_tokens

pytestmark = pytest.mark.gpu
M64 = 2 ** 64 - 1


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


def registry_of(docs, th, kind, window, gear_seed=0, fp_seed=0):
    """Every content-defined chunk of every document, and its windows, as
    (fingerprint, length, id) triples (oracle fingerprints)."""
    reg, seen = [], set()
    for doc in docs:
        s = 0
        for e in cdc.cdc_ends(doc, th, gear_seed):
            cands = [(s, e - s)]
            if window > 0:
                cands += [(w, min(window, e - w)) for w in range(s, e, window)]
            for w, wl in cands:
                fp = cdc.fingerprint(doc, w, wl, kind, fp_seed)
                if (fp, wl) not in seen:
                    seen.add((fp, wl))
                    reg.append((fp, wl, len(reg)))
            s = e
    return reg


def gpu_match(torch, tokens, th, reg_entries, kind, **kw):
    import position_independent_kv_stitch_amd as pic
    reg = pic.Registry(kind, reg_entries) if reg_entries is not None else None
    t = torch.from_numpy(np.ascontiguousarray(tokens, dtype=np.int32)).to("cuda:0")
    out, n_out = pic.match(t, th, reg, kind=kind, **kw)
    recs, m = pic.match_records(out, n_out)
    if reg is not None:
        reg.destroy()
    return recs, m


def assert_same(recs, m, want, max_out=None):
    assert m == len(want), (m, len(want))
    k = len(want) if max_out is None else min(max_out, len(want))
    assert len(recs) >= k
    if k == 0:
        return
    got = recs[:k]
    exp_start = np.array([s.start for s in want[:k]], np.int64)
    exp_len = np.array([s.length for s in want[:k]], np.int32)
    exp_lvl = np.array([s.level for s in want[:k]], np.int32)
    exp_id = np.array([s.chunk_id for s in want[:k]], np.int32)
    exp_fp = np.frombuffer(b"".join(s.fp for s in want[:k]), np.uint8).reshape(k, 32)
    bad = np.nonzero((got["start"] != exp_start) | (got["length"] != exp_len) |
                     (got["level"] != exp_lvl) | (got["chunk_id"] != exp_id) |
                     (got["fp"] != exp_fp).any(axis=1))[0]
    assert bad.size == 0, (f"{bad.size} of {k} records differ; first at {bad[0]}: got "
                           f"{got[bad[0]]}, want {want[bad[0]]}")


SIZES = [1, 2, 5, 63, 64, 65, 127, 4095, 4096, 4097, 8191, 12289, 40000]


@pytest.mark.parametrize("kind", ["xxh64", "sha256"])
@pytest.mark.parametrize("n", SIZES)
def test_random_streams_no_registry(torch_cuda, kind, n):
    toks = random_tokens(n, seed=n)
    for th, window in [(1 << 58, 128), (1 << 56, 0), (1 << 61, 7)]:
        say(f"cdc random n={n} kind={kind} th=2^{th.bit_length() - 1} window={window}")
        want = cdc.match(toks, th, [], kind=kind, window=window)
        recs, m = gpu_match(torch_cuda, toks, th, None, kind, window=window)
        assert_same(recs, m, want)


@pytest.mark.parametrize("kind", ["xxh64", "sha256"])
def test_threshold_extremes_and_seeds(torch_cuda, kind):
    toks = random_tokens(5000, seed=11, signed=True)  # negative ids hash their two's complement
    cases = [(0, 128, 0, 0), (M64, 128, 0, 0), (M64, 0, 0, 0), (1 << 57, 128, 77, 5),
             (1 << 57, 1, 0x9E3779B97F4A7C15, M64), (1 << 55, 10000, 3, 1)]
    for th, window, gseed, fseed in cases:
        say(f"cdc extremes kind={kind} th={th} window={window} seeds={gseed},{fseed}")
        want = cdc.match(toks, th, [], kind=kind, window=window, gear_seed=gseed, fp_seed=fseed)
        recs, m = gpu_match(torch_cuda, toks, th, None, kind, window=window, gear_seed=gseed,
                            fp_seed=fseed)
        assert_same(recs, m, want)


def test_empty_stream(torch_cuda):
    import position_independent_kv_stitch_amd as pic
    t = torch_cuda.zeros(0, dtype=torch_cuda.int32, device="cuda:0")
    n_out = torch_cuda.full((1,), 12345, dtype=torch_cuda.int64, device="cuda:0")
    pic.match(t, 1 << 56, None, n_out=n_out, max_out=0)
    assert int(n_out.cpu()[0]) == 0


@pytest.mark.parametrize("kind", ["xxh64", "sha256"])
def test_registered_documents_are_found(torch_cuda, kind):
    """Documents registered alone, then embedded in a longer stream: the GPU
    finds exactly the chunks and windows the oracle finds, with their ids."""
    rng = np.random.default_rng(21)
    th = 1 << 56
    docs = [random_tokens(int(n), seed=100 + i) for i, n in
            enumerate(rng.integers(300, 6000, 12))]
    reg = registry_of(docs, th, kind, 128)
    order = rng.permutation(12)
    parts = []
    for d in order:
        parts.append(random_tokens(int(rng.integers(0, 300)), seed=200 + int(d)))
        parts.append(docs[d])
    stream = np.concatenate(parts)
    for window in (128, 0):
        say(f"cdc registered docs kind={kind} window={window} n={len(stream)} reg={len(reg)}")
        want = cdc.match(stream, th, reg, kind=kind, window=window)
        assert sum(s.chunk_id >= 0 for s in want) > 20
        recs, m = gpu_match(torch_cuda, stream, th, reg, kind, window=window)
        assert_same(recs, m, want)


def test_output_cut_short_keeps_the_count(torch_cuda):
    toks = random_tokens(30000, seed=5)
    th = 1 << 58
    want = cdc.match(toks, th, [], window=64)
    assert len(want) > 100
    for max_out in (0, 1, 37, len(want) - 1, len(want), len(want) + 5):
        say(f"cdc max_out={max_out} of {len(want)}")
        recs, m = gpu_match(torch_cuda, toks, th, None, "xxh64", window=64, max_out=max_out)
        assert_same(recs, m, want, max_out=max_out)


def test_registry_changes_between_calls(torch_cuda):
    """A registry grown between two calls (and past the first table's size)
    is seen by the second call; an unchanged registry is reused."""
    import position_independent_kv_stitch_amd as pic
    th = 1 << 56
    docs = [random_tokens(3000, seed=300 + i) for i in range(6)]
    stream = np.concatenate([random_tokens(100, seed=399)] + docs)
    full = registry_of(docs, th, "sha256", 128)
    first = registry_of(docs[:1], th, "sha256", 128)
    reg = pic.Registry("sha256", first)
    t = torch_cuda.from_numpy(stream).to("cuda:0")
    for entries in (first, first, None):
        if entries is None:  # add the rest; ids continue after the first batch
            known = {(fp, ln) for fp, ln, _ in first}
            entries = list(first)
            for fp, ln, _ in full:
                if (fp, ln) not in known:
                    entries.append((fp, ln, len(entries)))
                    reg.add(fp, ln, len(entries) - 1)
        say(f"cdc registry size {len(entries)}")
        out, n_out = pic.match(t, th, reg, kind="sha256")
        recs, m = pic.match_records(out, n_out)
        assert_same(recs, m, cdc.match(stream, th, entries, kind="sha256"))
    reg.destroy()


@pytest.mark.parametrize("kind", ["xxh64", "sha256"])
def test_rag_stream_full_size(torch_cuda, kind):
    """The batched-RAG prompt stream (64 requests, ~1.4 M tokens, 10% of the
    placed documents edited) against a registry of every pool document's
    chunks and 128-token windows: every record equal to the oracle's."""
    ts = rag_token_stream(0, edit_prob=0.1)
    reg = registry_of(ts.docs, CDC_THRESHOLD, kind, 128)
    say(f"cdc rag full kind={kind} n={len(ts.tokens)} reg={len(reg)}")
    want = cdc.match(ts.tokens, CDC_THRESHOLD, reg, kind=kind)
    recs, m = gpu_match(torch_cuda, ts.tokens, CDC_THRESHOLD, reg, kind)
    assert_same(recs, m, want)
    hits = int((recs["chunk_id"][:m] >= 0).sum())
    say(f"  segments {m}, registered {hits}")
    assert hits > len(want) // 3


def test_registry_temporaries_per_stream(torch_cuda):
    """With a registry, pic_match keeps its temporaries in a buffer per
    stream and replaces it by a larger one when a call needs more.  Calls of
    growing and shrinking length alternate over two streams without waiting,
    each with its own output, and the registry is destroyed right after they
    are enqueued: destroy must wait for every call, also those whose buffer
    was since replaced, and every call must equal the oracle."""
    import position_independent_kv_stitch_amd as pic
    torch = torch_cuda
    th = 1 << 56
    docs = [random_tokens(2500, seed=500 + i) for i in range(4)]
    entries = registry_of(docs, th, "xxh64", 128)
    reg = pic.Registry("xxh64", entries)
    sizes = [3000, 20000, 500, 60000, 7000, 120000]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    inputs, outs = [], []
    for i, n in enumerate(sizes):
        toks = np.concatenate([random_tokens(n, seed=600 + i), docs[i % 4]])
        inputs.append(toks)
        t = torch.from_numpy(toks).to("cuda:0")
        torch.cuda.synchronize()
        outs.append((t,) + pic.match(t, th, reg, kind="xxh64", stream=streams[(i // 2) % 2]))
    reg.destroy()
    torch.cuda.synchronize()
    for i, (toks, (_, out, n_out)) in enumerate(zip(inputs, outs)):
        recs, m = pic.match_records(out, n_out)
        say(f"cdc temporaries call {i}: {len(toks)} tokens, {m} segments")
        assert_same(recs, m, cdc.match(toks, th, entries, kind="xxh64"))
