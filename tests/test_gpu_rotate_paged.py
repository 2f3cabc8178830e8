"""GPU parity of pic_rotate_paged (paged in-place turn with copy-on-write for
shared pages) against the fp64 oracle, through the C ABI: every element
outside the rotary slice of K bit-exact (V and untouched pages included),
rotated fp32 within 1e-5 * max|k|, rotated bf16 within one ulp."""
import sys

import numpy as np
import pytest

import oracle
from parity_util import compare_bits, compare_k, max_abs, to_host
from pic_workloads import PageSegment, normal_values, paged_cow_case

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


def run(torch, wl, n_phys, segs, seed, layer_begin=0, layer_end=None):
    import position_independent_kv_stitch_amd as pic
    shape = (wl.n_layers, n_phys, wl.page_size, wl.n_heads, wl.row_dim)
    k = normal_values(shape, wl.dtype, seed, "cuda:0")
    v = normal_values(shape, wl.dtype, seed + 1, "cuda:0") if wl.has_v else None
    k0 = to_host(k)
    v0 = to_host(v) if v is not None else None
    pic.rotate_paged(k, v, segs, rope_dim=wl.rope_dim, theta=wl.theta, style=wl.style,
                     rope_offset=wl.rope_offset, layer_begin=layer_begin, layer_end=layer_end)
    torch.cuda.synchronize()
    want_k, want_v = k0.copy(), (v0.copy() if v0 is not None else None)
    assert oracle.rotate_paged(wl, want_k, want_v, wl.page_size, segs, layer_begin,
                               layer_end) == "ok"
    stats = compare_k(to_host(k), want_k, wl.rope_offset, wl.rope_dim, max_abs(k0),
                      what="paged K")
    if v is not None:
        compare_bits(to_host(v), want_v, "paged V")
    return stats


CASES = [(seed, dt, style, mla, ps)
         for seed in range(2)
         for dt in ("f32", "bf16")
         for style in ("half", "interleaved")
         for mla in (False, True)
         for ps in (4, 16)]


@pytest.mark.parametrize("seed,dt,style,mla,ps", CASES)
def test_random_small(torch_cuda, seed, dt, style, mla, ps):
    wl, n_phys, segs = paged_cow_case(seed + 10 * ps, dtype=dt, style=style, mla=mla,
                                      page_size=ps)
    n_cow = sum(1 for s in segs for c in (s.cow or ()) if c >= 0)
    say(f"paged cow seed={seed} {dt} {style} mla={mla} page={ps}: {len(segs)} segments, "
        f"{n_cow} copied pages")
    stats = run(torch_cuda, wl, n_phys, segs, seed)
    say(f"  {stats}")


def test_layer_subrange_and_owned_only(torch_cuda):
    """Layers outside [layer_begin, layer_end) stay as they were; segments
    without copy targets touch only the rotary slice."""
    wl, n_phys, segs = paged_cow_case(40, dtype="bf16", n_layers=4, share=0.0)
    segs = [PageSegment(s.pages, None, s.delta, s.first, s.length, s.recompute_k) for s in segs]
    run(torch_cuda, wl, n_phys, segs, 3, layer_begin=1, layer_end=3)


def test_large_shifts_and_long_segments(torch_cuda):
    """Shifts up to +-65,536 (Qwen3-8B's in-place range) over segments of up
    to 2,000 tokens in 16-token pages, half of the chunks shared."""
    wl, n_phys, segs = paged_cow_case(41, dtype="bf16", n_layers=2, max_len=2000, n_chunks=6,
                                      delta_range=65536)
    run(torch_cuda, wl, n_phys, segs, 4)


def test_zero_shift_copies_are_bit_exact(torch_cuda):
    wl, n_phys, segs = paged_cow_case(42, dtype="f32", share=1.0)
    segs = [PageSegment(s.pages, s.cow, 0, s.first, s.length, s.recompute_k) for s in segs]
    stats = run(torch_cuda, wl, n_phys, segs, 5)
    assert stats["bit_diffs"] == 0


def test_config5_paged_cow_full(torch_cuda):
    """The bench's paged workload at full size (36 layers, 64 x 2048 tokens
    in 16-token pages, 16 chunks shared): one call over all layers and
    segments, then
    - on the whole buffer: every copy target holds its source's V bit for
      bit, owned pages keep their V, shared source pages keep K and V, and
      the first 16 tokens (page 0) of every segment keep their K bits;
    - at layers 0 and 35, two shared and two owned segments against the
      oracle run on just their pages."""
    torch = torch_cuda
    import position_independent_kv_stitch_amd as pic
    from pic_workloads import config5_paged_cow
    wl, n_phys, segs = config5_paged_cow()
    say("config5 paged: generating inputs")
    shape = (wl.n_layers, n_phys, wl.page_size, wl.n_heads, wl.row_dim)
    k = normal_values(shape, wl.dtype, 0, "cuda:0")
    v = normal_values(shape, wl.dtype, 1, "cuda:0")
    k0, v0 = k.clone(), v.clone()
    shared = [g for g, s in enumerate(segs) if s.cow is not None]
    owned = [g for g, s in enumerate(segs) if s.cow is None]
    pick = shared[:2] + owned[:2]
    mini = sorted({p for g in pick for p in segs[g].pages}
                  | {c for g in pick for c in (segs[g].cow or ())})
    at = {p: i for i, p in enumerate(mini)}
    idx = torch.tensor(mini, dtype=torch.long, device="cuda:0")
    sample = [0, wl.n_layers - 1]
    before = {L: (to_host(k[L:L + 1, idx]), to_host(v[L:L + 1, idx])) for L in sample}
    say(f"config5 paged: one call, {len(segs)} segments, {len(shared)} shared")
    pic.rotate_paged(k, v, segs, rope_dim=wl.rope_dim, theta=wl.theta, style=wl.style,
                     rope_offset=wl.rope_offset)
    torch.cuda.synchronize()

    def pages(ids):
        return torch.tensor(list(ids), dtype=torch.long, device="cuda:0")

    def same(a, b):
        return torch.equal(a.view(torch.int16), b.view(torch.int16))

    src = pages(p for g in shared for p in segs[g].pages)
    dst = pages(c for g in shared for c in segs[g].cow)
    own = pages(p for g in owned for p in segs[g].pages)
    assert same(v[:, dst], v0[:, src]), "copy targets hold their sources' V"
    assert same(v[:, own], v0[:, own]), "owned pages keep their V"
    assert same(k[:, src], k0[:, src]) and same(v[:, src], v0[:, src]), "shared sources unchanged"
    first = pages(segs[g].pages[0] for g in owned)
    assert same(k[:, first], k0[:, first]), "recompute tokens of owned segments keep their K"
    assert same(k[:, pages(segs[g].cow[0] for g in shared)],
                k0[:, pages(segs[g].pages[0] for g in shared)]), "recompute tokens copied as they are"
    del k0, v0
    msegs = [PageSegment(tuple(at[p] for p in segs[g].pages),
                         tuple(at[c] for c in segs[g].cow) if segs[g].cow else None,
                         segs[g].delta, segs[g].first, segs[g].length, segs[g].recompute_k)
             for g in pick]
    for L in sample:
        want_k, want_v = before[L][0].copy(), before[L][1].copy()
        assert oracle.rotate_paged(wl, want_k, want_v, wl.page_size, msegs, 0, 1) == "ok"
        stats = compare_k(to_host(k[L:L + 1, idx]), want_k, wl.rope_offset, wl.rope_dim,
                          max_abs(before[L][0]), what=f"paged K layer {L}")
        compare_bits(to_host(v[L:L + 1, idx]), want_v, f"paged V layer {L}")
        say(f"  layer {L}: {stats}")


def test_back_to_back_calls_reuse_staging(torch_cuda):
    """Seven calls enqueued without waiting, on separate buffers, of
    different sizes (each call stages two launches' metadata, so the staging
    slots are reused several times while earlier calls are still queued):
    every call must still see its own tiles and shift tables."""
    torch = torch_cuda
    import position_independent_kv_stitch_amd as pic
    cases = []
    for i, max_len in enumerate((40, 70, 300, 900, 2000, 120, 3000)):
        wl, n_phys, segs = paged_cow_case(60 + i, dtype="bf16", n_layers=2, max_len=max_len,
                                          n_chunks=3 + i % 3, delta_range=65536)
        shape = (wl.n_layers, n_phys, wl.page_size, wl.n_heads, wl.row_dim)
        k = normal_values(shape, wl.dtype, 70 + i, "cuda:0")
        v = normal_values(shape, wl.dtype, 80 + i, "cuda:0")
        cases.append((wl, segs, k, v, to_host(k), to_host(v)))
    torch.cuda.synchronize()
    for wl, segs, k, v, _, _ in cases:
        pic.rotate_paged(k, v, segs, rope_dim=wl.rope_dim, theta=wl.theta, style=wl.style,
                         rope_offset=wl.rope_offset)
    torch.cuda.synchronize()
    for i, (wl, segs, k, v, k0, v0) in enumerate(cases):
        want_k, want_v = k0.copy(), v0.copy()
        assert oracle.rotate_paged(wl, want_k, want_v, wl.page_size, segs) == "ok"
        stats = compare_k(to_host(k), want_k, wl.rope_offset, wl.rope_dim, max_abs(k0),
                          what=f"call {i}")
        compare_bits(to_host(v), want_v, f"call {i} V")
        say(f"  call {i}: {len(segs)} segments, {stats}")
