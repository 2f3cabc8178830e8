"""pic_rotate_paged on the CPU: the oracle's paged copy-on-write turn pinned
by properties the definition fixes, and the library's argument checks
against the oracle's statement of the rules (every refused call returns
before any device work, so these run without a GPU).

The oracle composes three things: address translation through the block
tables, the copy of shared pages, and the in-place turn (pinned on its own
in test_oracle_pins).  The pins below check each against an independent
statement: pages no segment maps stay as they were, shared pages stay as
they were and their copies hold every slot, each turned row equals the key
rotated by the segment's shift (angles from numpy in fp64), and turning by
d then by -d gives the keys back.
"""
import ctypes as C

import numpy as np
import pytest

import oracle
from pic_workloads import PageSegment, paged_cow_case


def rotate_rows(rows, wl, delta):
    """rows [..., H, D] (fp64) with the rotary slice turned by delta: the
    RoPE shift rotation written from its definition (plane i: angle delta *
    theta^(-2i/rope_dim), pairs (i, i + R/2) or (2i, 2i + 1))."""
    out = rows.copy()
    R, ro = wl.rope_dim, wl.rope_offset
    ang = delta * wl.theta ** (-np.arange(R // 2) * 2.0 / R)
    c, s = np.cos(ang), np.sin(ang)
    if wl.style == "half":
        x = rows[..., ro:ro + R // 2]
        y = rows[..., ro + R // 2:ro + R]
        out[..., ro:ro + R // 2] = x * c - y * s
        out[..., ro + R // 2:ro + R] = x * s + y * c
    else:
        x = rows[..., ro:ro + R:2]
        y = rows[..., ro + 1:ro + R:2]
        out[..., ro:ro + R:2] = x * c - y * s
        out[..., ro + 1:ro + R:2] = x * s + y * c
    return out


def run_case(seed, style, mla):
    wl, n_phys, segs = paged_cow_case(seed, dtype="f64", style=style, mla=mla)
    rng = np.random.default_rng(100 + seed)
    shape = (wl.n_layers, n_phys, wl.page_size, wl.n_heads, wl.row_dim)
    k0 = rng.standard_normal(shape)
    v0 = rng.standard_normal(shape) if wl.has_v else None
    k, v = k0.copy(), (v0.copy() if v0 is not None else None)
    assert oracle.rotate_paged(wl, k, v, wl.page_size, segs, dtype="f64") == "ok"
    return wl, n_phys, segs, k0, v0, k, v


CASES = [(seed, style, mla) for seed in range(6) for style in ("half", "interleaved")
         for mla in (False, True)]


@pytest.mark.parametrize("seed,style,mla", CASES)
def test_oracle_pages_copies_and_turned_rows(seed, style, mla):
    wl, n_phys, segs, k0, v0, k, v = run_case(seed, style, mla)
    ps = wl.page_size
    mapped, targets, sources = set(), set(), set()
    for sg in segs:
        mapped.update(sg.pages)
        for pg, cw in zip(sg.pages, sg.cow or [-1] * len(sg.pages)):
            if cw >= 0:
                targets.add(cw)
                sources.add(pg)
    # pages no segment maps or copies to: unchanged; shared pages: unchanged
    for p in range(n_phys):
        if p not in mapped and p not in targets or p in sources:
            assert np.array_equal(k[:, p], k0[:, p]), p
            if v is not None:
                assert np.array_equal(v[:, p], v0[:, p]), p
    for sg in segs:
        cow = sg.cow or [-1] * len(sg.pages)
        home = [cw if cw >= 0 else pg for pg, cw in zip(sg.pages, cow)]
        turned = set()
        for t in range(sg.length):
            q = sg.first + t
            i, slot = q // ps, q % ps
            want = k0[:, sg.pages[i], slot]
            if t >= sg.recompute_k and sg.delta != 0:
                want = rotate_rows(want, wl, sg.delta)
                turned.add((i, slot))
            got = k[:, home[i], slot]
            assert np.max(np.abs(got - want)) <= 1e-12 * max(1.0, abs(sg.delta)) * np.max(np.abs(k0)), \
                (sg, t)
        # a copy holds every slot: outside the turned run bit for bit, and V whole
        for i, (pg, cw) in enumerate(zip(sg.pages, cow)):
            if cw < 0:
                continue
            for slot in range(ps):
                if (i, slot) not in turned:
                    assert np.array_equal(k[:, cw, slot], k0[:, pg, slot])
            if v is not None:
                assert np.array_equal(v[:, cw], v0[:, pg])


@pytest.mark.parametrize("style", ["half", "interleaved"])
def test_oracle_turn_then_inverse_gives_keys_back(style):
    """Owned pages only (no copies): d then -d recovers the keys (fp64)."""
    wl, n_phys, segs = paged_cow_case(7, dtype="f64", style=style, share=0.0)
    segs = [PageSegment(s.pages, None, s.delta, s.first, s.length, s.recompute_k) for s in segs]
    inv = [PageSegment(s.pages, None, -s.delta, s.first, s.length, s.recompute_k) for s in segs]
    rng = np.random.default_rng(3)
    k0 = rng.standard_normal((wl.n_layers, n_phys, wl.page_size, wl.n_heads, wl.row_dim))
    k = k0.copy()
    assert oracle.rotate_paged(wl, k, None, wl.page_size, segs, dtype="f64") == "ok"
    assert not np.allclose(k, k0)
    assert oracle.rotate_paged(wl, k, None, wl.page_size, inv, dtype="f64") == "ok"
    assert np.max(np.abs(k - k0)) < 1e-9


def test_oracle_zero_shift_copies_exactly():
    wl, n_phys, segs = paged_cow_case(11, dtype="bf16", share=1.0)
    segs = [PageSegment(s.pages, s.cow, 0, s.first, s.length, s.recompute_k) for s in segs]
    rng = np.random.default_rng(5)
    shape = (wl.n_layers, n_phys, wl.page_size, wl.n_heads, wl.row_dim)
    k0 = rng.integers(0, 1 << 16, size=shape).astype(np.uint16) & 0x7F7F
    k = k0.copy()
    assert oracle.rotate_paged(wl, k, None, wl.page_size, segs, dtype="bf16") == "ok"
    for sg in segs:
        for pg, cw in zip(sg.pages, sg.cow):
            assert np.array_equal(k[:, cw], k0[:, pg])


# -------------------------------------------------------------- validation

def seg(pages, first, length, delta=5, k=0, cow=None):
    return PageSegment(tuple(pages), tuple(cow) if cow is not None else None, delta, first,
                       length, k)


PS = 4
RULES = [
    ("ok", [seg([0, 1], 1, 6), seg([2], 0, 4, cow=[5])]),
    ("ok", [seg([0], 0, 2), seg([0], 2, 2)]),                       # one page, disjoint slots
    ("ok", [seg([0], 0, 4, cow=[5]), seg([0], 0, 4, cow=[6])]),     # a shared page, two copies
    ("ok", [seg([0], 0, 4, cow=[5]), seg([0], 0, 2, delta=0)]),     # shared page read, not turned
    ("ok", [seg([0], 0, 4, k=4), seg([0], 0, 4, cow=[5])]),         # nothing turned in place
    ("range", [seg([0], 4, 1)]),                                    # first >= page_size
    ("range", [seg([0], -1, 1)]),
    ("range", [seg([0], 0, 0)]),                                    # empty segment
    ("range", [seg([0], 0, 3, k=4)]),                               # recompute_k > length
    ("range", [seg([8], 0, 2)]),                                    # page id past the pool
    ("range", [seg([0], 0, 2, cow=[8])]),                           # copy target past the pool
    ("range", [seg([0], 0, 2, cow=[-2])]),
    ("range", [seg([0], 0, 2 ** 31 - 3)]),                          # pages span 2^31 positions
    ("range", [seg([0], 3, 2 ** 31 - 6)]),
    ("bad_arg", [seg([0], 3, 2 ** 31 - 7)]),                        # span 2^31 - 4 fits int32
    ("bad_arg", [seg([0, 1], 0, 4)]),                               # n_pages != ceil(.)
    ("bad_arg", [seg([0], 2, 4)]),
    ("overlap", [seg([0], 0, 3), seg([0], 2, 2)]),                  # slot 2 turned twice
    ("overlap", [seg([0, 1], 2, 4), seg([1], 1, 1)]),
    ("overlap", [seg([0], 0, 2, cow=[5]), seg([1], 0, 2, cow=[5])]),  # a target used twice
    ("overlap", [seg([0], 0, 2, cow=[1]), seg([1], 0, 2)]),         # a target another maps
    ("overlap", [seg([0], 0, 2, cow=[5]), seg([0], 2, 2)]),         # shared page turned in place
    # every segment's own checks come before clashes between segments
    ("range", [seg([0], 0, 2, cow=[5]), seg([1], 0, 2, cow=[5]), seg([9], 0, 1)]),
    ("bad_arg", [seg([0], 0, 3), seg([0], 2, 2), seg([1, 2], 0, 1)]),
]


@pytest.mark.parametrize("want,segs", RULES)
def test_oracle_validation_rules(want, segs):
    assert oracle.validate_rotate_paged(PS, 8, segs) == want


def library_status(segs, page_size=PS, n_phys=8, layers=(0, 2)):
    """pic_rotate_paged's status for a bf16 GQA shape (refused calls never
    reach the view, which is a dummy)."""
    from position_independent_kv_stitch_amd import _binding as B
    lib = B.load_library()
    shape, rope, keep = B._shape_and_rope("bf16", 2, 2, 128, 0, 128, "half", 5e5, True, None)
    arr = (B.PageSegmentC * max(1, len(segs)))()
    for i, sg in enumerate(segs):
        pa = (C.c_int32 * len(sg.pages))(*sg.pages)
        keep.append(pa)
        cp = C.POINTER(C.c_int32)()
        if sg.cow is not None:
            ca = (C.c_int32 * len(sg.cow))(*sg.cow)
            keep.append(ca)
            cp = C.cast(ca, C.POINTER(C.c_int32))
        arr[i] = B.PageSegmentC(C.cast(pa, C.POINTER(C.c_int32)), cp, sg.delta, len(sg.pages),
                                sg.first, sg.length, sg.recompute_k)
    view = B.KvView(0x10000, 0x20000, 0, 0, 0, 0, 0)
    st = lib.pic_rotate_paged(C.byref(shape), C.byref(rope), C.byref(view), page_size, n_phys,
                              arr, len(segs), layers[0], layers[1], None)
    return st, lib.pic_last_error()


@pytest.mark.parametrize("want,segs", [r for r in RULES if r[0] != "ok"])
def test_library_refuses_what_the_oracle_refuses(want, segs):
    """The same statuses from the library, before any device work."""
    from position_independent_kv_stitch_amd import _binding as B
    code = {"range": B.PIC_ERR_RANGE, "bad_arg": B.PIC_ERR_INVALID_ARG,
            "overlap": B.PIC_ERR_OVERLAP}[want]
    st, msg = library_status(segs)
    assert st == code, msg


def test_library_refuses_bad_counts():
    from position_independent_kv_stitch_amd import _binding as B
    assert library_status([], page_size=0)[0] == B.PIC_ERR_INVALID_ARG
    assert library_status([], n_phys=0)[0] == B.PIC_ERR_INVALID_ARG
    assert library_status([seg([0], 0, 2)], layers=(1, 3))[0] == B.PIC_ERR_INVALID_ARG
    assert library_status([seg([0], 0, 2)], layers=(2, 1))[0] == B.PIC_ERR_INVALID_ARG


def mutate(segs, rng, n_phys, ps):
    """One random defect (or none) in a valid segment set."""
    segs = list(segs)
    g = int(rng.integers(0, len(segs)))
    sg = segs[g]
    kind = int(rng.integers(0, 8))
    pages, cow = list(sg.pages), (list(sg.cow) if sg.cow is not None else None)
    first, length, k, delta = sg.first, sg.length, sg.recompute_k, sg.delta
    if kind == 0:
        pages[int(rng.integers(0, len(pages)))] = int(rng.choice([n_phys, -1, n_phys + 3]))
    elif kind == 1:
        k = length + int(rng.integers(1, 3))
    elif kind == 2:
        first = ps + int(rng.integers(0, 3))
    elif kind == 3:
        pages = pages + [0]
    elif kind == 4 and len(segs) > 1:  # map another segment's page
        other = segs[(g + 1) % len(segs)]
        pages[int(rng.integers(0, len(pages)))] = int(rng.choice(other.pages))
    elif kind == 5 and cow is not None:  # a copy target onto a mapped page
        cow[int(rng.integers(0, len(cow)))] = int(rng.choice(pages))
    elif kind == 6 and len(segs) > 1 and segs[(g + 1) % len(segs)].cow is not None:
        oc = [c for c in segs[(g + 1) % len(segs)].cow if c >= 0]
        if oc:  # reuse another segment's copy target
            cow = cow or [-1] * len(pages)
            cow[int(rng.integers(0, len(cow)))] = int(rng.choice(oc))
    segs[g] = PageSegment(tuple(pages), tuple(cow) if cow is not None else None, delta, first,
                          length, k)
    return segs


def test_library_and_oracle_agree_on_mutated_sets():
    """Valid random sets with one random defect each: wherever the oracle
    refuses, the library gives the same status (valid sets are not sent:
    the library would launch)."""
    from position_independent_kv_stitch_amd import _binding as B
    code = {"range": B.PIC_ERR_RANGE, "bad_arg": B.PIC_ERR_INVALID_ARG,
            "overlap": B.PIC_ERR_OVERLAP}
    rng = np.random.default_rng(2024)
    refused = {k: 0 for k in code}
    for seed in range(300):
        wl, n_phys, segs = paged_cow_case(seed, page_size=4, max_len=12, n_chunks=3)
        bad = mutate(segs, rng, n_phys, 4)
        want = oracle.validate_rotate_paged(4, n_phys, bad)
        if want == "ok":
            continue
        refused[want] += 1
        st, msg = library_status(bad, page_size=4, n_phys=n_phys)
        assert st == code[want], (seed, want, msg)
    assert all(v > 5 for v in refused.values()), refused


def test_binding_page_lists():
    """The binding's page-list conversion: int32 arrays pass without a copy,
    other integer sequences are converted, ids outside int32 and non-integer
    ids are refused, and an empty list still gets a non-NULL pointer."""
    from position_independent_kv_stitch_amd._binding import _int32_array
    a = np.arange(5, dtype=np.int32)
    got, n = _int32_array(a)
    assert n == 5 and got is a
    got, n = _int32_array((3, 1, 2))
    assert n == 3 and got.dtype == np.int32 and got.tolist() == [3, 1, 2]
    got, n = _int32_array(np.array([7, 9], dtype=np.int64))
    assert got.dtype == np.int32 and got.tolist() == [7, 9]
    got, n = _int32_array([])
    assert n == 0 and got.size == 1 and got.ctypes.data != 0
    for bad in ([2 ** 31], [-2 ** 31 - 1]):
        with pytest.raises(ValueError):
            _int32_array(bad)
    with pytest.raises(TypeError):
        _int32_array([1.5, 2.0])
    with pytest.raises(ValueError):
        _int32_array([[1, 2]])
