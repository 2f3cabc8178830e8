"""pic_rotate_inplace_noalloc (the entry point for callers that cannot
allocate) against pic_rotate_inplace: the same kernels on metadata staged
in the library's static device array instead of stream-ordered memory, so
the results must be bit-identical.  Two calls in a row, the second smaller,
enqueued back to back (the second overwrites the array the first used, in
stream order); the smaller case is also checked against the oracle."""
import sys

import numpy as np
import pytest

import oracle
from parity_util import compare_k, max_abs, to_host
from pic_workloads import Segment, Workload, config5, normal_values

pytestmark = pytest.mark.gpu


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


def small_case(seed):
    rng = np.random.default_rng(seed)
    segs, at = [], 0
    for _ in range(5):
        n = int(rng.integers(1, 300))
        segs.append(Segment(at, n, int(rng.integers(-65536, 65537)), int(rng.integers(0, 9))))
        at += n + int(rng.integers(0, 4))
    return Workload("no-alloc small", "bf16", 3, 8, 128, 0, 128, "half", 1e6, False,
                    inplace=True, n_tokens=at, segments=segs)


def run(pic, wl, buf, noalloc):
    pic.rotate_inplace(buf, wl.segments, rope_dim=wl.rope_dim, theta=wl.theta, style=wl.style,
                       rope_offset=wl.rope_offset, noalloc=noalloc)


def test_noalloc_equals_rotate_inplace_two_calls(torch_cuda):
    torch = torch_cuda
    import position_independent_kv_stitch_amd as pic
    big = config5(n_layers=4)  # 64 segments x 2048 tokens: 318 KiB of staged metadata
    small = small_case(5)
    cases = [(big, normal_values(big.buf_shape(), "bf16", 1, "cuda:0")),
             (small, normal_values(small.buf_shape(), "bf16", 2, "cuda:0"))]
    refs = [buf.clone() for _, buf in cases]
    before = to_host(cases[1][1])  # the small call's input, for the oracle
    torch.cuda.synchronize()
    say("no-alloc: two calls back to back (big, then small)")
    for wl, buf in cases:
        run(pic, wl, buf, noalloc=True)
    for (wl, _), ref in zip(cases, refs):
        run(pic, wl, ref, noalloc=False)
    torch.cuda.synchronize()
    for i, ((wl, buf), ref) in enumerate(zip(cases, refs)):
        same = torch.equal(buf.view(torch.int16), ref.view(torch.int16))
        say(f"  call {i} ({len(wl.segments)} segments, {wl.n_tokens} tokens): identical={same}")
        assert same
    wl, buf = cases[1]
    want = before.copy()
    assert oracle.rotate_inplace(wl, want) == "ok"
    stats = compare_k(to_host(buf), want, 0, 128, max_abs(before), what="no-alloc small")
    say(f"  small call vs the oracle: {stats}")


def test_noalloc_repeated_calls_reuse_the_array(torch_cuda):
    """Six calls on separate buffers enqueued without waiting (each call's
    fill kernels overwrite the array after the previous call's rotation, in
    stream order), each equal to pic_rotate_inplace."""
    torch = torch_cuda
    import position_independent_kv_stitch_amd as pic
    cases = [small_case(20 + i) for i in range(6)]
    bufs = [normal_values(wl.buf_shape(), "bf16", 30 + i, "cuda:0") for i, wl in enumerate(cases)]
    refs = [b.clone() for b in bufs]
    torch.cuda.synchronize()
    for wl, b in zip(cases, bufs):
        run(pic, wl, b, noalloc=True)
    for wl, r in zip(cases, refs):
        run(pic, wl, r, noalloc=False)
    torch.cuda.synchronize()
    for i, (b, r) in enumerate(zip(bufs, refs)):
        assert torch.equal(b.view(torch.int16), r.view(torch.int16)), i
