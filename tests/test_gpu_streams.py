"""One plan used from two HIP streams at once: pic_attend (matrix-core and
vector paths), pic_attend_latent and pic_attend_boundary calls on the same
plan are enqueued alternately on two streams without waiting, so their
kernels overlap.  Each stream has its own partial-result workspace and the
plan's metadata is uploaded once (on whichever stream first needs it, the
other stream waiting for the upload), so every output must equal the
oracle within the bounds the single-stream tests use.  Streams keep the
default priority."""
import sys

import numpy as np
import pytest

import oracle
from parity_util import to_host
from pic_workloads import normal_values, pool_values, random_small

pytestmark = pytest.mark.gpu
U = 2.0 ** -24
ROUNDS = 4


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


def f64(bits):
    return oracle.ref._to_f64(bits)


def with_context(wl, rng, extra=7):
    for rq in wl.requests:
        end = max([e.dst_offset + e.length for e in rq.entries] + [1])
        span = len(rq.page_table) * wl.page_size if wl.page_size else wl.capacity
        rq.context_len = int(min(span, end + int(rng.integers(0, extra + 1))))
    return wl


def matrix_bound(hq, keys, vals, scale):
    """The worst-case error of the matrix-core attention kernels (fp32
    logits and sums, weights as two bf16 terms) for queries hq over the
    given key and value rows, as derived for the latent and boundary
    parity tests."""
    s = np.abs(f64(hq)).reshape(-1, hq.shape[-1]) @ np.abs(f64(keys)).T
    dz = scale * (hq.shape[-1] + 1) * U * float(s.max())
    return 2 * (2 * dz + 1e-5 + 2.0 ** -16 + 300 * U) * float(np.abs(f64(vals)).max())


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_attend_one_plan_two_streams(torch_cuda, dt):
    """bf16 128-dim rows take the matrix-core path, f32 the vector kernels."""
    torch = torch_cuda
    import position_independent_kv_stitch_amd as pic
    rng = np.random.default_rng(3)
    wl = with_context(random_small(61, dtype=dt, paged=True, n_requests=3, n_layers=1,
                                   max_len=300, deltas=[0, 5, -300, 65536]), rng)
    pk, pv = pool_values(wl, seed=1, device="cuda:0")
    ck = normal_values(wl.dst_shape(), dt, 2, "cuda:0")
    cv = normal_values(wl.dst_shape(), dt, 3, "cuda:0")
    qs = [normal_values((len(wl.requests), wl.n_heads * 4, wl.row_dim), dt, 10 + i, "cuda:0")
          for i in range(2)]
    outs = [torch.empty(q.shape, dtype=torch.float32, device="cuda:0") for q in qs]
    plan = pic.Plan.from_workload(wl)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    for _ in range(ROUNDS):
        for q, out, st in zip(qs, outs, streams):
            pic.attend(plan, pk, pv, ck, cv, q, layer=0, out=out, sink_tokens=4, sink_bias=-15.0,
                       stream=st)
    torch.cuda.synchronize()
    hcv, hpv = to_host(cv), to_host(pv)
    vmax = max(np.abs(f64(hcv)).max(), np.abs(f64(hpv)).max())
    for i, (q, out) in enumerate(zip(qs, outs)):
        want = oracle.attend(wl, to_host(pk), hpv, to_host(ck), hcv, to_host(q), 0,
                             sink_tokens=4, sink_bias=-15.0)
        err = float(np.abs(out.cpu().numpy().astype(np.float64) - want).max())
        say(f"attend {dt} stream {i}: max err {err:.3g}")
        assert err <= 5e-4 * vmax, (i, err, vmax)
    plan.destroy()


def test_attend_latent_one_plan_two_streams(torch_cuda):
    torch = torch_cuda
    import position_independent_kv_stitch_amd as pic
    rng = np.random.default_rng(4)
    wl = with_context(random_small(62, dtype="bf16", mla=True, paged=True, n_requests=3,
                                   n_layers=1, max_len=300), rng)
    pk, _ = pool_values(wl, seed=1, device="cuda:0")
    ck = normal_values(wl.dst_shape(), "bf16", 2, "cuda:0")
    scale = 192 ** -0.5
    qs = [normal_values((len(wl.requests), 32, 576), "bf16", 20 + i, "cuda:0") for i in range(2)]
    outs = [torch.empty((len(wl.requests), 32, 512), dtype=torch.float32, device="cuda:0")
            for _ in qs]
    plan = pic.Plan.from_workload(wl)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    for _ in range(ROUNDS):
        for q, out, st in zip(qs, outs, streams):
            pic.attend_latent(plan, pk, ck, q, layer=0, out=out, scale=scale, stream=st)
    torch.cuda.synchronize()
    hpk, hck = to_host(pk), to_host(ck)
    rows = np.concatenate([hpk.reshape(-1, 576), hck.reshape(-1, 576)])
    for i, (q, out) in enumerate(zip(qs, outs)):
        hq = to_host(q)
        want = oracle.attend_latent(wl, hpk, hck, hq, 0, scale=scale)
        err = float(np.abs(out.cpu().numpy().astype(np.float64) - want).max())
        tol = matrix_bound(hq, rows, rows[:, :512], scale)
        say(f"attend_latent stream {i}: max err {err:.3g} (tol {tol:.3g})")
        assert err <= tol, (i, err, tol)
    plan.destroy()


def test_attend_latent_workspace_grows(torch_cuda):
    """The plan keeps a partial-result workspace per stream and replaces it
    by a larger one when a call needs more (the need grows with the query
    heads): calls at 16, 128, 32 and 256 heads alternate over two streams
    without waiting, and the plan is destroyed right after they are
    enqueued.  Destroy must wait for every call, including those that used a
    workspace since replaced, and every output must match the oracle."""
    torch = torch_cuda
    import position_independent_kv_stitch_amd as pic
    rng = np.random.default_rng(6)
    wl = with_context(random_small(65, dtype="bf16", mla=True, paged=True, n_requests=3,
                                   n_layers=1, max_len=300), rng)
    pk, _ = pool_values(wl, seed=3, device="cuda:0")
    ck = normal_values(wl.dst_shape(), "bf16", 4, "cuda:0")
    scale = 192 ** -0.5
    heads = [16, 128, 32, 256, 16, 128]
    qs = [normal_values((len(wl.requests), h, 576), "bf16", 40 + i, "cuda:0")
          for i, h in enumerate(heads)]
    outs = [torch.empty((len(wl.requests), h, 512), dtype=torch.float32, device="cuda:0")
            for h in heads]
    plan = pic.Plan.from_workload(wl)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    for i, (q, out) in enumerate(zip(qs, outs)):
        pic.attend_latent(plan, pk, ck, q, layer=0, out=out, scale=scale,
                          stream=streams[(i // 2) % 2])
    plan.destroy()
    torch.cuda.synchronize()
    hpk, hck = to_host(pk), to_host(ck)
    rows = np.concatenate([hpk.reshape(-1, 576), hck.reshape(-1, 576)])
    for i, (q, out) in enumerate(zip(qs, outs)):
        hq = to_host(q)
        want = oracle.attend_latent(wl, hpk, hck, hq, 0, scale=scale)
        err = float(np.abs(out.cpu().numpy().astype(np.float64) - want).max())
        tol = matrix_bound(hq, rows, rows[:, :512], scale)
        say(f"attend_latent call {i} ({heads[i]} heads): max err {err:.3g} (tol {tol:.3g})")
        assert err <= tol, (i, err, tol)


def test_attend_boundary_one_plan_two_streams(torch_cuda):
    torch = torch_cuda
    import position_independent_kv_stitch_amd as pic
    wl = random_small(63, dtype="bf16", paged=True, n_requests=3, n_layers=1, max_len=300)
    pk, pv = pool_values(wl, seed=1, device="cuda:0")
    ck = normal_values(wl.dst_shape(), "bf16", 2, "cuda:0")
    cv = normal_values(wl.dst_shape(), "bf16", 3, "cuda:0")
    plan = pic.Plan.from_workload(wl)
    k, scale = 8, 0.09
    n = pic.boundary_row_count(plan, k)
    assert n == len(oracle.boundary_rows(wl, k)) and n > 0
    qs = [normal_values((n, wl.n_heads * 4, wl.row_dim), "bf16", 30 + i, "cuda:0")
          for i in range(2)]
    outs = [torch.empty(q.shape, dtype=torch.float32, device="cuda:0") for q in qs]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    for _ in range(ROUNDS):
        for q, out, st in zip(qs, outs, streams):
            pic.attend_boundary(plan, pk, pv, ck, cv, q, layer=0, boundary_k=k, out=out,
                                scale=scale, stream=st)
    torch.cuda.synchronize()
    hpk, hpv, hck, hcv = to_host(pk), to_host(pv), to_host(ck), to_host(cv)
    keys = np.concatenate([hpk.reshape(-1, wl.row_dim), hck.reshape(-1, wl.row_dim)])
    vals = np.concatenate([hpv.reshape(-1, wl.row_dim), hcv.reshape(-1, wl.row_dim)])
    for i, (q, out) in enumerate(zip(qs, outs)):
        hq = to_host(q)
        want = oracle.attend_boundary(wl, hpk, hpv, hck, hcv, hq, 0, k, scale=scale)
        err = float(np.abs(out.cpu().numpy().astype(np.float64) - want).max())
        tol = matrix_bound(hq, keys, vals, scale)
        say(f"attend_boundary stream {i}: {n} rows, max err {err:.3g} (tol {tol:.3g})")
        assert err <= tol, (i, err, tol)
    plan.destroy()


def test_plan_destroyed_while_other_streams_run(torch_cuda):
    """pic_plan_destroy waits for the plan's own work on every stream it ran
    on (not the whole device): a plan destroyed right after enqueueing
    stitches on two streams leaves both results complete."""
    torch = torch_cuda
    import position_independent_kv_stitch_amd as pic
    from parity_util import compare_bits, compare_k, max_abs
    from pic_workloads import sentinel_like
    wl = random_small(64, dtype="bf16", paged=True, n_requests=3, n_layers=3, max_len=300)
    pk, pv = pool_values(wl, seed=2, device="cuda:0")
    dsts = [(sentinel_like(wl.dst_shape(), "bf16", "cuda:0"),
             sentinel_like(wl.dst_shape(), "bf16", "cuda:0")) for _ in range(2)]
    plan = pic.Plan.from_workload(wl)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    for (dk, dv), st in zip(dsts, streams):
        pic.stitch(plan, pk, pv, dk, dv, stream=st)
    plan.destroy()
    torch.cuda.synchronize()
    rk = to_host(sentinel_like(wl.dst_shape(), "bf16", "cpu"))
    rv = rk.copy()
    assert oracle.stitch(wl, to_host(pk), to_host(pv), rk, rv) == "ok"
    for i, (dk, dv) in enumerate(dsts):
        stats = compare_k(to_host(dk), rk, wl.rope_offset, wl.rope_dim, max_abs(to_host(pk)))
        compare_bits(to_host(dv), rv, f"V stream {i}")
        say(f"stitch stream {i}: {stats}")
