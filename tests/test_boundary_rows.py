"""pic_attend_boundary with caller-given (entry, token) rows: every argument
rule is checked on the host before any device work, so the refusals run
without a GPU (the views and q are dummies that are never read)."""
import ctypes as C

import numpy as np
import pytest

import position_independent_kv_stitch_amd as pic
from position_independent_kv_stitch_amd import _binding as B
from pic_workloads import Chunk, Entry, Request, Workload


def plan_of():
    # two requests; entries in plan order: 0 (r0 at 0, len 20), 1 (r0 at 30, len 10),
    # 2 (r1 at 5, len 15); contexts end at 40 and 20
    wl = Workload("rows", "bf16", 1, 2, 128, 0, 128, "half", 5e5, True, pool_tokens=40,
                  chunks=[Chunk(0, 20), Chunk(20, 20)], capacity=64,
                  requests=[Request([Entry(0, 0, 20), Entry(1, 30, 10)], None, 40),
                            Request([Entry(1, 5, 15)], None, 20)])
    return pic.Plan.from_workload(wl)


def status(plan, rows, n_rows=None, reserved=0, boundary_k=0):
    lib = plan._lib
    arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int32).reshape(-1, 2)) if rows is not None \
        else None
    ptr = arr.ctypes.data_as(C.POINTER(C.c_int32)) if arr is not None else None
    n = (len(arr) if arr is not None else 0) if n_rows is None else n_rows
    a = B.BoundaryArgs(0x100000, 8 * 128, 128, 0x200000, 8 * 128, 128, 8, 0, 0.09, boundary_k,
                       0, 0.0, ptr, n, reserved)
    view = B.KvView(0x10000, 0x20000, 0, 2 * 128, 128, 0, 64 * 2 * 128)
    st = lib.pic_attend_boundary(plan.handle, C.byref(view), C.byref(view), C.byref(a), None)
    return st, lib.pic_last_error().decode()


@pytest.mark.parametrize("rows,want", [
    ([(3, 0)], B.PIC_ERR_RANGE),               # entry outside the plan
    ([(-1, 0)], B.PIC_ERR_RANGE),
    ([(1, 10)], B.PIC_ERR_RANGE),              # token past the entry's length
    ([(0, -1)], B.PIC_ERR_RANGE),
    ([(2, 0), (1, 0)], B.PIC_ERR_INVALID_ARG),  # request 1 before request 0
    ([(0, 3), (2, 0), (1, 1)], B.PIC_ERR_INVALID_ARG),
])
def test_bad_rows_are_refused(rows, want):
    plan = plan_of()
    st, msg = status(plan, rows)
    assert st == want, msg
    plan.destroy()


def test_bad_counts_are_refused():
    plan = plan_of()
    assert status(plan, [(0, 1)], n_rows=-1)[0] == B.PIC_ERR_INVALID_ARG
    assert status(plan, [(0, 1)], reserved=1)[0] == B.PIC_ERR_INVALID_ARG
    assert status(plan, None, boundary_k=0)[0] == B.PIC_ERR_INVALID_ARG  # no rows: k >= 1
    plan.destroy()


def test_rows_beyond_a_short_context_are_refused():
    """Request 1's context ends at position 19 (entry 2 spans [5, 20)); a
    row at its last token is inside, but the plan with a 12-position context
    refuses tokens past position 11."""
    wl = Workload("rows", "bf16", 1, 2, 128, 0, 128, "half", 5e5, True, pool_tokens=40,
                  chunks=[Chunk(0, 20), Chunk(20, 20)], capacity=64,
                  requests=[Request([Entry(1, 5, 15)], None, 12)])
    plan = pic.Plan.from_workload(wl)
    assert status(plan, [(0, 7)])[0] == B.PIC_ERR_RANGE   # position 12
    plan.destroy()


def test_no_rows_enqueue_nothing():
    """An empty row list is valid and enqueues nothing (no device work)."""
    plan = plan_of()
    assert status(plan, np.zeros((0, 2), np.int32))[0] == B.PIC_OK
    plan.destroy()
