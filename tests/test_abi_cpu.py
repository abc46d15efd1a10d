"""The C-ABI library on the CPU: it loads, exports every symbol the header
declares, rejects bad arguments before enqueueing anything, and its host-side
helpers (segment grouping, pool pointer table) are right. No compute call is
made here: every call below returns during argument checks."""
import ctypes
import re
from pathlib import Path

import numpy as np
import pytest

import oracle as oracle_pkg
import segmented_gather_gemm_sgmv_amd as sg

from . import oracle_pins as pins
from . import workloads as wl

HEADER = Path(__file__).resolve().parents[1] / "include" / "sgmv.h"


def declared_functions():
    text = re.sub(r"/\*.*?\*/", "", HEADER.read_text(), flags=re.S)
    return sorted(set(re.findall(r"\b(sgmv_\w+)\s*\(", text)))


def test_header_declares_the_abi():
    assert declared_functions() == sorted(sg.EXPORTS)


@pytest.mark.parametrize("name", declared_functions())
def test_symbol_exported(name):
    assert hasattr(sg.lib, name)


def test_workspace_status_and_wait_limit_on_the_host():
    # argument errors return before any HIP call
    word = ctypes.c_uint32(0)
    assert sg.lib.sgmv_workspace_status(None, ctypes.byref(word), None) == -1
    assert sg.lib.sgmv_workspace_status(P1, None, None) == -1
    # the limit is a process-wide setting: set, read back, restore
    old = sg.sgmv_set_wait_limit(7)
    try:
        assert sg.sgmv_set_wait_limit(0) == 7
        assert sg.sgmv_set_wait_limit(1 << 20) == 0
    finally:
        assert sg.sgmv_set_wait_limit(old) == 1 << 20
    assert old == 1 << 15


def test_status_strings():
    for st in range(-9, 1):
        assert sg.lib.sgmv_status_string(st)
    assert sg.lib.sgmv_status_string(-99) == b"unknown status"


# Distinct 256-byte aligned fake device addresses. They are never
# dereferenced: each call below fails its argument checks (or is a no-op)
# before anything is enqueued.
P1, P2, P3, P4, P5, P6, P7 = (0x100000 * (i + 1) for i in range(7))


def shrink(V=P1, X=P2, A=P3, P=4, ss=P4, sa=P5, N=2, M=4, d_in=64, r=16, dt=1, ws=0x800000,
           wsb=1 << 20):
    return sg.lib.sgmv_shrink(V, X, A, P, ss, sa, N, M, d_in, r, dt, ws, wsb, None)


def expand(Y=P1, V=P2, B=P3, P=4, ss=P4, sa=P5, N=2, M=4, d_out=64, r=16, alpha=32.0, dt=1):
    return sg.lib.sgmv_expand(Y, V, B, P, ss, sa, N, M, d_out, r, alpha, dt, None)


def fused(Y=P1, X=P2, A=P3, B=P6, P=4, ss=P4, sa=P5, N=2, M=4, d_in=64, d_out=64, r=16, dt=1,
          ws=0x800000, wsb=1 << 20):
    return sg.lib.sgmv_fused(Y, X, A, B, P, ss, sa, N, M, d_in, d_out, r, 32.0, dt, ws, wsb, None)


def shrink_gather(V=P1, X=P2, rows=P7, A=P3, P=4, ss=P4, sa=P5, N=2, M=4, d_in=64, r=16, dt=1,
                  ws=0x800000, wsb=1 << 20):
    return sg.lib.sgmv_shrink_gather(V, X, rows, A, P, ss, sa, N, M, d_in, r, dt, ws, wsb, None)


def expand_scatter(Y=P1, V=P2, rows=P7, B=P3, P=4, ss=P4, sa=P5, N=2, M=4, d_out=64, r=16, alpha=32.0,
                   dt=1):
    return sg.lib.sgmv_expand_scatter(Y, V, rows, B, P, ss, sa, N, M, d_out, r, alpha, dt, None)


def fused_gather(Y=P1, X=P2, rows=P7, A=P3, B=P6, P=4, ss=P4, sa=P5, N=2, M=4, d_in=64, d_out=64, r=16,
                 dt=1, ws=0x800000, wsb=1 << 20):
    return sg.lib.sgmv_fused_gather(Y, X, rows, A, B, P, ss, sa, N, M, d_in, d_out, r, 32.0, dt, ws, wsb,
                                    None)


ALL_CALLS = [shrink, expand, fused, shrink_gather, expand_scatter, fused_gather]
GATHERED = [shrink_gather, expand_scatter, fused_gather]


@pytest.mark.parametrize("call", ALL_CALLS, ids=lambda f: f.__name__)
def test_argument_errors(call):
    assert call(r=12) == -3 and call(r=0) == -3 and call(r=128) == -3
    assert call(dt=2) == -4 and call(dt=-1) == -4
    assert call(M=-1) == -2 and call(N=-1) == -2 and call(P=-1) == -2
    dim = "d_out" if call in (expand, expand_scatter) else "d_in"
    assert call(**{dim: 12}) == -2 and call(**{dim: 0}) == -2
    first = "V" if call in (shrink, shrink_gather) else "Y"
    assert call(**{first: None}) == -1
    assert call(ss=None) == -1 and call(sa=None) == -1
    assert call(**{first: P1 + 8}) == -5


@pytest.mark.parametrize("call", ALL_CALLS, ids=lambda f: f.__name__)
def test_launches_beyond_the_dispatch_limit_are_refused(call):
    """A call whose launch would need more than 2^24 workgroups (2^32
    work-items in one dispatch) is refused before anything is enqueued:
    2^24 segments of one row each, rank 64 (16 shrink workgroups per
    segment). Half as many segments at rank 8 fit, and fail only the
    later (pointer) check."""
    big = dict(N=1 << 24, M=1 << 24)
    assert call(**big, r=64) == -2
    assert call(N=1 << 20, M=1 << 20, r=8, ss=None) == -1
    if call in (fused, fused_gather):
        assert sg.lib.sgmv_workspace_bytes(1 << 24, 1 << 24, 64, 64, 64, 1) == 0
        assert sg.lib.sgmv_workspace_bytes(1 << 20, 1 << 20, 64, 64, 8, 1) > 0


@pytest.mark.parametrize("call", ALL_CALLS, ids=lambda f: f.__name__)
def test_empty_is_noop(call):
    # nothing to do: OK without touching any pointer, even NULL ones
    first = "V" if call in (shrink, shrink_gather) else "Y"
    assert call(M=0, **{first: None}) == 0
    assert call(N=0, ss=None, sa=None) == 0


@pytest.mark.parametrize("call", GATHERED, ids=lambda f: f.__name__)
def test_gathered_calls_need_rows(call):
    assert call(rows=None) == -1
    assert call(M=0, rows=None) == 0
    assert call(rows=None, r=12) == -3   # the same order of checks as the contiguous call


def test_fused_workspace_checks():
    need = sg.lib.sgmv_workspace_bytes(2, 4, 64, 64, 16, 1)
    assert need >= 8 * 2 + 4 * 4 * 16
    assert fused(ws=None) == -6
    assert fused(wsb=need - 1) == -6
    assert fused(ws=0x800000 + 16) == -6   # not 256-byte aligned
    assert sg.lib.sgmv_workspace_bytes(2, 4, 64, 64, 12, 1) == 0


def test_shrink_workspace_checks():
    # one 16-row bf16 tile with a very long reduction (d_in = 28672, r = 64)
    # splits d_in between workgroups: a workspace is needed
    need = sg.lib.sgmv_workspace_bytes(1, 16, 28672, 4096, 64, 1)
    assert need > 2 * 16 * 64 * 4
    assert shrink(M=16, d_in=28672, r=64, ws=None, wsb=0) == -6
    # the parts' partial tiles alone (16 x 64 fp32 each) exceed 4 KB
    assert shrink(M=16, d_in=28672, r=64, wsb=4096) == -6
    assert shrink(M=16, d_in=28672, r=64, ws=0x800000 + 16, wsb=need) == -6
    # fp32 never needs one (no MFMA path): NULL is fine; argument errors still win
    assert shrink(M=64, d_in=4096, dt=0, ws=None, wsb=0, r=12) == -3


def test_workspace_bytes_grows_with_rows():
    # fp32 has no MFMA split, so only the fused kernel's V (M x r fp32) grows
    a = sg.lib.sgmv_workspace_bytes(64, 64, 4096, 4096, 16, 0)
    b = sg.lib.sgmv_workspace_bytes(64, 640, 4096, 4096, 16, 0)
    assert b - a >= 576 * 16 * 4


def test_build_segments_matches_oracle():
    pins.pin_segments(sg.sgmv_build_segments)
    rng = np.random.Generator(np.random.PCG64(30))
    for _ in range(50):
        ids = rng.integers(0, 9, size=int(rng.integers(0, 60))).astype(np.int32)
        got = sg.sgmv_build_segments(ids)
        want = oracle_pkg.build_segments(ids)
        for g, w in zip(got, want):
            assert np.array_equal(g, w)


def test_build_segments_rejects_negative_ids():
    with pytest.raises(sg.SGMVError):
        sg.sgmv_build_segments([0, -1, 2])


def test_pool_pointers_host():
    table = np.zeros(5, np.uint64)
    base = 0x7F0000000000
    assert sg.lib.sgmv_pool_pointers(table.ctypes.data, base, 5, 4096) == 0
    assert list(table) == [base + 4096 * k for k in range(5)]
    assert sg.lib.sgmv_pool_pointers(table.ctypes.data, base, 5, 4100) == -5
    assert sg.lib.sgmv_pool_pointers(table.ctypes.data, None, 5, 4096) == -1
    assert sg.lib.sgmv_pool_pointers(None, None, 0, 4096) == 0


def test_decode_skewed_segments_via_library():
    w = wl.decode_skewed(sg.sgmv_build_segments)
    _, ss, sa = oracle_pkg.build_segments(w.token_adapter)
    assert np.array_equal(ss, w.seg_start) and np.array_equal(sa, w.seg_adapter)
    assert w.M == 256 and w.seg_start[-1] == 256


def test_pointer_table_keeps_pool_alive():
    """A device pointer table must never outlive the pool it points into."""
    import gc
    import weakref

    import torch
    pool = torch.zeros((3, 8, 16), dtype=torch.bfloat16)
    ref = weakref.ref(pool)
    table = sg.sgmv_pool_pointers(pool)
    assert table.tolist() == [pool.data_ptr() + k * 8 * 16 * 2 for k in range(3)]
    del pool
    gc.collect()
    assert ref() is not None
    del table
    gc.collect()
    assert ref() is None


# -- the layer call --------------------------------------------------------------
def projections(n=3, d_in=64, d_out=64, P=4, **over):
    arr = (sg.SgmvProjection * max(n, 1))()
    for q in range(n):
        fields = dict(Y=P1 + q * 0x1000, X=P2 + q * 0x1000, A_ptrs=P3, B_ptrs=P6, num_adapters=P,
                      d_in=d_in, d_out=d_out)
        if q == n - 1:
            fields.update(over)   # overrides land on the last projection
        arr[q] = sg.SgmvProjection(**fields)
    return arr


def layer(arr=None, n=3, rows=None, ss=P4, sa=P5, N=2, M=4, r=16, dt=1, ws=0x800000, wsb=1 << 20):
    arr = projections(n) if arr is None else arr
    return sg.lib.sgmv_fused_layer(arr, n, rows, ss, sa, N, M, r, 32.0, dt, ws, wsb, None)


def test_layer_argument_errors():
    assert layer(r=12) == -3 and layer(dt=2) == -4
    assert layer(n=9, arr=projections(9)) == -2 and layer(n=-1) == -2
    assert sg.lib.sgmv_fused_layer(None, 2, None, P4, P5, 2, 4, 16, 32.0, 1, 0x800000, 1 << 20, None) == -1
    assert layer(M=-1) == -2 and layer(N=-1) == -2
    assert layer(arr=projections(3, num_adapters=-1)) == -2
    assert layer(arr=projections(3, d_in=12)) == -2 and layer(arr=projections(3, d_out=0)) == -2
    assert layer(arr=projections(3, Y=None)) == -1 and layer(arr=projections(3, X=None)) == -1
    assert layer(arr=projections(3, A_ptrs=None)) == -1 and layer(arr=projections(3, B_ptrs=None)) == -1
    assert layer(ss=None) == -1 and layer(sa=None) == -1
    assert layer(arr=projections(3, Y=P1 + 8)) == -5
    assert layer(ws=None) == -6 and layer(ws=0x800000 + 16) == -6


def test_layer_empty_is_noop():
    assert layer(n=0, arr=projections(0)) == 0
    assert layer(M=0, ss=None, sa=None) == 0
    assert layer(N=0, ss=None, sa=None) == 0
    assert sg.lib.sgmv_fused_layer(None, 0, None, None, None, 2, 4, 16, 32.0, 1, None, 0, None) == 0


def test_layer_workspace_is_the_sum_of_the_projections():
    arr = projections(3, d_in=4096)
    for q, d_in in enumerate((64, 1024, 4096)):
        arr[q].d_in = d_in
    total = sg.lib.sgmv_layer_workspace_bytes(arr, 3, 5, 300, 16, 1)
    parts = [sg.lib.sgmv_workspace_bytes(5, 300, d, 64, 16, 1) for d in (64, 1024, 4096)]
    assert total >= sum(parts) and total <= sum(parts) + 3 * 256 + 3 * (1 << 20)
    assert layer(arr=arr, N=5, M=300, wsb=total - 1) == -6
    assert sg.lib.sgmv_layer_workspace_bytes(arr, 9, 5, 300, 16, 1) == 0


def admit(A_slot=P1, B_slot=P2, A_host=P3, B_host=P4, Ab=1024, Bb=2048, A_ptrs=P5, B_ptrs=P6, slot=1, P=4):
    return sg.lib.sgmv_admit_adapter(A_slot, B_slot, A_host, B_host, Ab, Bb, A_ptrs, B_ptrs, slot, P, None)


def test_admit_argument_errors():
    for k in ("A_slot", "B_slot", "A_host", "B_host", "A_ptrs", "B_ptrs"):
        assert admit(**{k: None}) == -1
    assert admit(slot=-1) == -2 and admit(slot=4) == -2 and admit(P=0, slot=0) == -2
    assert admit(Ab=0) == -2 and admit(Bb=0) == -2
    assert admit(A_slot=P1 + 8) == -5 and admit(B_slot=P2 + 4) == -5


def test_check_segments():
    ok = sg.sgmv_check_segments
    ok([0, 1, 3, 3, 8], [2, 0, 3, 1], 8, 4)              # an empty segment is fine
    ok([0], [], 0, 4)
    pins.check_segments([2, 0, 3, 1], *oracle_pkg.build_segments(np.array([2, 0, 3, 1])))
    perm, ss, sa = sg.sgmv_build_segments(np.array([5, 1, 5, 0], np.int32))
    ok(ss, sa, 4, 6)
    for bad_start, bad_ids, M, P, status in [
        ([1, 3, 8], [0, 1], 8, 4, -2),       # does not start at 0
        ([0, 3, 7], [0, 1], 8, 4, -2),       # does not end at M
        ([0, 5, 3, 8], [0, 1, 2], 8, 4, -2),  # decreasing
        ([0, 3, 8], [0, 4], 8, 4, -8),       # id outside the pool
        ([0, 3, 8], [-1, 1], 8, 4, -8),      # negative id
        ([0], [], 3, 4, -2),                 # no segment cannot cover 3 rows
    ]:
        with pytest.raises(sg.SGMVError) as e:
            ok(bad_start, bad_ids, M, P)
        assert e.value.status == status
    assert sg.lib.sgmv_check_segments(None, None, 0, 0, 1) == -1
    with pytest.raises(ValueError):
        ok([0, 8], [0, 1], 8, 4)
