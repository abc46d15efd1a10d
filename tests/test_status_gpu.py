"""GPU tests of the workspace status word: failures seen on the device reach
the host, a failed workspace turns later calls into no-ops until it is
zero-filled, and every kernel ends.

Failure conditions are forced from the host only: offsets that decrease
(invalid metadata the kernels must contain), and a wait limit of zero polls
(each wait then gives up unless its result is already there at the first
poll). No test makes a kernel fault or hang: every access stays inside the
documented buffers and every wait is bounded.
"""
import numpy as np
import pytest
import torch

import segmented_gather_gemm_sgmv_amd as sg

from . import workloads as wl
from .gpu_common import TOL, assert_close, bits, oracle_bits, oracle_run, run_fused, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def control_zero(ws: torch.Tensor) -> bool:
    return int(torch.count_nonzero(ws)) == 0


def _case(rng, lengths, d_in, d_out, r=16, P=4, dtype=torch.bfloat16, starts=None):
    ids = rng.integers(0, P, size=len(lengths)).astype(np.int32)
    ss = wl.segments_from_lengths(lengths) if starts is None else np.asarray(starts, np.int32)
    M = int(sum(lengths)) if starts is None else int(starts[-1])
    w = wl.Workload("status", M, d_in, d_out, r, 2.0 * r, dtype, P, ss, ids)
    wl.fill_tensors(w, rng)
    w.Y = wl._normal(rng, (w.M, w.d_out), 1.0, dtype)
    return w


def _workspace(dev, w):
    need = sg.sgmv_workspace_bytes(w.num_segments, w.M, w.d_in, w.d_out, w.r, w.dtype)
    return torch.zeros(max(need, 256), dtype=torch.uint8, device=dev)


@pytest.mark.parametrize("starts", [[0, 10, 5, 20], [0, 40, 20, 80], [0, 3, 1, 50, 48, 64]],
                         ids=["vector", "mfma", "mixed"])
def test_decreasing_offsets_are_reported(dev, oracle, starts):
    """Offsets that decrease make segments share rows. The fused call ends,
    writes nothing outside Y, and reports SGMV_WS_BAD_OFFSETS; later calls on
    that workspace leave Y untouched until it is zero-filled, after which a
    valid call gives the oracle's result and leaves the workspace zero."""
    rng = np.random.Generator(np.random.PCG64(200 + len(starts)))
    M = starts[-1]
    bad = _case(rng, [1] * (len(starts) - 1), 512, 264, starts=starts)
    good = _case(rng, [3, 20, 1, 10], 512, 264)
    c = to_device(bad, dev)
    WS = torch.zeros(max(_workspace(dev, bad).numel(), _workspace(dev, good).numel()), dtype=torch.uint8,
                     device=dev)
    Ybuf = torch.full((M * bad.d_out + 4096,), -7.0, dtype=bad.dtype, device=dev)
    Y = Ybuf[:M * bad.d_out].view(M, bad.d_out)
    Y.copy_(c.Y0)
    sg.sgmv_fused(Y, c.X, c.A_ptrs, c.B_ptrs, c.seg_start, c.seg_adapter, bad.r, bad.alpha, workspace_buf=WS)
    torch.cuda.synchronize()
    assert torch.all(Ybuf[M * bad.d_out:] == -7.0)
    st = sg.sgmv_workspace_status(WS)
    assert st & sg.SGMV_WS_BAD_OFFSETS, st
    # a valid batch on the failed workspace: a no-op
    g = to_device(good, dev)
    Yg = g.Y0.clone()
    sg.sgmv_fused(Yg, g.X, g.A_ptrs, g.B_ptrs, g.seg_start, g.seg_adapter, good.r, good.alpha, workspace_buf=WS)
    torch.cuda.synchronize()
    assert torch.equal(Yg, g.Y0)
    assert sg.sgmv_workspace_status(WS) & sg.SGMV_WS_BAD_OFFSETS
    # zero-filled again: calls work and leave it zero
    WS.zero_()
    _, Y_ref = oracle_run(oracle, good)
    assert_close(run_fused(g, workspace=WS), Y_ref, what="after re-zeroing")
    assert sg.sgmv_workspace_status(WS) == 0 and control_zero(WS)


def test_valid_calls_leave_status_zero(dev, oracle):
    rng = np.random.Generator(np.random.PCG64(210))
    for lengths in ([1] * 8, [5, 30, 2, 70], [130, 3]):
        w = _case(rng, lengths, 1024, 520)
        c = to_device(w, dev)
        WS = _workspace(dev, w)
        _, Y_ref = oracle_run(oracle, w)
        assert_close(run_fused(c, workspace=WS), Y_ref)
        assert sg.sgmv_workspace_status(WS) == 0 and control_zero(WS)


def test_wait_that_gives_up_is_reported(dev, oracle):
    """With a wait limit of zero polls, a consumer whose producer is not done
    at its first poll gives up: the call ends, reports SGMV_WS_WAIT_TIMEOUT,
    and the failed workspace makes the next call a no-op. Producers here
    stream a long reduction (d_in = 28672, segments of 14 and 80 rows) while
    consumers have a short row to write, so some consumer polls early."""
    rng = np.random.Generator(np.random.PCG64(220))
    w = _case(rng, [14, 80, 1, 1, 3], 28672, 264, P=5)
    c = to_device(w, dev)
    _, Y_ref = oracle_run(oracle, w)
    old = sg.sgmv_set_wait_limit(0)
    try:
        seen = 0
        for _ in range(5):
            WS = _workspace(dev, w)
            Y = c.Y0.clone()
            sg.sgmv_fused(Y, c.X, c.A_ptrs, c.B_ptrs, c.seg_start, c.seg_adapter, w.r, w.alpha, workspace_buf=WS)
            torch.cuda.synchronize()
            st = sg.sgmv_workspace_status(WS)
            assert st & ~sg.SGMV_WS_WAIT_TIMEOUT == 0, st
            if st:
                seen += 1
                # the failed workspace turns the next call into a no-op
                Y2 = c.Y0.clone()
                sg.sgmv_fused(Y2, c.X, c.A_ptrs, c.B_ptrs, c.seg_start, c.seg_adapter, w.r, w.alpha,
                              workspace_buf=WS)
                torch.cuda.synchronize()
                assert torch.equal(Y2, c.Y0)
            else:
                assert_close(Y, Y_ref, what="no wait gave up")
        assert seen > 0, "no wait gave up with a limit of zero polls"
    finally:
        assert sg.sgmv_set_wait_limit(old) == 0
    WS.zero_()
    assert_close(run_fused(c, workspace=WS), Y_ref, what="default limit")
    assert sg.sgmv_workspace_status(WS) == 0 and control_zero(WS)


def test_split_shrink_wait_limit(dev, oracle):
    """The split shrink's parts wait for one another (one long segment, d_in
    split between workgroups): with a limit of zero a wait may give up, and
    then the status says so; with the default limit V matches the oracle."""
    rng = np.random.Generator(np.random.PCG64(230))
    w = _case(rng, [16], 28672, 64, r=64, P=2)
    c = to_device(w, dev)
    need = sg.sgmv_workspace_bytes(w.num_segments, w.M, w.d_in, w.d_out, w.r, w.dtype)
    assert need > 0, "this batch is meant to split d_in between workgroups"
    V_ref, _ = oracle_run(oracle, w)
    old = sg.sgmv_set_wait_limit(0)
    try:
        WS = torch.zeros(need, dtype=torch.uint8, device=dev)
        V = torch.zeros((w.M, w.r), dtype=torch.float32, device=dev)
        sg.sgmv_shrink(V, c.X, c.A_ptrs, c.seg_start, c.seg_adapter, w.r, workspace_buf=WS)
        torch.cuda.synchronize()
        st = sg.sgmv_workspace_status(WS)
        assert st in (0, sg.SGMV_WS_WAIT_TIMEOUT), st
    finally:
        sg.sgmv_set_wait_limit(old)
    WS.zero_()
    V = torch.zeros((w.M, w.r), dtype=torch.float32, device=dev)
    sg.sgmv_shrink(V, c.X, c.A_ptrs, c.seg_start, c.seg_adapter, w.r, workspace_buf=WS)
    torch.cuda.synchronize()
    assert_close(V, V_ref, what="V")
    assert sg.sgmv_workspace_status(WS) == 0 and control_zero(WS)


def test_workspace_cache_on_a_side_stream(dev, oracle):
    """Without an explicit workspace the binding allocates and zero-fills one
    per (device, stream) on that stream, so the first call on a side stream
    sees a zero workspace; a larger call replaces it on the same stream."""
    rng = np.random.Generator(np.random.PCG64(240))
    small = _case(rng, [1, 2, 17, 1], 1024, 264)
    large = _case(rng, [90, 1, 3, 200, 7], 1024, 2056)
    side = torch.cuda.Stream()
    sg._workspaces.clear()
    for w in (small, large, small):
        c = to_device(w, dev)
        _, Y_ref = oracle_run(oracle, w)
        Y = c.Y0.clone()
        torch.cuda.synchronize()
        with torch.cuda.stream(side):
            sg.sgmv_fused(Y, c.X, c.A_ptrs, c.B_ptrs, c.seg_start, c.seg_adapter, w.r, w.alpha, stream=side)
        side.synchronize()
        assert_close(Y, Y_ref, what="side stream")
    ws = sg._workspaces[(dev.index or 0, side.cuda_stream)]
    assert sg.sgmv_workspace_status(ws, stream=side) == 0 and control_zero(ws)
