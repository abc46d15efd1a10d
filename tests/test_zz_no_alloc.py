"""GPU test of sgmv_fused_noalloc, the fused call that allocates nothing: it
runs on the library's static per-device scratch array instead of a
caller-supplied workspace. Through the C ABI, its output must equal
sgmv_fused's on the same inputs (same kernels: bit for bit) on two calls in a
row, the second with a smaller batch, and match the oracle."""
import numpy as np
import pytest
import torch

import segmented_gather_gemm_sgmv_amd as sg

from . import workloads as wl
from .gpu_common import assert_close, bits, oracle_bits, oracle_run, run_fused, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _case(rng, lengths, d_in, d_out, r=16, P=6, integer=False, starts=None):
    ids = rng.integers(0, P, size=len(lengths)).astype(np.int32)
    ss = wl.segments_from_lengths(lengths) if starts is None else np.asarray(starts, np.int32)
    M = int(sum(lengths)) if starts is None else int(starts[-1])
    w = wl.Workload("noalloc", M, d_in, d_out, r, 2.0 * r, torch.bfloat16, P, ss, ids)
    wl.fill_tensors(w, rng)
    w.Y = wl._normal(rng, (w.M, w.d_out), 1.0, w.dtype)
    return wl.integer_case(rng, w) if integer else w


def _noalloc(c):
    Y = c.Y0.clone()
    sg.sgmv_fused_noalloc(Y, c.X, c.A_ptrs, c.B_ptrs, c.seg_start, c.seg_adapter, c.w.r, c.w.alpha)
    torch.cuda.synchronize()
    return Y


@pytest.mark.parametrize("integer", [False, True], ids=["normal", "integer"])
def test_noalloc_equals_fused_two_calls(dev, oracle, integer):
    """A mixed batch (one-row, mid-length and long segments), then a smaller
    one: each equals sgmv_fused bit for bit and the oracle to the tolerance
    (bit for bit on integer inputs)."""
    rng = np.random.Generator(np.random.PCG64(300 + integer))
    big = _case(rng, [1, 9, 130, 1, 3, 70, 15, 1, 40, 2], 2056, 1032, integer=integer)
    small = _case(rng, [2, 17, 1, 5], 520, 264, integer=integer)
    for w in (big, small):
        c = to_device(w, dev)
        Y = _noalloc(c)
        assert torch.equal(Y, run_fused(c)), w.M
        _, Y_ref = oracle_run(oracle, w)
        if integer:
            assert np.array_equal(bits(Y), oracle_bits(oracle, Y_ref, w.dtype)), w.M
        else:
            assert_close(Y, Y_ref, what=f"noalloc M={w.M}")


def test_noalloc_decode_and_rank64(dev, oracle):
    """A decode batch (the kernels without the MFMA path) and an r = 64
    prefill-like batch, back to back."""
    rng = np.random.Generator(np.random.PCG64(310))
    for w in (_case(rng, [1] * 48, 4096, 4096, P=64), _case(rng, [200, 31, 1], 1024, 2048, r=64)):
        c = to_device(w, dev)
        Y = _noalloc(c)
        assert torch.equal(Y, run_fused(c))
        _, Y_ref = oracle_run(oracle, w)
        assert_close(Y, Y_ref, what=f"noalloc r={w.r}")


def test_noalloc_rejects_batches_beyond_its_scratch(dev):
    """A batch whose fused workspace exceeds the static array is refused with
    SGMV_ERR_SCRATCH before anything is enqueued (Y untouched)."""
    rng = np.random.Generator(np.random.PCG64(320))
    M, d_out = 9000, 16384
    need = sg.sgmv_workspace_bytes(M, M, 64, d_out, 64, torch.bfloat16)
    assert need > sg.SGMV_NOALLOC_SCRATCH_BYTES
    X = torch.zeros((M, 64), dtype=torch.bfloat16, device=dev)
    Y = torch.ones((M, d_out), dtype=torch.bfloat16, device=dev)
    pool_a = torch.zeros((1, 64, 64), dtype=torch.bfloat16, device=dev)
    pool_b = torch.zeros((1, 64, d_out), dtype=torch.bfloat16, device=dev)
    ss = torch.arange(M + 1, dtype=torch.int32, device=dev)
    sa = torch.zeros(M, dtype=torch.int32, device=dev)
    with pytest.raises(sg.SGMVError) as e:
        sg.sgmv_fused_noalloc(Y, X, sg.sgmv_pool_pointers(pool_a), sg.sgmv_pool_pointers(pool_b), ss, sa, 64, 128.0)
    assert e.value.status == -9
    torch.cuda.synchronize()
    assert torch.all(Y == 1)


def test_noalloc_recovers_after_a_failed_call(dev, oracle):
    """A call with decreasing offsets leaves a failure status in the scratch
    array; the next call clears the array first and computes normally."""
    rng = np.random.Generator(np.random.PCG64(330))
    bad = _case(rng, [1, 1, 1], 512, 264, starts=[0, 40, 20, 80])
    _noalloc(to_device(bad, dev))
    good = _case(rng, [3, 20, 1, 10], 512, 264)
    c = to_device(good, dev)
    _, Y_ref = oracle_run(oracle, good)
    assert_close(_noalloc(c), Y_ref, what="after a failed call")
    assert torch.equal(_noalloc(c), run_fused(c))
