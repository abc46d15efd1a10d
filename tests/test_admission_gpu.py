"""GPU test of adapter admission (sgmv_admit_adapter): an adapter copied from
pinned host memory into a device slot, with its table entries updated in
stream order, is what the next SGMV call on that stream uses; a call
enqueued before the admission still uses the old adapter."""
import numpy as np
import pytest
import torch

import segmented_gather_gemm_sgmv_amd as sg

from . import workloads as wl
from .gpu_common import assert_close, oracle_run, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def pinned_copy(t: torch.Tensor) -> torch.Tensor:
    out = torch.empty(t.shape, dtype=t.dtype, pin_memory=True)
    out.copy_(t)
    return out


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_admission_is_stream_ordered(dev, oracle, dtype):
    rng = np.random.Generator(np.random.PCG64(110 + (dtype == torch.float32)))
    lengths, ids = [2, 40, 1, 7], [3, 1, 0, 3]
    w = wl.Workload("admit", int(sum(lengths)), 1024, 520, 16, 32.0, dtype, 5,
                    wl.segments_from_lengths(lengths), np.array(ids, np.int32))
    wl.fill_tensors(w, rng)
    w.Y = wl._normal(rng, (w.M, w.d_out), 1.0, dtype)
    c = to_device(w, dev)
    # a spare slot outside the pool, and new weights for adapters 3 and 1
    spare_A = torch.empty((2, w.r, w.d_in), dtype=dtype, device=dev)
    spare_B = torch.empty((2, w.r, w.d_out), dtype=dtype, device=dev)
    new = {k: (wl._normal(rng, (w.r, w.d_in), w.d_in ** -0.5, dtype),
               wl._normal(rng, (w.r, w.d_out), w.r ** -0.5, dtype)) for k in (3, 1)}
    hosts = {k: (pinned_copy(a), pinned_copy(b)) for k, (a, b) in new.items()}
    ws = torch.zeros(max(256, sg.sgmv_workspace_bytes(w.num_segments, w.M, w.d_in, w.d_out, w.r, dtype)),
                     dtype=torch.uint8, device=dev)
    Y_before, Y_after = c.Y0.clone(), c.Y0.clone()
    # one stream, no synchronisation in between
    sg.sgmv_fused(Y_before, c.X, c.A_ptrs, c.B_ptrs, c.seg_start, c.seg_adapter, w.r, w.alpha, workspace_buf=ws)
    for i, k in enumerate((3, 1)):
        sg.sgmv_admit_adapter(spare_A[i], spare_B[i], hosts[k][0], hosts[k][1], c.A_ptrs, c.B_ptrs, k)
    sg.sgmv_fused(Y_after, c.X, c.A_ptrs, c.B_ptrs, c.seg_start, c.seg_adapter, w.r, w.alpha, workspace_buf=ws)
    torch.cuda.synchronize()
    _, ref_before = oracle_run(oracle, w)
    assert_close(Y_before, ref_before, what="call enqueued before the admission")
    A2, B2 = w.A_pool.clone(), w.B_pool.clone()
    for k, (a, b) in new.items():
        A2[k], B2[k] = a, b
    w2 = wl.Workload("admitted", w.M, w.d_in, w.d_out, w.r, w.alpha, dtype, w.num_adapters, w.seg_start,
                     w.seg_adapter, X=w.X, Y=w.Y, A_pool=A2, B_pool=B2)
    _, ref_after = oracle_run(oracle, w2)
    assert_close(Y_after, ref_after, what="call enqueued after the admission")
    # the table now points at the spare slots; the old slots are untouched
    base_A, base_B = spare_A.data_ptr(), spare_B.data_ptr()
    tab_A, tab_B = c.A_ptrs.cpu().tolist(), c.B_ptrs.cpu().tolist()
    assert tab_A[3] == base_A and tab_A[1] == base_A + spare_A[0].numel() * spare_A.element_size()
    assert tab_B[3] == base_B and tab_B[1] == base_B + spare_B[0].numel() * spare_B.element_size()
    assert torch.equal(c.A_pool.cpu(), w.A_pool) and torch.equal(c.B_pool.cpu(), w.B_pool)
    assert torch.equal(spare_A[0].cpu(), new[3][0]) and torch.equal(spare_B[1].cpu(), new[1][1])


def test_adapter_pool_admit_and_run(dev, oracle):
    """AdapterPool: every slot filled by admission from pinned host memory,
    then a fused call on its tables equals the oracle on the same weights."""
    rng = np.random.Generator(np.random.PCG64(112))
    w = wl.Workload("pool", 40, 512, 264, 16, 32.0, torch.bfloat16, 4,
                    wl.segments_from_lengths([1, 17, 2, 20]), np.array([3, 0, 2, 3], np.int32))
    wl.fill_tensors(w, rng)
    w.Y = wl._normal(rng, (w.M, w.d_out), 1.0, w.dtype)
    sg.sgmv_check_segments(w.seg_start, w.seg_adapter, w.M, w.num_adapters)
    pool = sg.AdapterPool(w.num_adapters, w.d_in, w.d_out, w.r, w.dtype, device=dev)
    hosts = [(pinned_copy(w.A_pool[k]), pinned_copy(w.B_pool[k])) for k in range(w.num_adapters)]
    for k, (a, b) in enumerate(hosts):
        pool.admit(k, a, b)
    c = to_device(w, dev, A_pool=pool.A, B_pool=pool.B)
    Y = c.Y0.clone()
    sg.sgmv_fused(Y, c.X, pool.A_ptrs, pool.B_ptrs, c.seg_start, c.seg_adapter, w.r, w.alpha)
    torch.cuda.synchronize()
    _, Y_ref = oracle_run(oracle, w)
    assert_close(Y, Y_ref, what="pool")
    assert torch.equal(pool.A.cpu(), w.A_pool) and torch.equal(pool.B.cpu(), w.B_pool)
    with pytest.raises(IndexError):
        pool.admit(4, *hosts[0])
