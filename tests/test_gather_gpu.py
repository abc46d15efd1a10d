"""GPU parity of the gathered calls (sgmv_shrink_gather, sgmv_expand_scatter,
sgmv_fused_gather): X and Y stay in token order and segment row p is token
rows[p]. Compared through the C ABI with the oracle's gathered definition,
at the workloads' full sizes, with integer inputs bit for bit, and with
each token's adapter id read back out of its own row.
"""
import numpy as np
import pytest
import torch

import segmented_gather_gemm_sgmv_amd as sg

from . import oracle_pins as pins
from . import workloads as wl
from .gpu_common import (assert_close, bits, oracle_bits, oracle_run_gather, rows_tensor, run_fused,
                         run_fused_gather, run_split, run_split_gather, to_device)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def token_order(name):
    """A workload and the rows index that puts its tokens back in arrival
    order: decode_skewed keeps its Zipf draw's order (rows = the grouping's
    perm); the others get a seeded shuffle of their tokens."""
    if name == "tiny":
        w = wl.tiny()
    elif name == "decode_distinct":
        w = wl.decode_distinct()
    elif name == "decode_skewed":
        w = wl.decode_skewed(sg.sgmv_build_segments)
        perm, _, _ = sg.sgmv_build_segments(w.token_adapter)
        return w, perm
    elif name == "prefill":
        w = wl.prefill()
    else:
        raise KeyError(name)
    rng = np.random.Generator(np.random.PCG64(90))
    return w, rng.permutation(w.M).astype(np.int32)


CONFIGS = ["tiny", "decode_distinct", "decode_skewed", "prefill"]


@pytest.mark.parametrize("name", CONFIGS)
def test_gather_config_parity(dev, oracle, name):
    w, rows = token_order(name)
    c = to_device(w, dev)
    rt = rows_tensor(rows, dev)
    print(f"gather {name}: M={w.M} segments={w.num_segments}", flush=True)
    V_ref, Y_ref = oracle_run_gather(oracle, w, rows)
    V, Y = run_split_gather(c, rt)
    ev = assert_close(V, V_ref, what=f"{name} shrink_gather V")
    ey = assert_close(Y, Y_ref, what=f"{name} expand_scatter Y")
    Yf = run_fused_gather(c, rt)
    ef = assert_close(Yf, Y_ref, what=f"{name} fused_gather Y")
    # the same kernels on the batch moved into segment order give the same bits
    idx = torch.from_numpy(rows.astype(np.int64)).to(dev)
    cs = to_device(w, dev)
    cs.X = c.X[idx].contiguous()
    cs.Y0 = c.Y0[idx].contiguous()
    Vs, Ys = run_split(cs)
    assert torch.equal(V, Vs)
    assert torch.equal(Y[idx], Ys)
    assert torch.equal(Yf[idx], run_fused(cs))
    print(f"gather {name}: max rel err V {ev:.2e}  Y {ey:.2e}  fused {ef:.2e}")


@pytest.mark.parametrize("name", CONFIGS)
def test_gather_integer_exact(dev, oracle, name):
    w, rows = token_order(name)
    w = wl.integer_case(np.random.Generator(np.random.PCG64(91)), w)
    c = to_device(w, dev)
    rt = rows_tensor(rows, dev)
    V_ref, Y_ref = oracle_run_gather(oracle, w, rows)
    want = oracle_bits(oracle, Y_ref, w.dtype)
    V, Y = run_split_gather(c, rt)
    assert np.array_equal(V.cpu().numpy().astype(np.float64), V_ref)
    assert np.array_equal(bits(Y), want)
    assert np.array_equal(bits(run_fused_gather(c, rt)), want)


@pytest.mark.parametrize("name", ["decode_skewed", "prefill"])
@pytest.mark.parametrize("mode", ["A", "B"])
def test_gather_indexing_signature(dev, name, mode):
    """Each token's own adapter id, encoded in the weights, comes back out of
    its own row of Y: the gather reads the right row of X and the scatter
    writes the right row of Y, for the A fetch and the B fetch."""
    w, rows = token_order(name)
    X, A, B, alpha = pins.signature_inputs(w.seg_start, w.seg_adapter, w.num_adapters,
                                           w.d_in, w.d_out, w.r, mode, dtype=w.dtype)
    # tokens differ in X: token t carries 1 + (t mod 3) in column 0, so its
    # row decodes to its adapter only if X and Y rows are paired correctly
    X[:, 0] = torch.from_numpy((1 + np.arange(w.M) % 3).astype(np.float32)).to(w.dtype)
    w.X, w.A_pool, w.B_pool, w.alpha = X, A, B, alpha
    w.Y = torch.zeros((w.M, w.d_out), dtype=w.dtype)
    c = to_device(w, dev)
    seg_of_p = pins.row_adapter(w.seg_start, w.seg_adapter, w.M)
    want = np.empty(w.M, np.int64)
    want[rows] = seg_of_p
    mult = (1 + np.arange(w.M) % 3).astype(np.float64)
    rt = rows_tensor(rows, dev)
    for Y in (run_split_gather(c, rt)[1], run_fused_gather(c, rt)):
        y = Y.cpu().to(torch.float64).numpy()
        assert np.all(y[:, 4:] == 0)
        assert np.array_equal(y[:, :4] % mult[:, None], np.zeros((w.M, 4)))
        assert np.array_equal(pins.decode_signature(y / mult[:, None]), want)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("r", [8, 16, 32, 64])
def test_gather_random_small(dev, oracle, dtype, r):
    """Ragged segments (empty ones and ones of 16+ rows), random token order."""
    rng = np.random.Generator(np.random.PCG64(92 + r + (dtype == torch.float32)))
    for i in range(8):
        w = wl.random_case(rng, dtype=dtype, max_M=80, max_seg=5, max_pool=6, ranks=(r,), max_d=600)
        rows = rng.permutation(w.M).astype(np.int32)
        c = to_device(w, dev)
        rt = rows_tensor(rows, dev)
        V_ref, Y_ref = oracle_run_gather(oracle, w, rows)
        V, Y = run_split_gather(c, rt)
        assert_close(V, V_ref, what=f"case {i} V")
        assert_close(Y, Y_ref, what=f"case {i} Y")
        assert_close(run_fused_gather(c, rt), Y_ref, what=f"case {i} fused")


def test_gather_identity_rows_bitwise(dev):
    """rows = 0 .. M-1 is the contiguous call, bit for bit."""
    rng = np.random.Generator(np.random.PCG64(93))
    w = wl.Workload("mixed", 150, 1024, 264, 16, 32.0, torch.bfloat16, 3,
                    wl.segments_from_lengths([40, 3, 107]), np.array([2, 0, 1], np.int32))
    wl.fill_tensors(w, rng)
    w.Y = wl._normal(rng, (w.M, w.d_out), 1.0, w.dtype)
    c = to_device(w, dev)
    rt = rows_tensor(np.arange(w.M), dev)
    V, Y = run_split_gather(c, rt)
    V0, Y0 = run_split(c)
    assert torch.equal(V, V0) and torch.equal(Y, Y0)
    assert torch.equal(run_fused_gather(c, rt), run_fused(c))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_gather_bad_rows_are_contained(dev, oracle, dtype):
    """Entries outside [0, M) write nothing; a token named twice gets an
    unspecified value; every other token is exact; nothing outside Y is
    written; the fused workspace comes back zero."""
    rng = np.random.Generator(np.random.PCG64(94))
    w = wl.Workload("bad_rows", 120, 264, 136, 16, 32.0, dtype, 4,
                    wl.segments_from_lengths([3, 50, 1, 0, 66]), np.array([1, 3, 0, 2, 1], np.int32))
    wl.fill_tensors(w, rng)
    w.Y = wl._normal(rng, (w.M, w.d_out), 1.0, dtype)
    perm = rng.permutation(w.M).astype(np.int32)
    _, Y_ref = oracle_run_gather(oracle, w, perm)
    bad = perm.copy()
    bad[[0, 5, 60, 119]] = [-1, w.M, 1 << 30, -(1 << 30)]   # absent segment rows
    bad[70] = bad[71]                                        # token bad[71] named twice
    absent = set(perm[[0, 5, 60, 119, 70]].tolist())          # tokens no valid entry names
    twice = int(bad[71])
    exact = np.array([t for t in range(w.M) if t not in absent and t != twice])
    gone = np.array(sorted(absent))
    c = to_device(w, dev)
    rt = rows_tensor(bad, dev)
    G = 2048
    sentinel = -777.0
    need = sg.sgmv_workspace_bytes(w.num_segments, w.M, w.d_in, w.d_out, w.r, w.dtype)
    WS = torch.zeros(max(need, 256), dtype=torch.uint8, device=dev)
    for fused in (False, True):
        Ybuf = torch.full((G + w.M * w.d_out + G,), sentinel, dtype=dtype, device=dev)
        Y = Ybuf[G:G + w.M * w.d_out].view(w.M, w.d_out)
        Y.copy_(c.Y0)
        if fused:
            run_fused_gather(c, rt, Y=Y, workspace=WS)
            assert int(torch.count_nonzero(WS)) == 0
        else:
            run_split_gather(c, rt, Y=Y, workspace=WS)
        assert torch.all(Ybuf[:G] == sentinel) and torch.all(Ybuf[G + w.M * w.d_out:] == sentinel)
        y = Y.cpu()
        assert torch.equal(y[torch.from_numpy(gone)], w.Y[torch.from_numpy(gone)])
        assert_close(Y[torch.from_numpy(exact).to(dev)], Y_ref[exact], what=f"fused={fused}")
