"""GPU parity of the layer-batched call (sgmv_fused_layer): every projection
of one batch in one launch. Each projection must equal the oracle, within
the tolerance, and the single-projection fused call, bit for bit (the same
items run in the same order on the same XCDs)."""
import numpy as np
import pytest
import torch

import segmented_gather_gemm_sgmv_amd as sg

from . import workloads as wl
from .gpu_common import assert_close, compact_rows, oracle_run, oracle_run_gather, rows_tensor, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def layer_case(rng, dtype, lengths, ids, P, shapes, r=16):
    """One batch (segments of `lengths` with adapters `ids`) through
    projections of the given (d_in, d_out) shapes, each with its own X, Y and
    pools."""
    ws = []
    for d_in, d_out in shapes:
        w = wl.Workload("layer", int(sum(lengths)), d_in, d_out, r, 2.0 * r, dtype, P,
                        wl.segments_from_lengths(lengths), np.asarray(ids, np.int32))
        wl.fill_tensors(w, rng)
        w.Y = wl._normal(rng, (w.M, w.d_out), 1.0, dtype)
        ws.append(w)
    return ws


def run_layer(cs, rows=None, workspace=None):
    Ys = [c.Y0.clone() for c in cs]
    sg.sgmv_fused_layer([(Y, c.X, c.A_ptrs, c.B_ptrs) for Y, c in zip(Ys, cs)], cs[0].seg_start,
                        cs[0].seg_adapter, cs[0].w.r, cs[0].w.alpha, rows=rows, workspace_buf=workspace)
    torch.cuda.synchronize()
    return Ys


def run_single(c, rows=None):
    Y = c.Y0.clone()
    if rows is None:
        sg.sgmv_fused(Y, c.X, c.A_ptrs, c.B_ptrs, c.seg_start, c.seg_adapter, c.w.r, c.w.alpha)
    else:
        sg.sgmv_fused_gather(Y, c.X, rows, c.A_ptrs, c.B_ptrs, c.seg_start, c.seg_adapter, c.w.r, c.w.alpha)
    torch.cuda.synchronize()
    return Y


SHAPES = [(1024, 1024), (1024, 136), (264, 2048), (2048, 1024)]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("gathered", [False, True])
@pytest.mark.parametrize("r", [8, 16, 32])
def test_layer_matches_oracle_and_single_calls(dev, oracle, dtype, gathered, r):
    rng = np.random.Generator(np.random.PCG64(100 + gathered + 2 * (dtype == torch.float32) + 4 * r))
    ws = layer_case(rng, dtype, [3, 70, 1, 0, 130, 17, 2], [4, 1, 0, 2, 3, 1, 5], 6, SHAPES, r=r)
    cs = [to_device(w, dev) for w in ws]
    rows = rng.permutation(ws[0].M).astype(np.int32) if gathered else None
    rt = rows_tensor(rows, dev) if gathered else None
    print(f"layer {dtype} gathered={gathered}: M={ws[0].M}, {len(ws)} projections", flush=True)
    Ys = run_layer(cs, rows=rt)
    for q, (w, c, Y) in enumerate(zip(ws, cs, Ys)):
        _, Y_ref = oracle_run_gather(oracle, w, rows) if gathered else oracle_run(oracle, w)
        assert_close(Y, Y_ref, what=f"projection {q}")
        assert torch.equal(Y, run_single(c, rt)), f"projection {q} differs from its own fused call"


def test_layer_max_projections_and_workspace_reuse(dev, oracle):
    """Eight projections (the maximum), then three of other sizes on the same
    workspace: every call leaves it zero."""
    rng = np.random.Generator(np.random.PCG64(101))
    big = layer_case(rng, torch.bfloat16, [20, 1, 5, 40], [0, 3, 2, 1], 4,
                     [(256 + 8 * q, 128 + 64 * q) for q in range(sg.SGMV_MAX_PROJECTIONS)])
    small = layer_case(rng, torch.bfloat16, [2, 1, 1, 66, 3], [1, 0, 2, 3, 1], 4, SHAPES[:3], r=64)
    need = max(sg.sgmv_layer_workspace_bytes([(c.Y0, c.X, c.A_ptrs, c.B_ptrs) for c in cs], ws[0].num_segments,
                                             ws[0].M, ws[0].r, ws[0].dtype)
               for ws, cs in ((x, [to_device(w, dev) for w in x]) for x in (big, small)))
    WS = torch.zeros(need, dtype=torch.uint8, device=dev)
    for ws in (big, small, big):
        cs = [to_device(w, dev) for w in ws]
        Ys = run_layer(cs, workspace=WS)
        assert int(torch.count_nonzero(WS)) == 0, "workspace not returned to zero"
        for q, (w, c, Y) in enumerate(zip(ws, cs, Ys)):
            _, Y_ref = oracle_run(oracle, w)
            assert_close(Y, Y_ref, what=f"projection {q}")
            assert torch.equal(Y, run_single(c))


@pytest.mark.parametrize("name", ["slice70b", "layer7b"])
def test_layer_whole_layers(dev, oracle, name):
    """A whole layer at full size, all 7 projections in one launch: the 70B
    slice (pools of 2000 adapters, 10.35 GB) and the 7B decode layer, every
    row of every projection against the oracle (on the slots the rows name,
    copied back one projection at a time), and bit for bit against the
    single calls."""
    ws = wl.slice70b() if name == "slice70b" else wl.layer7b()
    cs = []
    for w in ws:
        A = wl.device_pool(w.num_adapters, w.r, w.d_in, w.d_in ** -0.5, w.seed + 1, dev)
        B = wl.device_pool(w.num_adapters, w.r, w.d_out, w.r ** -0.5, w.seed + 2, dev)
        cs.append(to_device(w, dev, A_pool=A, B_pool=B))
    Ys = run_layer(cs)
    for w, c, Y in zip(ws, cs, Ys):
        assert torch.equal(Y, run_single(c)), f"{w.name}: layer call differs from the single call"
        _, Y_ref = oracle_run(oracle, compact_rows(w, c))
        e = assert_close(Y, Y_ref, what=f"{w.name} layer")
        print(f"{w.name}: layer max rel err {e:.2e} over {w.M} rows", flush=True)
    del cs, Ys
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
