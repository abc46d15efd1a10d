"""GPU parity: the HIP path through the C ABI against the oracle.

Bar: indexing (which rows receive which adapter) bit-exact; integer-valued
inputs bit-exact; general inputs within |gpu - oracle| <= 1e-2 (1 + |oracle|)
per element.
"""
import numpy as np
import pytest
import torch

import oracle as oracle_pkg
import segmented_gather_gemm_sgmv_amd as sg

from . import oracle_pins as pins
from . import workloads as wl
from .gpu_common import (TOL, assert_close, bits, compact_rows, oracle_bits, oracle_run, run_fused,
                         run_split, to_device)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def make_config(name):
    if name == "tiny":
        return wl.tiny()
    if name == "decode_distinct":
        return wl.decode_distinct()
    if name == "decode_skewed":
        return wl.decode_skewed(sg.sgmv_build_segments)
    if name == "prefill":
        return wl.prefill()
    raise KeyError(name)


CONFIGS = ["tiny", "decode_distinct", "decode_skewed", "prefill"]


@pytest.mark.parametrize("name", CONFIGS)
def test_config_parity(dev, oracle, name):
    w = make_config(name)
    c = to_device(w, dev)
    V_ref, Y_ref = oracle_run(oracle, w)
    V, Y = run_split(c)
    ev = assert_close(V, V_ref, what=f"{name} shrink V")
    ey = assert_close(Y, Y_ref, what=f"{name} shrink+expand Y")
    Yf = run_fused(c)
    ef = assert_close(Yf, Y_ref, what=f"{name} fused Y")
    print(f"{name}: max rel err V {ev:.2e}  Y {ey:.2e}  fused {ef:.2e}")


def _free(*ts):
    del ts
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_slice70b_parity(dev, oracle):
    """The 70B-layer slice at full size (512 rows, pools of 2000 adapters per
    projection, 10.35 GB in all), every row of every projection: V of the
    split path, Y of the split and fused paths. One projection's pools are
    on the device at a time; the 512 slots its rows name (at most 0.6 GB)
    come back for the oracle."""
    for w in wl.slice70b():
        A = wl.device_pool(w.num_adapters, w.r, w.d_in, w.d_in ** -0.5, w.seed + 1, dev)
        B = wl.device_pool(w.num_adapters, w.r, w.d_out, w.r ** -0.5, w.seed + 2, dev)
        c = to_device(w, dev, A_pool=A, B_pool=B)
        V, Y = run_split(c)
        Yf = run_fused(c)
        V_ref, Y_ref = oracle_run(oracle, compact_rows(w, c))
        ev = assert_close(V, V_ref, what=f"{w.name} V")
        ey = assert_close(Y, Y_ref, what=f"{w.name} Y")
        ef = assert_close(Yf, Y_ref, what=f"{w.name} fused Y")
        print(f"{w.name}: {w.M} rows, max rel err V {ev:.2e}  Y {ey:.2e}  fused {ef:.2e}", flush=True)
        del A, B, c, V, Y, Yf
        _free()


def test_slice70b_integer_exact(dev, oracle):
    """The 70B slice with integer values (X in -2..2, pools in -1..1, Y in
    -8..8, alpha = 2r) on its 2000-slot pools: every partial sum is an exact
    integer (|V| <= 2 * 28672 < 2^16), so V, split Y and fused Y equal the
    oracle bit for bit on every row."""
    rng = np.random.Generator(np.random.PCG64(41))
    for w in wl.slice70b():
        w.X = torch.from_numpy(rng.integers(-2, 3, size=(w.M, w.d_in)).astype(np.float32)).to(w.dtype)
        w.Y = torch.from_numpy(rng.integers(-8, 9, size=(w.M, w.d_out)).astype(np.float32)).to(w.dtype)
        w.alpha = 2.0 * w.r
        A = wl.device_int_pool(w.num_adapters, w.r, w.d_in, -1, 1, w.seed + 11, dev)
        B = wl.device_int_pool(w.num_adapters, w.r, w.d_out, -1, 1, w.seed + 12, dev)
        c = to_device(w, dev, A_pool=A, B_pool=B)
        V, Y = run_split(c)
        Yf = run_fused(c)
        V_ref, Y_ref = oracle_run(oracle, compact_rows(w, c))
        want = oracle_bits(oracle, Y_ref, w.dtype)
        assert np.array_equal(V.cpu().numpy().astype(np.float64), V_ref), w.name
        assert np.array_equal(bits(Y), want), w.name
        assert np.array_equal(bits(Yf), want), w.name
        print(f"{w.name}: bitwise on {w.M} rows", flush=True)
        del A, B, c, V, Y, Yf
        _free()


@pytest.mark.parametrize("mode", ["A", "B"])
def test_slice70b_indexing_signature(dev, oracle, mode):
    """Adapter-id signatures through the 70B slice's 2000-slot pools (ids up
    to 1999, three base-16 digits): every row's id comes back out of A (mode
    A) or B (mode B), in both paths, and the oracle agrees on the slots the
    rows name."""
    for w in wl.slice70b():
        X, A, B, alpha = pins.signature_inputs(w.seg_start, w.seg_adapter, w.num_adapters, w.d_in, w.d_out,
                                               w.r, mode, dtype=w.dtype, pool_device=dev)
        w.X, w.alpha = X, alpha
        w.Y = torch.zeros((w.M, w.d_out), dtype=w.dtype)
        c = to_device(w, dev, A_pool=A, B_pool=B)
        want = pins.row_adapter(w.seg_start, w.seg_adapter, w.M)
        for Y in (run_split(c)[1], run_fused(c)):
            y = Y.cpu().to(torch.float64).numpy()
            assert np.array_equal(pins.decode_signature(y), want), w.name
            assert np.all(y[:, 4:] == 0), w.name
        sub = compact_rows(w, c)
        _, Y_ref = oracle_run(oracle, sub)
        # the compacted pool numbers its slots 0..511: the oracle must find
        # slot p's encoded id, the original one, on row p
        assert np.array_equal(pins.decode_signature(Y_ref), want), w.name
        del A, B, c
        _free()


@pytest.mark.parametrize("name", CONFIGS)
def test_integer_exact(dev, oracle, name):
    """Integer-valued inputs: every partial sum is exact, so the GPU must
    match the oracle bit for bit, in either path, whatever its summation
    order."""
    w = wl.integer_case(np.random.Generator(np.random.PCG64(40)), make_config(name))
    c = to_device(w, dev)
    V_ref, Y_ref = oracle_run(oracle, w)
    want = oracle_bits(oracle, Y_ref, w.dtype)
    V, Y = run_split(c)
    assert np.array_equal(V.cpu().numpy().astype(np.float64), V_ref)
    assert np.array_equal(bits(Y), want)
    assert np.array_equal(bits(run_fused(c)), want)


@pytest.mark.parametrize("name", CONFIGS)
@pytest.mark.parametrize("mode", ["A", "B"])
def test_indexing_signature(dev, oracle, name, mode):
    """Each row's adapter id, written into the weights, must come back out
    exactly, for the A fetch and the B fetch separately."""
    w = make_config(name)
    X, A, B, alpha = pins.signature_inputs(w.seg_start, w.seg_adapter, w.num_adapters,
                                           w.d_in, w.d_out, w.r, mode, dtype=w.dtype)
    w.X, w.A_pool, w.B_pool, w.alpha = X, A, B, alpha
    w.Y = torch.zeros((w.M, w.d_out), dtype=w.dtype)
    c = to_device(w, dev)
    want = pins.row_adapter(w.seg_start, w.seg_adapter, w.M)
    for Y in (run_split(c)[1], run_fused(c)):
        y = Y.cpu().to(torch.float64).numpy()
        assert np.array_equal(pins.decode_signature(y), want)
        assert np.all(y[:, 4:] == 0)
    # and the oracle agrees
    _, Y_ref = oracle_run(oracle, w)
    assert np.array_equal(pins.decode_signature(Y_ref), want)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("r", [8, 16, 32, 64])
def test_random_small(dev, oracle, dtype, r):
    """Ragged segments (empty ones included), repeated adapters, non-square
    and ragged widths, nonzero Y, all ranks, both dtypes, both paths."""
    rng = np.random.Generator(np.random.PCG64(50 + r + (dtype == torch.float32)))
    for i in range(12):
        w = wl.random_case(rng, dtype=dtype, max_M=40, max_seg=7, max_pool=6, ranks=(r,), max_d=600)
        c = to_device(w, dev)
        V_ref, Y_ref = oracle_run(oracle, w)
        V, Y = run_split(c)
        assert_close(V, V_ref, what=f"case {i} V")
        assert_close(Y, Y_ref, what=f"case {i} Y")
        assert_close(run_fused(c), Y_ref, what=f"case {i} fused")
        wi = wl.integer_case(rng, w)
        ci = to_device(wi, dev)
        _, Yi_ref = oracle_run(oracle, wi)
        want = oracle_bits(oracle, Yi_ref, dtype)
        assert np.array_equal(bits(run_split(ci)[1]), want), f"case {i} integer split"
        assert np.array_equal(bits(run_fused(ci)), want), f"case {i} integer fused"


def test_long_segments_and_ragged_widths(dev, oracle):
    """Segments longer than one register block (8 rows) and widths that end
    inside a tile."""
    rng = np.random.Generator(np.random.PCG64(60))
    for dtype in (torch.bfloat16, torch.float32):
        for d_in, d_out in [(8, 24), (4104, 520), (1032, 4104)]:
            lengths = [37, 0, 9, 1, 100, 16, 17]
            ids = rng.integers(0, 5, size=len(lengths)).astype(np.int32)
            w = wl.Workload("long", int(sum(lengths)), d_in, d_out, 16, 32.0, dtype, 5,
                            wl.segments_from_lengths(lengths), ids)
            wl.fill_tensors(w, rng)
            w.Y = wl._normal(rng, (w.M, w.d_out), 1.0, dtype)
            c = to_device(w, dev)
            V_ref, Y_ref = oracle_run(oracle, w)
            V, Y = run_split(c)
            assert_close(V, V_ref, what="V")
            assert_close(Y, Y_ref, what="Y")
            assert_close(run_fused(c), Y_ref, what="fused")


def test_invalid_metadata_is_contained(dev, oracle):
    """Adapter ids outside the pool skip their segment; segment bounds past
    M are clamped. Nothing else changes."""
    rng = np.random.Generator(np.random.PCG64(61))
    w = wl.Workload("bad", 12, 64, 48, 8, 8.0, torch.bfloat16, 3,
                    np.array([0, 3, 5, 9, 12], np.int32), np.array([1, -1, 3, 2], np.int32))
    wl.fill_tensors(w, rng)
    w.Y = wl._normal(rng, (w.M, w.d_out), 1.0, w.dtype)
    c = to_device(w, dev)
    # oracle on the valid segments only
    ok = [0, 3]
    ref_w = wl.Workload("ok", 12, 64, 48, 8, 8.0, torch.bfloat16, 3,
                        np.array([0, 3, 9, 12], np.int32), np.array([1, 2, 2], np.int32),
                        X=w.X, Y=w.Y, A_pool=w.A_pool, B_pool=w.B_pool)
    _, Y_ref = oracle_run(oracle, ref_w)
    for Y in (run_split(c)[1], run_fused(c)):
        y = Y.cpu()
        # rows 3..8 (adapter -1 and adapter 3 = P) untouched, bitwise
        assert torch.equal(y[3:9], w.Y[3:9])
        assert_close(Y[0:3], Y_ref[0:3])
        assert_close(Y[9:12], Y_ref[9:12])
    # bounds past M: [0, 4, 40] over M = 12 -> second segment is rows 4..11
    w2 = wl.Workload("clamp", 12, 64, 48, 8, 8.0, torch.bfloat16, 3,
                     np.array([0, 4, 40], np.int32), np.array([0, 2], np.int32),
                     X=w.X, Y=w.Y, A_pool=w.A_pool, B_pool=w.B_pool)
    c2 = to_device(w2, dev)
    w2c = wl.Workload("clamped", 12, 64, 48, 8, 8.0, torch.bfloat16, 3,
                      np.array([0, 4, 12], np.int32), np.array([0, 2], np.int32),
                      X=w.X, Y=w.Y, A_pool=w.A_pool, B_pool=w.B_pool)
    _, Y_ref2 = oracle_run(oracle, w2c)
    assert_close(run_split(c2)[1], Y_ref2)
    assert_close(run_fused(c2), Y_ref2)


def test_empty_calls_are_noops(dev):
    w = wl.tiny()
    c = to_device(w, dev)
    Y = c.Y0.clone() + 1
    V = torch.full((w.M, w.r), 7.0, device=dev)
    empty = torch.zeros(1, dtype=torch.int32, device=dev)
    none = torch.zeros(0, dtype=torch.int32, device=dev)
    sg.sgmv_shrink(V, c.X, c.A_ptrs, empty, none, w.r)
    sg.sgmv_expand(Y, V, c.B_ptrs, empty, none, w.r, w.alpha)
    sg.sgmv_fused(Y, c.X, c.A_ptrs, c.B_ptrs, empty, none, w.r, w.alpha)
    torch.cuda.synchronize()
    assert torch.all(V == 7.0) and torch.all(Y == 1.0)
    X0 = torch.zeros((0, w.d_in), dtype=w.dtype, device=dev)
    Y0 = torch.zeros((0, w.d_out), dtype=w.dtype, device=dev)
    sg.sgmv_fused(Y0, X0, c.A_ptrs, c.B_ptrs, c.seg_start, c.seg_adapter, w.r, w.alpha)
    torch.cuda.synchronize()


def test_guard_bands(dev, oracle):
    """Sentinels before and after Y, V and the workspace survive every call."""
    rng = np.random.Generator(np.random.PCG64(62))
    w = wl.random_case(rng, dtype=torch.bfloat16, max_M=30, max_seg=5, ranks=(16,), max_d=300,
                       allow_empty=False)
    c = to_device(w, dev)
    G = 4096
    sentinel = -12345.0
    Ybuf = torch.full((G + w.M * w.d_out + G,), sentinel, dtype=w.dtype, device=dev)
    Vbuf = torch.full((G + w.M * w.r + G,), sentinel, dtype=torch.float32, device=dev)
    Y = Ybuf[G:G + w.M * w.d_out].view(w.M, w.d_out)
    V = Vbuf[G:G + w.M * w.r].view(w.M, w.r)
    Y.copy_(c.Y0)
    sg.sgmv_shrink(V, c.X, c.A_ptrs, c.seg_start, c.seg_adapter, w.r)
    sg.sgmv_expand(Y, V, c.B_ptrs, c.seg_start, c.seg_adapter, w.r, w.alpha)
    need = sg.sgmv_workspace_bytes(w.num_segments, w.M, w.d_in, w.d_out, w.r, w.dtype)
    WS = torch.zeros(256 + need + 4096, dtype=torch.uint8, device=dev)
    WS[:256] = 0xA5
    WS[256 + need:] = 0x5A
    sg.sgmv_fused(Y, c.X, c.A_ptrs, c.B_ptrs, c.seg_start, c.seg_adapter, w.r, w.alpha,
                  workspace_buf=WS[256:256 + need])
    torch.cuda.synchronize()
    for buf, n in ((Ybuf, w.M * w.d_out), (Vbuf, w.M * w.r)):
        assert torch.all(buf[:G] == sentinel) and torch.all(buf[G + n:] == sentinel)
    assert torch.all(WS[:256] == 0xA5) and torch.all(WS[256 + need:] == 0x5A)
    _, Y_ref = oracle_run(oracle, w)
    # Y got the delta twice (split then fused)
    Y_twice = oracle.expand(Y_ref, oracle.shrink(wl.storage(w.X), wl.storage(w.A_pool), w.seg_start,
                                                 w.seg_adapter),
                            wl.storage(w.B_pool), w.seg_start, w.seg_adapter, w.alpha)
    assert_close(Y, Y_twice, tol=2 * TOL)


def test_fused_workspace_reuse_and_reset(dev, oracle):
    """Every call leaves the whole workspace zero, so calls of any sizes
    (fewer segments and more rows, then more segments and fewer rows, both
    dtypes, fused and split) share one workspace."""
    rng = np.random.Generator(np.random.PCG64(63))
    long_case = wl.Workload("long", 150, 1024, 264, 16, 32.0, torch.bfloat16, 3,
                            wl.segments_from_lengths([40, 3, 107]), np.array([2, 0, 1], np.int32))
    wl.fill_tensors(long_case, rng)
    cases = [
        long_case,
        wl.random_case(rng, dtype=torch.float32, max_M=40, max_seg=2, ranks=(8,), max_d=256),
        wl.random_case(rng, dtype=torch.bfloat16, max_M=60, max_seg=7, ranks=(16,), max_d=256),
        wl.random_case(rng, dtype=torch.bfloat16, max_M=10, max_seg=3, ranks=(64,), max_d=256),
        wl.random_case(rng, dtype=torch.bfloat16, max_M=40, max_seg=7, ranks=(16,), max_d=256),
    ]
    need = max(sg.sgmv_workspace_bytes(x.num_segments, x.M, x.d_in, x.d_out, x.r, x.dtype)
               for x in cases)
    WS = torch.zeros(need, dtype=torch.uint8, device=dev)
    for w in cases + cases[::-1]:
        c = to_device(w, dev)
        V_ref, Y_ref = oracle_run(oracle, w)
        assert_close(run_fused(c, workspace=WS), Y_ref)
        assert int(torch.count_nonzero(WS)) == 0, "workspace not returned to zero (fused)"
        V, Y = run_split(c, workspace=WS)
        assert_close(V, V_ref)
        assert_close(Y, Y_ref)
        assert int(torch.count_nonzero(WS)) == 0, "workspace not returned to zero (shrink)"


def test_deterministic(dev):
    """Fixed-order reductions: repeated calls give identical bits."""
    w = wl.decode_skewed(sg.sgmv_build_segments)
    c = to_device(w, dev)
    V1, Y1 = run_split(c)
    V2, Y2 = run_split(c)
    assert torch.equal(V1, V2) and torch.equal(Y1, Y2)
    assert torch.equal(run_fused(c), run_fused(c))


def test_fused_equals_split_bitwise_on_integers(dev):
    w = wl.integer_case(np.random.Generator(np.random.PCG64(64)), wl.decode_distinct())
    c = to_device(w, dev)
    assert torch.equal(run_split(c)[1], run_fused(c))


def test_fused_back_to_back_fresh_values(dev, oracle):
    """Consecutive fused calls on one workspace, each with new inputs and
    multi-row segments: every call must see its own V, never the previous
    call's (integer inputs, so the check is bitwise)."""
    rng = np.random.Generator(np.random.PCG64(65))
    lengths = [1, 7, 30, 2, 64, 5, 1, 17]
    WS = torch.zeros(1 << 20, dtype=torch.uint8, device=dev)
    for call in range(6):
        ids = rng.integers(0, 9, size=len(lengths)).astype(np.int32)
        w = wl.Workload("b2b", int(sum(lengths)), 1024, 2048 + 8 * call, 16, 32.0, torch.bfloat16, 9,
                        wl.segments_from_lengths(lengths), ids)
        wl.fill_tensors(w, rng)
        wl.integer_case(rng, w)
        c = to_device(w, dev)
        _, Y_ref = oracle_run(oracle, w)
        assert np.array_equal(bits(run_fused(c, workspace=WS)), oracle_bits(oracle, Y_ref, w.dtype)), call


@pytest.mark.parametrize("r,d_in", [(16, 4096), (64, 4096), (16, 4104), (32, 4224), (64, 28672)])
def test_few_long_rows_split_reduction(dev, oracle, r, d_in):
    """Batches with few tiles of long rows split d_in between workgroups and
    combine the parts in the workspace, in a fixed order: check the values
    that integer inputs stay bit-exact and that the workspace is left zero.
    d_in = 4104 ends in a partial
    macro step; with 4104 and 4224 (33 macro steps in 8 parts) the last part
    has no steps at all and contributes zeros. d_in = 28672 with r = 64 is
    the largest reduction of the workloads (the 70B down projection) at the
    largest rank: integer partial sums still stay below 2^24."""
    rng = np.random.Generator(np.random.PCG64(66 + r + d_in))
    WS = torch.zeros(1 << 23, dtype=torch.uint8, device=dev)
    for lengths in ([16], [37], [1, 20, 3, 40], [64, 64], [70, 2, 150]):
        w = wl.Workload("few_long", int(sum(lengths)), d_in, 1032, r, 2.0 * r, torch.bfloat16, 5,
                        wl.segments_from_lengths(lengths),
                        rng.integers(0, 5, size=len(lengths)).astype(np.int32))
        wl.fill_tensors(w, rng)
        c = to_device(w, dev)
        V_ref, Y_ref = oracle_run(oracle, w)
        V, Y = run_split(c, workspace=WS)
        assert_close(V, V_ref, what=f"{lengths} V")
        assert_close(Y, Y_ref, what=f"{lengths} Y")
        assert_close(run_fused(c, workspace=WS), Y_ref, what=f"{lengths} fused")
        assert int(torch.count_nonzero(WS)) == 0
        wi = wl.integer_case(rng, w)
        ci = to_device(wi, dev)
        Vi_ref, Yi_ref = oracle_run(oracle, wi)
        Vi, Yi = run_split(ci, workspace=WS)
        assert np.array_equal(Vi.cpu().numpy().astype(np.float64), Vi_ref)
        assert np.array_equal(bits(Yi), oracle_bits(oracle, Yi_ref, wi.dtype))
        assert np.array_equal(bits(run_fused(ci, workspace=WS)), oracle_bits(oracle, Yi_ref, wi.dtype))


@pytest.mark.parametrize("P", [255, 256, 257])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_pool_table_boundaries(dev, oracle, P, dtype):
    """Pools of up to 256 adapters are looked up from a copy of the whole
    pointer table held in registers (four entries per lane), larger ones by a
    dependent load: ids in every quarter of the table, and the last entry,
    must reach the right adapter on both sides of the limit (integer inputs,
    bitwise)."""
    rng = np.random.Generator(np.random.PCG64(70 + P))
    lengths = [1, 1, 3, 1, 2, 1, 1, 1, 1, 5]
    ids = np.array([0, 63, 64, 127, 128, 191, 192, P - 1, P // 2, 255 % P], np.int32)
    w = wl.Workload("pool", int(sum(lengths)), 256, 264, 16, 32.0, dtype, P,
                    wl.segments_from_lengths(lengths), ids)
    wl.fill_tensors(w, rng)
    wl.integer_case(rng, w)
    c = to_device(w, dev)
    V_ref, Y_ref = oracle_run(oracle, w)
    V, Y = run_split(c)
    assert np.array_equal(V.cpu().numpy().astype(np.float64), V_ref)
    assert np.array_equal(bits(Y), oracle_bits(oracle, Y_ref, dtype))
    assert np.array_equal(bits(run_fused(c)), oracle_bits(oracle, Y_ref, dtype))


@pytest.mark.parametrize("N,mean", [(255, 0.7), (256, 0.7), (257, 0.7), (1500, 0.7), (70000, 0.7),
                                    (300, 20.0), (700, 20.0)])
def test_many_segments_with_long_ones(dev, oracle, N, mean):
    """Batches of many segments with a few long ones at the start, in the
    middle and at the end. The MFMA tiles find their pieces in the segment
    list by a search (one round for N < 256, several above); batches whose
    segments average 16 rows or more request the search's first round before
    anything else. mean 0.7: most segments empty or one row long; mean 20:
    lengths spread over 0 .. 40. Integer inputs, bitwise, split and fused."""
    rng = np.random.Generator(np.random.PCG64(80 + N))
    if mean < 1:
        lengths = rng.choice([0, 0, 0, 1, 1, 2], size=N)
    else:
        lengths = rng.integers(0, 41, size=N)
    for pos, n in [(0, 40), (N // 3, 16), (N // 2, 100), (N - 1, 70)]:
        lengths[pos] = n
    ids = rng.integers(0, 7, size=N).astype(np.int32)
    w = wl.Workload("many", int(lengths.sum()), 256, 264, 16, 32.0, torch.bfloat16, 7,
                    wl.segments_from_lengths(lengths), ids)
    assert (w.M >= 16 * N) == (mean > 1)
    wl.fill_tensors(w, rng)
    wl.integer_case(rng, w)
    c = to_device(w, dev)
    V_ref, Y_ref = oracle_run(oracle, w)
    V, Y = run_split(c)
    assert np.array_equal(V.cpu().numpy().astype(np.float64), V_ref)
    assert np.array_equal(bits(Y), oracle_bits(oracle, Y_ref, w.dtype))
    assert np.array_equal(bits(run_fused(c)), oracle_bits(oracle, Y_ref, w.dtype))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_mid_length_segments(dev, oracle, dtype):
    """Batches whose segments average between 2 and 16 rows: vector segments
    of 0 .. 15 rows (several row blocks each) mixed with one long segment,
    integer inputs, bitwise, split and fused, and the workspace left zero."""
    rng = np.random.Generator(np.random.PCG64(90))
    WS = torch.zeros(1 << 22, dtype=torch.uint8, device=dev)
    for lengths in ([15, 1, 9, 0, 3, 12, 7, 2, 14, 5], [2, 2, 3, 2, 2], [13, 40, 1, 6, 11]):
        ids = rng.integers(0, 6, size=len(lengths)).astype(np.int32)
        w = wl.Workload("mid", int(sum(lengths)), 264, 2056, 16, 32.0, dtype, 6,
                        wl.segments_from_lengths(lengths), ids)
        assert 2 * len(lengths) <= w.M < 16 * len(lengths)
        wl.fill_tensors(w, rng)
        wl.integer_case(rng, w)
        c = to_device(w, dev)
        V_ref, Y_ref = oracle_run(oracle, w)
        V, Y = run_split(c, workspace=WS)
        assert np.array_equal(V.cpu().numpy().astype(np.float64), V_ref)
        assert np.array_equal(bits(Y), oracle_bits(oracle, Y_ref, dtype))
        assert np.array_equal(bits(run_fused(c, workspace=WS)), oracle_bits(oracle, Y_ref, dtype))
        assert int(torch.count_nonzero(WS)) == 0


@pytest.mark.parametrize("r", [16, 64])
def test_expand_tile_with_many_pieces(dev, oracle, r):
    """A batch of short segments on average (so the MFMA expand tiles know
    their pieces before they request anything) whose 64-row tiles meet up to
    four long segments each, with distinct adapters: every piece after a
    tile's first has its B tile requested while the previous piece is
    worked on. Integer inputs, bitwise, split and fused, with the vector
    segments in 8-row blocks around them."""
    rng = np.random.Generator(np.random.PCG64(95))
    WS = torch.zeros(1 << 22, dtype=torch.uint8, device=dev)
    long_runs = [16, 16, 16, 16, 17, 23, 16, 20, 5, 9, 16, 16]
    lengths = long_runs + [1] * 20 + [8, 3, 12, 1, 1]
    ids = (np.arange(len(lengths)) % 7).astype(np.int32)
    w = wl.Workload("pieces", int(sum(lengths)), 520, 1032, r, 2.0 * r, torch.bfloat16, 7,
                    wl.segments_from_lengths(lengths), ids)
    assert w.M < 16 * len(lengths)
    wl.fill_tensors(w, rng)
    wl.integer_case(rng, w)
    c = to_device(w, dev)
    V_ref, Y_ref = oracle_run(oracle, w)
    V, Y = run_split(c, workspace=WS)
    assert np.array_equal(V.cpu().numpy().astype(np.float64), V_ref)
    want = oracle_bits(oracle, Y_ref, w.dtype)
    assert np.array_equal(bits(Y), want)
    assert np.array_equal(bits(run_fused(c, workspace=WS)), want)
    assert int(torch.count_nonzero(WS)) == 0


@pytest.mark.parametrize("r,bound", [(64, 768), (16, 1024)])
def test_tile_kind_bound(dev, oracle, r, bound):
    """Batches just below and just above the row count where the MFMA shrink
    changes from 16-row units to 64-row tiles (768 rows at r = 64, 1024
    below): the same segments, extended by one row, give the oracle's
    result bitwise on integer inputs through both kernels, split and
    fused."""
    rng = np.random.Generator(np.random.PCG64(96 + r))
    WS = torch.zeros(1 << 23, dtype=torch.uint8, device=dev)
    for M in (bound, bound + 1):
        lengths = [M - 3 * 150 - 7, 150, 150, 150, 1, 2, 4]
        ids = np.array([3, 0, 5, 1, 2, 4, 6], dtype=np.int32)
        w = wl.Workload("bound", M, 264, 520, r, 2.0 * r, torch.bfloat16, 7, wl.segments_from_lengths(lengths), ids)
        assert w.M == M
        wl.fill_tensors(w, rng)
        wl.integer_case(rng, w)
        c = to_device(w, dev)
        V_ref, Y_ref = oracle_run(oracle, w)
        V, Y = run_split(c, workspace=WS)
        assert np.array_equal(V.cpu().numpy().astype(np.float64), V_ref), M
        want = oracle_bits(oracle, Y_ref, w.dtype)
        assert np.array_equal(bits(Y), want), M
        assert np.array_equal(bits(run_fused(c, workspace=WS)), want), M
        assert int(torch.count_nonzero(WS)) == 0


def test_graph_replays(dev, oracle):
    """The calls are stream-ordered and allocate nothing, so they can be
    captured in a HIP graph. Replays of a captured fused call and of a
    captured shrink + expand, with eager work and synchronisations between
    replays, must each give the oracle's result bitwise (integer inputs) and
    leave the workspace zero. A mixed batch: one-row, mid-length and long
    segments, so the vector and MFMA paths and the split combine all run."""
    rng = np.random.Generator(np.random.PCG64(95))
    lengths = [1, 9, 130, 1, 3, 70, 15, 1]
    ids = rng.integers(0, 6, size=len(lengths)).astype(np.int32)
    w = wl.Workload("graph", int(sum(lengths)), 1024, 520, 16, 32.0, torch.bfloat16, 6,
                    wl.segments_from_lengths(lengths), ids)
    wl.fill_tensors(w, rng)
    wl.integer_case(rng, w)
    c = to_device(w, dev)
    _, Y_ref = oracle_run(oracle, w)
    want = oracle_bits(oracle, Y_ref, w.dtype)
    WS = torch.zeros(sg.sgmv_workspace_bytes(w.num_segments, w.M, w.d_in, w.d_out, w.r, w.dtype),
                     dtype=torch.uint8, device=dev)
    Y = torch.empty_like(c.Y0)
    V = torch.empty((w.M, w.r), dtype=torch.float32, device=dev)
    stream = torch.cuda.Stream()
    graphs = {}
    for name in ("fused", "split"):
        g = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=stream):
            Y.copy_(c.Y0)
            if name == "fused":
                sg.sgmv_fused(Y, c.X, c.A_ptrs, c.B_ptrs, c.seg_start, c.seg_adapter, w.r, w.alpha,
                              workspace_buf=WS)
            else:
                sg.sgmv_shrink(V, c.X, c.A_ptrs, c.seg_start, c.seg_adapter, w.r, workspace_buf=WS)
                sg.sgmv_expand(Y, V, c.B_ptrs, c.seg_start, c.seg_adapter, w.r, w.alpha)
        graphs[name] = g
    for rep in range(4):
        for name, g in graphs.items():
            Y.fill_(0)  # eager work between replays
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert np.array_equal(bits(Y), want), (name, rep)
            assert int(torch.count_nonzero(WS)) == 0, (name, rep)


@pytest.mark.parametrize("name", ["decode_distinct", "decode_skewed", "prefill"])
def test_one_call_per_segment_equals_one_call(dev, oracle, name):
    """Splitting a batch into one call per segment (the schedule SGMV
    replaces) gives the one-call result: bit for bit on integer inputs, and
    within the tolerance of the oracle on the workload's own values."""
    w = make_config(name)
    for integer in (False, True):
        if integer:
            w = wl.integer_case(np.random.Generator(np.random.PCG64(41)), w)
        c = to_device(w, dev)
        Y_one = run_fused(c)
        Y_seg = c.Y0.clone()
        for s in range(w.num_segments):
            a, b = int(w.seg_start[s]), int(w.seg_start[s + 1])
            meta = torch.tensor([0, b - a, int(w.seg_adapter[s])], dtype=torch.int32, device=dev)
            sg.sgmv_fused(Y_seg[a:b], c.X[a:b], c.A_ptrs, c.B_ptrs, meta[:2], meta[2:], w.r, w.alpha)
        torch.cuda.synchronize()
        if integer:
            assert torch.equal(Y_seg, Y_one)
        else:
            _, Y_ref = oracle_run(oracle, w)
            assert_close(Y_seg, Y_ref, what=f"{name} per segment")


@pytest.mark.parametrize("r", [16, 64])
def test_long_segment_among_empty_ones(dev, oracle, r):
    """bf16 batches where every segment could be short (M - N + 1 < 16) run on
    kernels built without the MFMA path; empty segments can still leave one
    long segment, which the vector path must compute, in every call."""
    rng = np.random.Generator(np.random.PCG64(120 + r))
    lengths = [0] * 14 + [37] + [0] * 10 + [1, 2]      # M = 40, N = 27: M - N + 1 = 14
    ids = rng.integers(0, 6, size=len(lengths)).astype(np.int32)
    w = wl.Workload("empty_and_long", int(sum(lengths)), 2056, 1032, r, 2.0 * r, torch.bfloat16, 6,
                    wl.segments_from_lengths(lengths), ids)
    wl.fill_tensors(w, rng)
    w.Y = wl._normal(rng, (w.M, w.d_out), 1.0, w.dtype)
    c = to_device(w, dev)
    V_ref, Y_ref = oracle_run(oracle, w)
    V, Y = run_split(c)
    assert_close(V, V_ref, what="V")
    assert_close(Y, Y_ref, what="split Y")
    assert_close(run_fused(c), Y_ref, what="fused Y")
    Yl = c.Y0.clone()
    sg.sgmv_fused_layer([(Yl, c.X, c.A_ptrs, c.B_ptrs)], c.seg_start, c.seg_adapter, w.r, w.alpha)
    torch.cuda.synchronize()
    assert_close(Yl, Y_ref, what="layer Y")


def _sampled_oracle(oracle, w, rows):
    """The oracle on chosen rows of w only: each row becomes a segment of its
    own with its segment's adapter."""
    ids = pins.row_adapter(w.seg_start, w.seg_adapter, w.M)[rows].astype(np.int32)
    sub = wl.Workload(w.name, len(rows), w.d_in, w.d_out, w.r, w.alpha, w.dtype, w.num_adapters,
                      wl.segments_from_lengths([1] * len(rows)), ids, X=w.X[torch.from_numpy(rows)],
                      Y=w.Y[torch.from_numpy(rows)], A_pool=w.A_pool, B_pool=w.B_pool)
    return oracle_run(oracle, sub)


def test_large_batch(dev, oracle):
    """40,000 rows (X and Y of 328 MB each): segments spanning hundreds of
    64-row tiles next to short ones, every call, checked on sampled rows of
    every segment (its first and last rows and random ones)."""
    rng = np.random.Generator(np.random.PCG64(130))
    lengths = [20000, 1, 15, 16, 9000, 0, 10968]
    ids = np.array([3, 0, 2, 1, 4, 2, 0], np.int32)
    w = wl.Workload("large", int(sum(lengths)), 4096, 4096, 16, 32.0, torch.bfloat16, 5,
                    wl.segments_from_lengths(lengths), ids)
    wl.fill_tensors(w, rng)
    rows = set()
    for s in range(len(lengths)):
        a, b = int(w.seg_start[s]), int(w.seg_start[s + 1])
        if b > a:
            rows |= {a, b - 1} | set(rng.integers(a, b, size=min(6, b - a)).tolist())
    rows = np.array(sorted(rows), np.int64)
    print(f"large batch: M={w.M}, {len(rows)} sampled rows", flush=True)
    c = to_device(w, dev)
    V_ref, Y_ref = _sampled_oracle(oracle, w, rows)
    r_t = torch.from_numpy(rows).to(dev)
    V, Y = run_split(c)
    assert_close(V[r_t], V_ref, what="V")
    assert_close(Y[r_t], Y_ref, what="split Y")
    assert_close(run_fused(c)[r_t], Y_ref, what="fused Y")
    perm = rng.permutation(w.M).astype(np.int32)
    rows_t = torch.from_numpy(perm).to(dev)
    Xg = torch.empty_like(c.X)
    Xg[rows_t.long()] = c.X   # token perm[p] holds segment row p
    Yg = torch.empty_like(c.Y0)
    Yg[rows_t.long()] = c.Y0
    sg.sgmv_fused_gather(Yg, Xg, rows_t, c.A_ptrs, c.B_ptrs, c.seg_start, c.seg_adapter, w.r, w.alpha)
    torch.cuda.synchronize()
    assert_close(Yg[rows_t.long()][r_t], Y_ref, what="fused_gather Y")


def test_graph_replays_gathered_and_layer(dev, oracle):
    """The gathered calls and the layer call captured in HIP graphs and
    replayed, with eager work in between: every replay bitwise equal to the
    oracle (integer inputs), the workspace left zero."""
    rng = np.random.Generator(np.random.PCG64(96))
    lengths = [1, 9, 130, 1, 3, 70, 15, 1]
    ids = rng.integers(0, 6, size=len(lengths)).astype(np.int32)
    ws_ = []
    for d_in, d_out in ((1024, 520), (520, 1024)):
        w = wl.Workload("graph", int(sum(lengths)), d_in, d_out, 16, 32.0, torch.bfloat16, 6,
                        wl.segments_from_lengths(lengths), ids)
        wl.fill_tensors(w, rng)
        ws_.append(wl.integer_case(rng, w))
    rows = rng.permutation(ws_[0].M).astype(np.int32)
    cs = [to_device(w, dev) for w in ws_]
    rt = torch.from_numpy(rows).to(dev)
    want_g = [oracle_bits(oracle, orc_y, w.dtype) for w, orc_y in
              ((w, oracle.sgmv_gather(wl.storage(w.Y), wl.storage(w.X), wl.storage(w.A_pool),
                                      wl.storage(w.B_pool), w.seg_start, w.seg_adapter, rows, w.alpha))
               for w in ws_)]
    want = [oracle_bits(oracle, oracle_run(oracle, w)[1], w.dtype) for w in ws_]
    need = max(sg.sgmv_layer_workspace_bytes([(c.Y0, c.X, c.A_ptrs, c.B_ptrs) for c in cs],
                                             ws_[0].num_segments, ws_[0].M, 16, torch.bfloat16),
               sg.sgmv_workspace_bytes(ws_[0].num_segments, ws_[0].M, 1024, 1024, 16, torch.bfloat16))
    WS = torch.zeros(need, dtype=torch.uint8, device=dev)
    Ys = [torch.empty_like(c.Y0) for c in cs]
    V = torch.empty((ws_[0].M, 16), dtype=torch.float32, device=dev)
    stream = torch.cuda.Stream()
    graphs = {}
    for name in ("fused_gather", "split_gather", "layer"):
        g = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=stream):
            for Y, c in zip(Ys, cs):
                Y.copy_(c.Y0)
            c0 = cs[0]
            if name == "fused_gather":
                sg.sgmv_fused_gather(Ys[0], c0.X, rt, c0.A_ptrs, c0.B_ptrs, c0.seg_start, c0.seg_adapter, 16,
                                     32.0, workspace_buf=WS)
            elif name == "split_gather":
                sg.sgmv_shrink_gather(V, c0.X, rt, c0.A_ptrs, c0.seg_start, c0.seg_adapter, 16, workspace_buf=WS)
                sg.sgmv_expand_scatter(Ys[0], V, rt, c0.B_ptrs, c0.seg_start, c0.seg_adapter, 16, 32.0)
            else:
                sg.sgmv_fused_layer([(Y, c.X, c.A_ptrs, c.B_ptrs) for Y, c in zip(Ys, cs)], c0.seg_start,
                                    c0.seg_adapter, 16, 32.0, workspace_buf=WS)
        graphs[name] = g
    for rep in range(4):
        for name, g in graphs.items():
            for Y in Ys:
                Y.fill_(0)  # eager work between replays
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            if name == "layer":
                for q in range(2):
                    assert np.array_equal(bits(Ys[q]), want[q]), (name, q, rep)
            else:
                assert np.array_equal(bits(Ys[0]), want_g[0]), (name, rep)
            assert int(torch.count_nonzero(WS)) == 0, (name, rep)
