"""GPU numerics beyond the tolerance tests: non-finite adapters stay inside
their own segment's rows, and the matrix-core expand keeps its stated bound
when V needs more than 16 significant bits.

Inputs are integer-valued wherever a bitwise comparison is made: every
partial sum is then an exact integer below 2^24, so the GPU's fp32 results
equal the oracle's fp64 ones before the single final rounding, whatever
the order of summation.
"""
import numpy as np
import pytest
import torch

from . import workloads as wl
from .gpu_common import bits, oracle_bits, oracle_run, run_fused, run_split, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _ints(rng, shape, lo, hi, dtype):
    return torch.from_numpy(rng.integers(lo, hi + 1, size=shape).astype(np.float32)).to(dtype)


def _integer_workload(rng, lengths, ids, P, d_in, d_out, r):
    w = wl.Workload("numerics", int(sum(lengths)), d_in, d_out, r, 2.0 * r, torch.bfloat16, P,
                    wl.segments_from_lengths(lengths), np.asarray(ids, np.int32))
    w.X = _ints(rng, (w.M, d_in), -2, 2, w.dtype)
    w.A_pool = _ints(rng, (P, r, d_in), -1, 1, w.dtype)
    w.B_pool = _ints(rng, (P, r, d_out), -1, 1, w.dtype)
    w.Y = _ints(rng, (w.M, d_out), -8, 8, w.dtype)
    return w


# Batches with a poisoned adapter (id 1) on a long segment that shares a
# 16-row shrink tile and a 64-row expand tile with finite long segments, and
# on a short (vector path) segment between finite short ones. The second
# batch has more than 2048 rows, so its shrink runs on 64-row tiles at every rank.
POISON_CASES = {
    "small_batch": ([5, 20, 30, 3, 2, 40, 1, 16], [0, 1, 2, 1, 3, 4, 5, 2], 1024, 520),
    "large_batch": ([1000, 20, 30, 1100, 3, 2], [0, 1, 2, 3, 1, 4], 256, 264),
}


@pytest.mark.parametrize("where", ["A", "B"])
@pytest.mark.parametrize("case", sorted(POISON_CASES))
@pytest.mark.parametrize("r", [16, 64])
def test_nonfinite_adapter_is_isolated(dev, oracle, where, case, r):
    """An adapter holding +inf and NaN (in A, or in B) makes non-finite
    exactly the outputs the oracle makes non-finite; every other output,
    in rows that share tiles with the poisoned segments included, equals the
    oracle bit for bit, in the split and the fused path."""
    lengths, ids, d_in, d_out = POISON_CASES[case]
    rng = np.random.Generator(np.random.PCG64(300 + r + (where == "B")))
    w = _integer_workload(rng, lengths, ids, 6, d_in, d_out, r)
    if where == "A":
        w.A_pool[1, 3, 17] = float("inf")
        w.A_pool[1, r - 1, d_in - 5] = float("nan")
    else:
        w.B_pool[1, 5, 100] = float("inf")
        w.B_pool[1, r - 2, d_out - 3] = float("nan")
    c = to_device(w, dev)
    V_ref, Y_ref = oracle_run(oracle, w)
    bad_ref = ~np.isfinite(Y_ref)
    row_ids = np.repeat(np.asarray(ids), lengths)
    assert bad_ref.any() and (~bad_ref).any()
    assert not bad_ref[row_ids != 1].any(), "the oracle keeps the finite segments finite"
    want = oracle_bits(oracle, np.where(bad_ref, 0.0, Y_ref), w.dtype)
    V, Y = run_split(c)
    Vn = V.cpu().numpy().astype(np.float64)
    np.testing.assert_array_equal(np.isfinite(Vn), np.isfinite(V_ref))
    assert np.array_equal(Vn[np.isfinite(V_ref)], V_ref[np.isfinite(V_ref)])
    for path, Yg in (("split", Y), ("fused", run_fused(c))):
        y = Yg.cpu().to(torch.float64).numpy()
        np.testing.assert_array_equal(~np.isfinite(y), bad_ref, err_msg=f"{path}: non-finite pattern")
        got = bits(Yg)
        assert np.array_equal(got[~bad_ref], want[~bad_ref]), f"{path}: finite outputs differ"


@pytest.mark.parametrize("r", [16, 64])
def test_matrix_core_expand_bound_beyond_16_bits(dev, oracle, r):
    """V of up to about 4.2e6 (|V| > 2^16, 23 significant bits, exact in
    fp32): the shrink stays exact, and Y keeps within the bound the library
    states for the matrix-core expand, per element:
        (alpha / r) * S * (2^-16 + 2r * 2^-24) + 2^-8 * (|Y| + (alpha / r) * S)
    with S = sum_j |V_j| |B_jn|: the 16-bit representation of V, fp32
    accumulation of 2r products, and the bf16 rounding of the output (half
    an ulp, 2^-9 relative, doubled for the stored value's own error)."""
    rng = np.random.Generator(np.random.PCG64(320 + r))
    lengths, ids = [40, 3, 70, 1, 17], [0, 1, 2, 3, 0]
    d_in, d_out, P = 1024, 520, 4
    w = wl.Workload("wide_v", int(sum(lengths)), d_in, d_out, r, 2.0 * r, torch.bfloat16, P,
                    wl.segments_from_lengths(lengths), np.asarray(ids, np.int32))
    w.X = _ints(rng, (w.M, d_in), 1, 64, w.dtype)
    w.A_pool = _ints(rng, (P, r, d_in), 1, 64, w.dtype)
    w.B_pool = _ints(rng, (P, r, d_out), -3, 3, w.dtype)
    w.Y = _ints(rng, (w.M, d_out), -8, 8, w.dtype)
    c = to_device(w, dev)
    V_ref, Y_ref = oracle_run(oracle, w)
    assert V_ref.max() > 2 ** 16 and V_ref.max() < 2 ** 24
    scale = w.alpha / w.r
    Bk = wl.to_float64(w.B_pool)
    row_ids = np.repeat(np.asarray(ids), lengths)
    S = np.einsum("mj,mjn->mn", np.abs(V_ref), np.abs(Bk[row_ids]))
    bound = scale * S * (2.0 ** -16 + 2 * r * 2.0 ** -24) + 2.0 ** -8 * (np.abs(Y_ref) + scale * S)
    V, Y = run_split(c)
    assert np.array_equal(V.cpu().numpy().astype(np.float64), V_ref)
    for path, Yg in (("split", Y), ("fused", run_fused(c))):
        err = np.abs(Yg.cpu().to(torch.float64).numpy() - Y_ref)
        worst = float((err / bound).max())
        assert worst <= 1.0, f"{path}: error reaches {worst:.3f} of the stated bound"
        print(f"r={r} {path}: max error / bound = {worst:.3f}", flush=True)
