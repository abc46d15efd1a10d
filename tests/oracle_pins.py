"""Pins for the oracle: checks against values fixed independently of the
oracle's own formula.

Each ``pin_*`` takes an :class:`oracle.Oracle` and raises AssertionError when
the oracle disagrees with what the pages and the mathematics fix. They run on
the real oracle (``test_oracle_pins.py``) and on copies of it with planted
mistakes (``test_oracle_mutants.py``), which must each fail at least one pin.

What each pin rests on:

* dense_single_adapter — one segment covering the whole batch is one dense
  product X A B, computed by numpy's matmul (Punica guide, "The Heterogeneous
  Batching Bottleneck": when every request shares weights the work is one
  dense GEMM; the same holds for one shared adapter).
* dense_mask — the whole batch as dense GEMMs against every adapter at once,
  with a one-hot mask selecting each row's adapter: a different route to the
  same sum, which exposes index, segment and operand-orientation mistakes.
* integer_bruteforce — exact Python-integer arithmetic, row by row, on small
  integer inputs (the result is an exact integer; no rounding anywhere).
* handworked — the fixture in ``golden/handworked_tiny.json``, worked by hand.
* zero_adapter — a zero A or zero B leaves the segment's rows exactly as they
  came in, and other rows are unaffected.
* linearity — the delta is linear in X.
* permutation — permuting segments together with their adapter ids permutes
  the output rows (bitwise: the per-row arithmetic is the same).
* signature — adapter ids encoded into the weights come back out, row by row.
* scale — alpha doubled doubles the delta exactly (power-of-two scaling).
* bf16_rounding — the oracle's rounding agrees with torch's fp32 -> bf16
  conversion, and with hand-checked ties.
* f32_rounding — the oracle's rounding of its float64 results to binary32
  (the expected bits of every fp32 bitwise GPU test) against values worked by
  hand from the binary32 format: ties to even, a near-tie that a double
  rounding would get wrong, overflow at the exact threshold, and the
  subnormal grid.
* segments — the grouping of tokens by adapter is a stable sort with correct
  run starts.
* gather_per_token — with the batch left in token order, the gathered call
  gives every token the per-row equation with its own adapter, worked in
  Python integers without segments; V comes back in segment order.
"""
from __future__ import annotations

import json
import os

import numpy as np
import torch

from . import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rel_close(a, b, tol):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    err = np.abs(a - b) / (1.0 + np.abs(b))
    assert err.max(initial=0.0) <= tol, f"max rel err {err.max():.3e} > {tol:.1e}"


def _f64(t):
    return wl.to_float64(t)


def _run(orc, w: wl.Workload):
    return orc.sgmv(wl.storage(w.Y), wl.storage(w.X), wl.storage(w.A_pool), wl.storage(w.B_pool),
                    w.seg_start, w.seg_adapter, w.alpha)


def pin_dense_single_adapter(orc):
    rng = np.random.Generator(np.random.PCG64(11))
    for dtype in (torch.float32, torch.bfloat16):
        w = wl.Workload("dense", 7, 48, 40, 8, 24.0, dtype, 3, np.array([0, 7], np.int32),
                        np.array([2], np.int32))
        wl.fill_tensors(w, rng)
        w.Y = wl._normal(rng, (w.M, w.d_out), 1.0, dtype)
        got = _run(orc, w)
        A = _f64(w.A_pool[2]).T          # logical d_in x r
        B = _f64(w.B_pool[2])            # logical r x d_out
        want = _f64(w.Y) + (w.alpha / w.r) * (_f64(w.X) @ A @ B)
        _rel_close(got, want, 1e-12)
        V = orc.shrink(wl.storage(w.X), wl.storage(w.A_pool), w.seg_start, w.seg_adapter)
        _rel_close(V, _f64(w.X) @ A, 1e-12)


def pin_dense_mask(orc):
    rng = np.random.Generator(np.random.PCG64(12))
    for _ in range(20):
        w = wl.random_case(rng, dtype=torch.float32, max_M=14, max_seg=5, max_pool=4)
        got = _run(orc, w)
        P, r = w.num_adapters, w.r
        A_all = np.concatenate([_f64(w.A_pool[k]).T for k in range(P)], axis=1)  # d_in x P*r
        B_all = np.concatenate([_f64(w.B_pool[k]) for k in range(P)], axis=0)    # P*r x d_out
        mask = np.zeros((w.M, P * r))
        for s in range(w.num_segments):
            k = int(w.seg_adapter[s])
            mask[w.seg_start[s]:w.seg_start[s + 1], k * r:(k + 1) * r] = 1.0
        want = _f64(w.Y) + (w.alpha / r) * (((_f64(w.X) @ A_all) * mask) @ B_all)
        _rel_close(got, want, 1e-12)


def pin_integer_bruteforce(orc):
    rng = np.random.Generator(np.random.PCG64(13))
    for _ in range(30):
        w = wl.integer_case(rng, wl.random_case(rng, dtype=torch.bfloat16, max_M=10, max_d=24))
        got = _run(orc, w)
        X = w.X.to(torch.int64).tolist()
        A = w.A_pool.to(torch.int64).tolist()
        B = w.B_pool.to(torch.int64).tolist()
        Y = w.Y.to(torch.int64).tolist()
        scale = int(w.alpha) // w.r
        assert scale * w.r == int(w.alpha)
        for s in range(w.num_segments):
            k = int(w.seg_adapter[s])
            for m in range(int(w.seg_start[s]), int(w.seg_start[s + 1])):
                v = [sum(X[m][i] * A[k][j][i] for i in range(w.d_in)) for j in range(w.r)]
                for n in range(w.d_out):
                    Y[m][n] += scale * sum(v[j] * B[k][j][n] for j in range(w.r))
        assert np.array_equal(got, np.array(Y, dtype=np.float64).reshape(w.M, w.d_out))


def pin_handworked(orc):
    with open(os.path.join(GOLDEN, "handworked_tiny.json")) as f:
        g = json.load(f)
    X = np.array(g["X"], np.float32)
    A = np.array(g["A_pool_rows_r_by_d_in"], np.float32)
    B = np.array(g["B_pool_rows_r_by_d_out"], np.float32)
    Y = np.array(g["Y_in"], np.float32)
    V = orc.shrink(X, A, g["seg_start"], g["seg_adapter"])
    assert np.array_equal(V, np.array(g["V"], np.float64)), V
    out = orc.sgmv(Y, X, A, B, g["seg_start"], g["seg_adapter"], g["alpha"])
    assert np.array_equal(out, np.array(g["Y_out"], np.float64)), out


def pin_zero_adapter(orc):
    rng = np.random.Generator(np.random.PCG64(14))
    for which in ("A", "B"):
        w = wl.random_case(rng, dtype=torch.bfloat16, max_M=16, max_seg=6, max_pool=4, allow_empty=False)
        zero_k = int(w.seg_adapter[0])
        pool = w.A_pool if which == "A" else w.B_pool
        pool[zero_k].zero_()
        got = _run(orc, w)
        y_in = _f64(w.Y)
        for s in range(w.num_segments):
            rows = slice(int(w.seg_start[s]), int(w.seg_start[s + 1]))
            if int(w.seg_adapter[s]) == zero_k:
                assert np.array_equal(got[rows], y_in[rows])
            else:
                # rows of other adapters do change (random weights)
                assert not np.array_equal(got[rows], y_in[rows])


def pin_linearity(orc):
    rng = np.random.Generator(np.random.PCG64(15))
    w = wl.random_case(rng, dtype=torch.float32, max_M=12, allow_empty=False)
    # integer-valued X1, X2 and a, b in quarters: a*X1 + b*X2 is exact in fp32
    X1 = torch.from_numpy(rng.integers(-100, 101, size=(w.M, w.d_in)).astype(np.float32))
    X2 = torch.from_numpy(rng.integers(-100, 101, size=(w.M, w.d_in)).astype(np.float32))
    a, b = 0.75, -1.5
    X12 = a * X1 + b * X2
    y0 = wl.storage(w.Y)
    args = (wl.storage(w.A_pool), wl.storage(w.B_pool), w.seg_start, w.seg_adapter, w.alpha)
    d1 = orc.sgmv(y0, X1.numpy(), *args) - _f64(w.Y)
    d2 = orc.sgmv(y0, X2.numpy(), *args) - _f64(w.Y)
    d12 = orc.sgmv(y0, X12.numpy(), *args) - _f64(w.Y)
    _rel_close(d12, a * d1 + b * d2, 1e-9)
    assert np.abs(d1).max() > 0
    # the delta does not depend on Y_in
    y_other = wl._normal(rng, (w.M, w.d_out), 1.0, torch.float32)
    d1b = orc.sgmv(y_other.numpy(), X1.numpy(), *args) - _f64(y_other)
    _rel_close(d1b, d1, 1e-9)


def pin_permutation(orc):
    rng = np.random.Generator(np.random.PCG64(16))
    for _ in range(5):
        w = wl.random_case(rng, dtype=torch.bfloat16, max_M=16, max_seg=6)
        got = _run(orc, w)
        order = rng.permutation(w.num_segments)
        lens = np.diff(w.seg_start)
        rows = np.concatenate([np.arange(w.seg_start[s], w.seg_start[s + 1]) for s in order] +
                              [np.zeros(0, np.int64)]).astype(np.int64)
        w2 = wl.Workload("perm", w.M, w.d_in, w.d_out, w.r, w.alpha, w.dtype, w.num_adapters,
                         wl.segments_from_lengths(lens[order]), w.seg_adapter[order].copy(),
                         X=w.X[torch.from_numpy(rows)], Y=w.Y[torch.from_numpy(rows)],
                         A_pool=w.A_pool, B_pool=w.B_pool)
        got2 = _run(orc, w2)
        assert np.array_equal(got2, got[rows])


def signature_inputs(seg_start, seg_adapter, num_adapters, d_in, d_out, r, mode, dtype=torch.bfloat16,
                     pool_device=None):
    """Weights that write each row's adapter id into columns 0..3 of its output.

    X[:, 0] = 1 and every other X is 0; alpha = r (scale 1); Y_in = 0. Base-16
    digit c of the id, plus one, lands in column c. Mode "A" encodes the id in
    A (B is an identity block), mode "B" in B (A picks X[:, 0]). The pools are
    built on `pool_device` (default: the host)."""
    M = int(seg_start[-1])
    X = torch.zeros((M, d_in), dtype=dtype)
    X[:, 0] = 1
    A = torch.zeros((num_adapters, r, d_in), dtype=dtype, device=pool_device)
    B = torch.zeros((num_adapters, r, d_out), dtype=dtype, device=pool_device)
    ids = torch.arange(num_adapters, device=pool_device)
    digits = torch.stack([(ids >> (4 * c)) & 15 for c in range(4)], dim=1) + 1  # P x 4
    if mode == "A":
        A[:, :4, 0] = digits.to(dtype)
        for c in range(4):
            B[:, c, c] = 1
    else:
        A[:, 0, 0] = 1
        B[:, 0, :4] = digits.to(dtype)
    return X, A, B, float(r)


def decode_signature(y: np.ndarray) -> np.ndarray:
    """Adapter id per row from columns 0..3 of a signature run's output."""
    d = np.rint(np.asarray(y[:, :4], np.float64)).astype(np.int64) - 1
    return d[:, 0] + 16 * d[:, 1] + 256 * d[:, 2] + 4096 * d[:, 3]


def row_adapter(seg_start, seg_adapter, M):
    out = np.full(M, -1, np.int64)
    for s in range(len(seg_adapter)):
        out[seg_start[s]:seg_start[s + 1]] = seg_adapter[s]
    return out


def pin_signature(orc):
    rng = np.random.Generator(np.random.PCG64(17))
    for _ in range(4):
        w = wl.random_case(rng, dtype=torch.bfloat16, max_M=16, max_seg=6, max_pool=5)
        for mode in ("A", "B"):
            X, A, B, alpha = signature_inputs(w.seg_start, w.seg_adapter, w.num_adapters,
                                              w.d_in, w.d_out, w.r, mode)
            Y = torch.zeros((w.M, w.d_out), dtype=torch.bfloat16)
            got = orc.sgmv(wl.storage(Y), wl.storage(X), wl.storage(A), wl.storage(B),
                           w.seg_start, w.seg_adapter, alpha)
            assert np.array_equal(decode_signature(got), row_adapter(w.seg_start, w.seg_adapter, w.M))
            assert np.all(got[:, 4:] == 0)


def pin_scale(orc):
    rng = np.random.Generator(np.random.PCG64(18))
    w = wl.random_case(rng, dtype=torch.bfloat16, allow_empty=False)
    w.Y = torch.zeros_like(w.Y)
    w.alpha = float(w.r)
    one = _run(orc, w)
    w.alpha = 2.0 * w.r
    two = _run(orc, w)
    assert np.array_equal(two, 2.0 * one)
    assert np.any(one != 0)


def pin_bf16_rounding(orc):
    rng = np.random.Generator(np.random.PCG64(19))
    vals = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(1000.0),
        rng.standard_normal(2000).astype(np.float32) * np.float32(1e-39),   # subnormal range
        np.array([0.0, -0.0, 1.0, -1.0, 3.0e38, -3.0e38, 1e-45], np.float32),
    ])
    want = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = orc.round_bf16(vals.astype(np.float64))
    assert np.array_equal(got, want)
    # hand-checked ties and near-ties (bf16 keeps 8 significant bits):
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7 -> ties to even -> 1.0 (0x3F80)
    # 1 + 3*2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6 -> even -> 1 + 2^-6 (0x3F82)
    # 1 + 2^-8 + 2^-40 is just above halfway -> 1 + 2^-7 (0x3F81); a double
    # rounding through fp32 would lose the 2^-40 and give 0x3F80
    cases = {1 + 2.0 ** -8: 0x3F80, 1 + 3 * 2.0 ** -8: 0x3F82, 1 + 2.0 ** -8 + 2.0 ** -40: 0x3F81,
             -(1 + 2.0 ** -8 + 2.0 ** -40): 0xBF81, 2.0 ** 128: 0x7F80, 1e300: 0x7F80}
    got = orc.round_bf16(np.array(list(cases.keys())))
    assert [int(v) for v in got] == list(cases.values()), [hex(int(v)) for v in got]


def pin_f32_rounding(orc):
    """Binary32 keeps 24 significant bits, exponents down to 2^-126 for
    normal numbers, subnormals on the fixed grid 2^-149, and its largest
    finite value is (2 - 2^-23) 2^127. Rounding is to nearest, ties to even.
    Each expected value below is worked by hand from those facts."""
    f32_max = float(np.float32(3.4028234663852886e38))
    assert f32_max == (2.0 - 2.0 ** -23) * 2.0 ** 127
    cases = [
        # 1 + 2^-24 lies halfway between 1 and 1 + 2^-23: even -> 1
        (1 + 2.0 ** -24, 1.0),
        # 1 + 3 2^-24 lies halfway between 1 + 2^-23 (odd) and 1 + 2^-22 (even)
        (1 + 3 * 2.0 ** -24, 1 + 2.0 ** -22),
        # just above the first tie: up. Rounding first to 25 bits and then to
        # 24 (a double rounding) would make it an exact tie and give 1.0
        (1 + 2.0 ** -24 + 2.0 ** -52, 1 + 2.0 ** -23),
        # just below the second tie: down to 1 + 2^-23
        (1 + 3 * 2.0 ** -24 - 2.0 ** -52, 1 + 2.0 ** -23),
        (-(1 + 2.0 ** -24 + 2.0 ** -52), -(1 + 2.0 ** -23)),
        # exactly representable values pass through
        (0.0, 0.0), (1.5, 1.5), (-1234.5, -1234.5), (2.0 ** -126, 2.0 ** -126), (f32_max, f32_max),
        # overflow: (2 - 2^-24) 2^127 is halfway between the largest finite
        # value (odd significand) and 2^128: even -> infinity; just below it
        # rounds to the largest finite value
        ((2.0 - 2.0 ** -24) * 2.0 ** 127, np.inf),
        (-(2.0 - 2.0 ** -24) * 2.0 ** 127, -np.inf),
        ((2.0 - 2.0 ** -24 - 2.0 ** -50) * 2.0 ** 127, f32_max),
        (1e300, np.inf), (np.inf, np.inf), (-np.inf, -np.inf),
        # subnormals: the grid is 2^-149; 2^-150 is halfway between 0 and
        # 2^-149 -> even (0); 3 2^-150 halfway between 2^-149 (odd) and 2^-148
        (2.0 ** -149, 2.0 ** -149), (2.0 ** -150, 0.0), (3 * 2.0 ** -150, 2.0 ** -148),
        (2.0 ** -150 + 2.0 ** -170, 2.0 ** -149), (5 * 2.0 ** -151, 2.0 ** -149),
        (-(3 * 2.0 ** -150), -(2.0 ** -148)), (2.0 ** -160, 0.0),
        # the largest subnormal and the step into the normal range
        ((2.0 ** 23 - 1) * 2.0 ** -149, (2.0 ** 23 - 1) * 2.0 ** -149),
        ((2.0 ** 23 - 0.5) * 2.0 ** -149, 2.0 ** -126),
    ]
    x = np.array([c[0] for c in cases], np.float64)
    got = orc.round_f32(x).astype(np.float64)
    want = np.array([c[1] for c in cases], np.float64)
    bad = [(x[i], got[i], want[i]) for i in range(len(cases)) if not got[i] == want[i]]
    assert not bad, bad
    # signs of zero survive: -0.0 and a negative value that rounds to zero
    z = orc.round_f32(np.array([-0.0, -(2.0 ** -151)]))
    assert np.all(z == 0) and np.all(np.signbit(z))
    assert np.isnan(orc.round_f32(np.array([np.nan]))[0])
    # a value between two binary32 neighbours goes to the nearer one: with
    # 24 significant bits the neighbours of 1 + t (0 < t < 2^-23) are 1 and
    # 1 + 2^-23
    rng = np.random.Generator(np.random.PCG64(23))
    t = rng.uniform(0, 2.0 ** -23, size=2000)
    t = t[np.abs(t - 2.0 ** -24) > 2.0 ** -50]
    got = orc.round_f32(1.0 + t).astype(np.float64)
    assert np.array_equal(got, np.where(t < 2.0 ** -24, 1.0, 1.0 + 2.0 ** -23))


def check_segments(token_adapter, perm, seg_start, seg_adapter):
    """The defining properties of grouping tokens by adapter: perm is a
    permutation; ids along perm are non-decreasing; equal ids keep their
    original order (stable); segments are the maximal runs, in order."""
    ids = np.asarray(token_adapter, np.int64)
    M = ids.shape[0]
    perm = np.asarray(perm, np.int64)
    assert sorted(perm.tolist()) == list(range(M))
    s_ids = ids[perm]
    assert np.all(np.diff(s_ids) >= 0)
    for p in range(1, M):
        if s_ids[p] == s_ids[p - 1]:
            assert perm[p] > perm[p - 1]
    ss = np.asarray(seg_start, np.int64)
    sa = np.asarray(seg_adapter, np.int64)
    assert ss.shape[0] == sa.shape[0] + 1 and ss[0] == 0 and ss[-1] == M
    for s in range(sa.shape[0]):
        assert ss[s] < ss[s + 1]
        assert np.all(s_ids[ss[s]:ss[s + 1]] == sa[s])
        if s > 0:
            assert sa[s] != sa[s - 1]
    assert len(set(sa.tolist())) == sa.shape[0]


def pin_segments(build_segments):
    rng = np.random.Generator(np.random.PCG64(20))
    cases = [np.zeros(0, np.int32), np.array([5], np.int32), np.array([3, 3, 3], np.int32),
             np.array([2, 0, 3, 1], np.int32), np.array([1, 0, 1, 0, 1], np.int32)]
    cases += [rng.integers(0, 7, size=int(rng.integers(1, 40))).astype(np.int32) for _ in range(50)]
    cases.append(wl.zipf_ids(rng, 256, 64))
    for ids in cases:
        perm, ss, sa = build_segments(ids)
        check_segments(ids, perm, ss, sa)
    # worked by hand: ids [1, 0, 1, 0, 1] -> tokens 1, 3 (id 0) then 0, 2, 4 (id 1)
    perm, ss, sa = build_segments(np.array([1, 0, 1, 0, 1], np.int32))
    assert list(perm) == [1, 3, 0, 2, 4] and list(ss) == [0, 2, 5] and list(sa) == [0, 1]


def pin_gather_per_token(orc, build_segments=None):
    """The batch left in token order: tokens carry adapter ids in any order,
    the grouping gives (perm, offsets, ids), and the gathered call with
    rows = perm must give every token t exactly the per-row equation with its
    own adapter, y_t += (alpha/r) x_t A_k(t) B_k(t) (Punica guide, "The
    Heterogeneous Batching Bottleneck"), worked in Python integers with no
    segments at all. V comes back in segment order: V[p] belongs to token
    perm[p]."""
    import oracle as oracle_pkg
    build_segments = build_segments or oracle_pkg.build_segments
    rng = np.random.Generator(np.random.PCG64(22))
    for _ in range(12):
        M = int(rng.integers(1, 13))
        P = int(rng.integers(1, 5))
        r = int(rng.choice([8, 16]))
        d_in, d_out = 8 * int(rng.integers(1, 4)), 8 * int(rng.integers(1, 4))
        ids = rng.integers(0, P, size=M).astype(np.int32)
        perm, ss, sa = build_segments(ids)
        w = wl.Workload("gather", M, d_in, d_out, r, 2.0 * r, torch.bfloat16, P, ss, sa)
        wl.integer_case(rng, w)
        X = w.X.to(torch.int64).tolist()
        A = w.A_pool.to(torch.int64).tolist()
        B = w.B_pool.to(torch.int64).tolist()
        Y = w.Y.to(torch.int64).tolist()
        Vt = []
        for t in range(M):
            k = int(ids[t])
            v = [sum(X[t][i] * A[k][j][i] for i in range(d_in)) for j in range(r)]
            Vt.append(v)
            for n in range(d_out):
                Y[t][n] += 2 * sum(v[j] * B[k][j][n] for j in range(r))
        args = (wl.storage(w.A_pool), wl.storage(w.B_pool), ss, sa)
        got = orc.sgmv_gather(wl.storage(w.Y), wl.storage(w.X), *args, perm, w.alpha)
        assert np.array_equal(got, np.array(Y, dtype=np.float64).reshape(M, d_out))
        V = orc.shrink_gather(wl.storage(w.X), wl.storage(w.A_pool), ss, sa, perm)
        want_v = np.array([Vt[int(t)] for t in perm], dtype=np.float64).reshape(M, r)
        assert np.array_equal(V, want_v)


ALL_PINS = [pin_dense_single_adapter, pin_dense_mask, pin_integer_bruteforce, pin_handworked,
            pin_zero_adapter, pin_linearity, pin_permutation, pin_signature, pin_scale,
            pin_bf16_rounding, pin_f32_rounding, pin_gather_per_token]
