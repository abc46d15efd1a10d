"""SGMV oracle: a plain, slow CPU implementation of the segmented LoRA delta.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The product
library never loads it, and it shares no code with the HIP path.

What it follows (Punica guide, aifetchly blog):

* section "The Heterogeneous Batching Bottleneck", equation for ``y_i``: each
  row adds ``(alpha / r) * x_i A_k(i) B_k(i)`` to its base output, with
  ``A_k`` of logical shape d_in x r and ``B_k`` of logical shape r x d_out;
* section "The SGMV Mathematical Formulation": contiguous segments given by
  offsets ``s_0 .. s_N``, each tied to one adapter through an array of
  pointers, rows ``s_i .. s_{i+1}`` (half-open) multiplied by that adapter;
* section "Hardware-Level Optimizations in SGMV": requests are grouped by
  adapter ("pre-sorts segment descriptors") so each segment is contiguous —
  ``build_segments`` below.

Every floating-point step runs in float64 in ``sgmv_oracle.c`` (built with
gcc by :func:`build`); inputs are widened exactly from fp32 or bf16.

Pins: every function here is checked against values fixed independently of
its own formula — see ``tests/test_oracle_pins.py`` (dense single-adapter
GEMM, a dense mask formulation, exact integer brute force, a hand-worked
fixture, zero adapters, linearity, permutation equivariance, adapter-id
signatures, exact power-of-two scaling, bf16 rounding against torch's
conversion) and ``tests/test_oracle_mutants.py`` (planted mistakes in a copy
of the C source must each fail a pin). No function is parity-unpinned.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
SOURCE = _HERE / "sgmv_oracle.c"
LIBRARY = _HERE / "liboracle.so"

F32 = 0
BF16 = 1

_DP = ctypes.POINTER(ctypes.c_double)


def build(source: Path = SOURCE, output: Path = LIBRARY) -> Path:
    """Compile the oracle with gcc: no fast-math, no contraction into FMA."""
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-fPIC", "-shared", "-std=c11", str(source), "-o", str(output), "-lm"]
    subprocess.run(cmd, check=True)
    return output


class Oracle:
    """ctypes view of one build of ``sgmv_oracle.c``."""

    def __init__(self, lib_path: Path | str = LIBRARY):
        lib_path = Path(lib_path)
        if not lib_path.exists():
            build(output=lib_path)
        self.lib = ctypes.CDLL(str(lib_path))
        i32, i64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
        self.lib.oracle_shrink.argtypes = [_DP, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32]
        self.lib.oracle_shrink.restype = ctypes.c_int
        self.lib.oracle_expand.argtypes = [_DP, _DP, vp, vp, vp, i32, i32, i32, i32, i32,
                                           ctypes.c_double, i32]
        self.lib.oracle_expand.restype = ctypes.c_int
        self.lib.oracle_widen.argtypes = [_DP, vp, i64, i32]
        self.lib.oracle_round_bf16.argtypes = [vp, _DP, i64]
        self.lib.oracle_round_f32.argtypes = [vp, _DP, i64]

    # -- helpers -----------------------------------------------------------
    @staticmethod
    def _storage(a: np.ndarray) -> tuple[np.ndarray, int]:
        """Inputs are fp32 arrays or bf16 bit patterns held as uint16/int16."""
        a = np.ascontiguousarray(a)
        if a.dtype == np.float32:
            return a, F32
        if a.dtype in (np.uint16, np.int16):
            return a, BF16
        raise TypeError(f"oracle inputs are float32 or bf16 bits, got {a.dtype}")

    @staticmethod
    def _meta(seg_start, seg_adapter):
        ss = np.ascontiguousarray(seg_start, dtype=np.int32)
        sa = np.ascontiguousarray(seg_adapter, dtype=np.int32)
        if ss.shape[0] != sa.shape[0] + 1:
            raise ValueError("seg_start must hold one more entry than seg_adapter")
        return ss, sa

    def widen(self, a: np.ndarray) -> np.ndarray:
        a, dt = self._storage(a)
        out = np.empty(a.shape, dtype=np.float64)
        self.lib.oracle_widen(out.ctypes.data_as(_DP), a.ctypes.data, a.size, dt)
        return out

    # -- the method ----------------------------------------------------------
    def shrink(self, X, A_pool, seg_start, seg_adapter, V_init=None) -> np.ndarray:
        """V = X_seg . A_k per segment (float64, M x r).

        ``X``: M x d_in; ``A_pool``: P x r x d_in (slot k holds A_k as r rows of
        d_in). Rows in no segment keep ``V_init`` (zeros by default)."""
        X, dt = self._storage(X)
        A_pool, dta = self._storage(A_pool)
        if dt != dta:
            raise TypeError("X and A_pool must share one storage type")
        ss, sa = self._meta(seg_start, seg_adapter)
        M, d_in = X.shape
        P, r, d_in_a = A_pool.shape
        if d_in_a != d_in:
            raise ValueError("A_pool slots must have d_in columns")
        V = np.zeros((M, r)) if V_init is None else np.array(V_init, dtype=np.float64)
        rc = self.lib.oracle_shrink(V.ctypes.data_as(_DP), X.ctypes.data, A_pool.ctypes.data,
                                    ss.ctypes.data, sa.ctypes.data, sa.shape[0], P, M, d_in, r, dt)
        if rc != 0:
            raise ValueError("adapter id outside the pool")
        return V

    def expand(self, Y_in, V, B_pool, seg_start, seg_adapter, alpha: float) -> np.ndarray:
        """Y = Y_in + (alpha / r) * V . B_k per segment (float64, M x d_out)."""
        B_pool, dt = self._storage(B_pool)
        ss, sa = self._meta(seg_start, seg_adapter)
        Y = self.widen(Y_in) if Y_in.dtype != np.float64 else np.array(Y_in, dtype=np.float64)
        Y = np.ascontiguousarray(Y)
        V = np.ascontiguousarray(V, dtype=np.float64)
        M, d_out = Y.shape
        P, r, d_out_b = B_pool.shape
        if d_out_b != d_out or V.shape != (M, r):
            raise ValueError("shape mismatch between Y, V and B_pool")
        rc = self.lib.oracle_expand(Y.ctypes.data_as(_DP), V.ctypes.data_as(_DP),
                                    B_pool.ctypes.data, ss.ctypes.data, sa.ctypes.data,
                                    sa.shape[0], P, M, r, d_out, float(alpha), dt)
        if rc != 0:
            raise ValueError("adapter id outside the pool")
        return Y

    def sgmv(self, Y_in, X, A_pool, B_pool, seg_start, seg_adapter, alpha: float) -> np.ndarray:
        """Y = Y_in + (alpha / r) * X_seg . A_k . B_k: expand after shrink."""
        V = self.shrink(X, A_pool, seg_start, seg_adapter)
        return self.expand(Y_in, V, B_pool, seg_start, seg_adapter, alpha)

    # -- the batch left in token order ---------------------------------------
    # Punica guide, figure "CUDA Threadblock Tiling": a segment's block gathers
    # the rows of activations that belong to it. Here the batch is not moved
    # into segment order first: segment row p (rows seg_start[s] ..
    # seg_start[s+1]-1 as above) is token row rows[p] of X and of Y.
    @staticmethod
    def _rows(rows, M: int) -> np.ndarray:
        rows = np.asarray(rows, dtype=np.int64)
        if rows.shape != (M,) or not np.array_equal(np.sort(rows), np.arange(M)):
            raise ValueError("rows must be a permutation of 0 .. M-1")
        return rows

    def shrink_gather(self, X, A_pool, seg_start, seg_adapter, rows) -> np.ndarray:
        """V[p] = X[rows[p]] . A_k for every segment row p (float64, M x r, in
        segment order): the gathered rows of X, then the shrink above."""
        X, _ = self._storage(X)
        rows = self._rows(rows, X.shape[0])
        return self.shrink(np.ascontiguousarray(X[rows]), A_pool, seg_start, seg_adapter)

    def expand_scatter(self, Y_in, V, B_pool, seg_start, seg_adapter, rows, alpha: float) -> np.ndarray:
        """Y[rows[p]] = Y_in[rows[p]] + (alpha / r) * V[p] . B_k (float64, token
        order): the gathered rows of Y, the expand above, then each result put
        back at its token row."""
        rows = self._rows(rows, Y_in.shape[0])
        Y = self.widen(Y_in) if Y_in.dtype != np.float64 else np.array(Y_in, dtype=np.float64)
        Y[rows] = self.expand(np.ascontiguousarray(Y[rows]), V, B_pool, seg_start, seg_adapter, alpha)
        return Y

    def sgmv_gather(self, Y_in, X, A_pool, B_pool, seg_start, seg_adapter, rows,
                    alpha: float) -> np.ndarray:
        """Y[rows[p]] += (alpha / r) * X[rows[p]] . A_k . B_k (float64, token order)."""
        V = self.shrink_gather(X, A_pool, seg_start, seg_adapter, rows)
        return self.expand_scatter(Y_in, V, B_pool, seg_start, seg_adapter, rows, alpha)

    def round_bf16(self, y: np.ndarray) -> np.ndarray:
        """float64 -> bf16 bit patterns (uint16), nearest-even, one rounding."""
        y = np.ascontiguousarray(y, dtype=np.float64)
        out = np.empty(y.shape, dtype=np.uint16)
        self.lib.oracle_round_bf16(out.ctypes.data, y.ctypes.data_as(_DP), y.size)
        return out

    def round_f32(self, y: np.ndarray) -> np.ndarray:
        y = np.ascontiguousarray(y, dtype=np.float64)
        out = np.empty(y.shape, dtype=np.float32)
        self.lib.oracle_round_f32(out.ctypes.data, y.ctypes.data_as(_DP), y.size)
        return out


def build_segments(token_adapter) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Group a batch's tokens by adapter into contiguous segments.

    Returns ``(perm, seg_start, seg_adapter)``: ``perm`` is the stable sort of
    token indices by adapter id (row ``p`` of the segmented batch is token
    ``perm[p]``), ``seg_start`` holds N+1 offsets with ``seg_start[0] = 0`` and
    ``seg_start[N] = M``, and ``seg_adapter[s]`` is segment ``s``'s adapter.
    (Punica guide, "Hardware-Level Optimizations in SGMV": tokens of one
    adapter are gathered into a contiguous range; "The SGMV Mathematical
    Formulation": the offsets ``s_0 .. s_N``.)"""
    ids = np.asarray(token_adapter, dtype=np.int64)
    perm = np.argsort(ids, kind="stable")
    sorted_ids = ids[perm]
    starts = [0]
    adapters = []
    for p in range(sorted_ids.shape[0]):
        if p == 0 or sorted_ids[p] != sorted_ids[p - 1]:
            if p > 0:
                starts.append(p)
            adapters.append(int(sorted_ids[p]))
    if sorted_ids.shape[0] > 0:
        starts.append(int(sorted_ids.shape[0]))
    return (perm.astype(np.int32), np.asarray(starts, dtype=np.int32),
            np.asarray(adapters, dtype=np.int32))


_default: Oracle | None = None


def get() -> Oracle:
    """The oracle built from ``sgmv_oracle.c`` (compiled on first use), or
    the build named by the environment variable SGMV_ORACLE_LIBRARY (the
    tests load a sanitizer build of the same source that way)."""
    global _default
    if _default is None:
        _default = Oracle(os.environ.get("SGMV_ORACLE_LIBRARY") or LIBRARY)
    return _default


def threads_used() -> int:
    """OpenMP threads the oracle's loops run on now (the OpenMP runtime the
    oracle library is linked with: OMP_NUM_THREADS, else all CPUs of this
    process's affinity mask, unless set_threads changed it)."""
    return int(get().lib.omp_get_max_threads())


def set_threads(n: int) -> int:
    """Run the oracle's loops on n OpenMP threads from now on; returns the
    previous count."""
    lib = get().lib
    old = int(lib.omp_get_max_threads())
    lib.omp_set_num_threads(int(n))
    return old
