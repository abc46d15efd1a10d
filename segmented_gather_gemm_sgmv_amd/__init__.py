"""Python binding of libsgmv.so, the MI355X SGMV library (C ABI in
``include/sgmv.h``).

Argument marshalling only: every function below checks tensor placement,
dtype and contiguity, passes raw device pointers, sizes and the current HIP
stream to the C function of the same name, and raises on a non-zero status.
All arithmetic runs in the library's gfx950 kernels. PyTorch supplies device
memory and streams.

If ``libsgmv.so`` has not been built, importing this package raises
``ImportError``: there is no fallback path.
"""
from __future__ import annotations

import ctypes
from pathlib import Path
from typing import Dict, Optional, Tuple

import numpy as np
import torch

_HERE = Path(__file__).resolve().parent
LIBRARY = _HERE / "libsgmv.so"

SGMV_F32 = 0
SGMV_BF16 = 1
SGMV_OK = 0

_DTYPES = {torch.float32: SGMV_F32, torch.bfloat16: SGMV_BF16}

# (name, restype, argtypes) for every symbol include/sgmv.h declares.
_i32, _i64, _vp, _f32, _sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_size_t
EXPORTS = {
    "sgmv_shrink": (ctypes.c_int, [_vp, _vp, _vp, _i32, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _vp,
                                   _sz, _vp]),
    "sgmv_expand": (ctypes.c_int, [_vp, _vp, _vp, _i32, _vp, _vp, _i32, _i32, _i32, _i32, _f32, _i32, _vp]),
    "sgmv_fused": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i32, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                  _f32, _i32, _vp, _sz, _vp]),
    "sgmv_fused_noalloc": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i32, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                          _f32, _i32, _vp]),
    "sgmv_shrink_gather": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i32, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                          _vp, _sz, _vp]),
    "sgmv_expand_scatter": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i32, _vp, _vp, _i32, _i32, _i32, _i32, _f32,
                                           _i32, _vp]),
    "sgmv_fused_gather": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _i32, _i32, _i32, _i32,
                                         _i32, _f32, _i32, _vp, _sz, _vp]),
    "sgmv_fused_layer": (ctypes.c_int, [_vp, _i32, _vp, _vp, _vp, _i32, _i32, _i32, _f32, _i32, _vp, _sz,
                                        _vp]),
    "sgmv_layer_workspace_bytes": (_sz, [_vp, _i32, _i32, _i32, _i32, _i32]),
    "sgmv_admit_adapter": (ctypes.c_int, [_vp, _vp, _vp, _vp, _sz, _sz, _vp, _vp, _i32, _i32, _vp]),
    "sgmv_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "sgmv_build_segments": (ctypes.c_int, [_vp, _i32, _vp, _vp, _vp, _vp]),
    "sgmv_pool_pointers": (ctypes.c_int, [_vp, _vp, _i32, _i64]),
    "sgmv_check_segments": (ctypes.c_int, [_vp, _vp, _i32, _i32, _i32]),
    "sgmv_stream_probe": (ctypes.c_int, [_vp, _sz, _vp, _i32, _vp]),
    "sgmv_workspace_status": (ctypes.c_int, [_vp, _vp, _vp]),
    "sgmv_set_wait_limit": (ctypes.c_uint32, [ctypes.c_uint32]),
    "sgmv_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "sgmv_version": (ctypes.c_int, []),
}


def _load() -> ctypes.CDLL:
    if not LIBRARY.exists():
        raise ImportError(f"{LIBRARY} is not built; run `python -m segmented_gather_gemm_sgmv_amd.build`")
    lib = ctypes.CDLL(str(LIBRARY))
    for name, (res, args) in EXPORTS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


class SGMVError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {lib.sgmv_status_string(status).decode()} (status {status})")
        self.status = status


def _check(fn: str, status: int) -> None:
    if status != SGMV_OK:
        raise SGMVError(fn, status)


def _dev(t: torch.Tensor, name: str, dtype=None, dim=None) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if dim is not None and t.dim() != dim:
        raise ValueError(f"{name} must have {dim} dimensions")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(t: torch.Tensor, stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")
    return _DTYPES[t.dtype]


def _workspace_args(t: Optional[torch.Tensor], need: int, like: torch.Tensor, stream):
    if need == 0 and t is None:
        return None, 0
    if t is None:
        t = workspace(like.device, need, stream)
    return _dev(t, "workspace"), t.numel() * t.element_size()


def sgmv_shrink(V: torch.Tensor, X: torch.Tensor, A_ptrs: torch.Tensor, seg_start: torch.Tensor,
                seg_adapter: torch.Tensor, r: int, workspace_buf: Optional[torch.Tensor] = None,
                stream=None) -> torch.Tensor:
    """V[M, r] (fp32, overwritten per segment row) = X[M, d_in] . A_k."""
    M, d_in = X.shape
    if V.shape != (M, r):
        raise ValueError("V must be M x r")
    need = sgmv_workspace_bytes(seg_adapter.numel(), M, d_in, d_in, r, X.dtype)
    ws, ws_bytes = _workspace_args(workspace_buf, need, X, stream)
    st = lib.sgmv_shrink(_dev(V, "V", torch.float32, 2), _dev(X, "X", dim=2),
                         _dev(A_ptrs, "A_ptrs", torch.int64, 1), A_ptrs.numel(),
                         _dev(seg_start, "seg_start", torch.int32, 1),
                         _dev(seg_adapter, "seg_adapter", torch.int32, 1), seg_adapter.numel(),
                         M, d_in, r, _dtype_code(X), ws, ws_bytes, _stream(X, stream))
    _check("sgmv_shrink", st)
    return V


def sgmv_expand(Y: torch.Tensor, V: torch.Tensor, B_ptrs: torch.Tensor, seg_start: torch.Tensor,
                seg_adapter: torch.Tensor, r: int, alpha: float, stream=None) -> torch.Tensor:
    """Y[M, d_out] += (alpha / r) * V . B_k per segment (in place)."""
    M, d_out = Y.shape
    if V.shape != (M, r):
        raise ValueError("V must be M x r")
    st = lib.sgmv_expand(_dev(Y, "Y", dim=2), _dev(V, "V", torch.float32, 2),
                         _dev(B_ptrs, "B_ptrs", torch.int64, 1), B_ptrs.numel(),
                         _dev(seg_start, "seg_start", torch.int32, 1),
                         _dev(seg_adapter, "seg_adapter", torch.int32, 1), seg_adapter.numel(),
                         M, d_out, r, float(alpha), _dtype_code(Y), _stream(Y, stream))
    _check("sgmv_expand", st)
    return Y


def sgmv_workspace_bytes(num_segments: int, M: int, d_in: int, d_out: int, r: int,
                         dtype: torch.dtype) -> int:
    return int(lib.sgmv_workspace_bytes(num_segments, M, d_in, d_out, r, _DTYPES[dtype]))


_workspaces: Dict[Tuple[int, int], torch.Tensor] = {}


def _torch_stream(device: torch.device, stream):
    """`stream` (None, a torch stream or a raw hipStream_t handle) as a torch
    stream object on `device`."""
    if stream is None:
        return torch.cuda.current_stream(device)
    if isinstance(stream, (torch.cuda.Stream, torch.cuda.ExternalStream)):
        return stream
    return torch.cuda.ExternalStream(int(stream), device=device)


def workspace(device: torch.device, nbytes: int, stream=None) -> torch.Tensor:
    """A zero-filled workspace for sgmv_shrink and sgmv_fused, cached per
    (device, stream).

    Every call leaves the workspace zero again when its kernel completes, so
    one buffer serves every later call on the same stream. The buffer is
    allocated and zero-filled on that stream, so the fill is ordered before
    the calls that use it, and the caching allocator hands a replaced buffer
    to later work on the same stream only."""
    device = torch.device(device)
    if device.index is None:
        device = torch.device(device.type, torch.cuda.current_device())
    s = _torch_stream(device, stream)
    key = (device.index, s.cuda_stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        with torch.cuda.device(device), torch.cuda.stream(s):
            ws = torch.zeros(max(nbytes, 1 << 16), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def sgmv_workspace_status(ws: torch.Tensor, stream=None) -> int:
    """The workspace's sticky status word (0, or the OR of SGMV_WS_WAIT_TIMEOUT
    and SGMV_WS_BAD_OFFSETS), read after the work enqueued on `stream`
    (default: the current stream) has completed. A non-zero status stays
    until the workspace is zero-filled again; until then every call on it is
    a no-op."""
    word = ctypes.c_uint32(0)
    _check("sgmv_workspace_status", lib.sgmv_workspace_status(_dev(ws, "workspace"), ctypes.byref(word),
                                                              _stream(ws, stream)))
    return int(word.value)


def sgmv_set_wait_limit(polls: int) -> int:
    """Polls a waiting workgroup makes before it gives up, for calls launched
    from now on (process-wide); returns the previous value."""
    return int(lib.sgmv_set_wait_limit(int(polls)))


SGMV_WS_WAIT_TIMEOUT = 1
SGMV_WS_BAD_OFFSETS = 2


def sgmv_fused(Y: torch.Tensor, X: torch.Tensor, A_ptrs: torch.Tensor, B_ptrs: torch.Tensor,
               seg_start: torch.Tensor, seg_adapter: torch.Tensor, r: int, alpha: float,
               workspace_buf: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Y += (alpha / r) * X . A_k . B_k per segment, in one launch (in place)."""
    M, d_in = X.shape
    M2, d_out = Y.shape
    if M2 != M:
        raise ValueError("X and Y must have the same number of rows")
    if A_ptrs.numel() != B_ptrs.numel():
        raise ValueError("A_ptrs and B_ptrs must have one entry per adapter")
    need = sgmv_workspace_bytes(seg_adapter.numel(), M, d_in, d_out, r, X.dtype)
    ws, ws_bytes = _workspace_args(workspace_buf, need, X, stream)
    st = lib.sgmv_fused(_dev(Y, "Y", dim=2), _dev(X, "X", dim=2),
                        _dev(A_ptrs, "A_ptrs", torch.int64, 1), _dev(B_ptrs, "B_ptrs", torch.int64, 1),
                        A_ptrs.numel(), _dev(seg_start, "seg_start", torch.int32, 1),
                        _dev(seg_adapter, "seg_adapter", torch.int32, 1), seg_adapter.numel(),
                        M, d_in, d_out, r, float(alpha), _dtype_code(X), ws, ws_bytes,
                        _stream(X, stream))
    _check("sgmv_fused", st)
    return Y


SGMV_NOALLOC_SCRATCH_BYTES = 16 << 20


def sgmv_fused_noalloc(Y: torch.Tensor, X: torch.Tensor, A_ptrs: torch.Tensor, B_ptrs: torch.Tensor,
                       seg_start: torch.Tensor, seg_adapter: torch.Tensor, r: int, alpha: float,
                       stream=None) -> torch.Tensor:
    """sgmv_fused on the library's static per-device scratch array instead of
    a workspace: nothing is allocated. Calls that overlap in time on one GPU
    must not be made (they share the array)."""
    M, d_in = X.shape
    M2, d_out = Y.shape
    if M2 != M:
        raise ValueError("X and Y must have the same number of rows")
    if A_ptrs.numel() != B_ptrs.numel():
        raise ValueError("A_ptrs and B_ptrs must have one entry per adapter")
    st = lib.sgmv_fused_noalloc(_dev(Y, "Y", dim=2), _dev(X, "X", dim=2),
                                _dev(A_ptrs, "A_ptrs", torch.int64, 1), _dev(B_ptrs, "B_ptrs", torch.int64, 1),
                                A_ptrs.numel(), _dev(seg_start, "seg_start", torch.int32, 1),
                                _dev(seg_adapter, "seg_adapter", torch.int32, 1), seg_adapter.numel(),
                                M, d_in, d_out, r, float(alpha), _dtype_code(X), _stream(X, stream))
    _check("sgmv_fused_noalloc", st)
    return Y


def _rows_arg(rows: torch.Tensor, M: int) -> int:
    if rows.numel() != M:
        raise ValueError("rows must hold one entry per row of the batch")
    return _dev(rows, "rows", torch.int32, 1)


def sgmv_shrink_gather(V: torch.Tensor, X: torch.Tensor, rows: torch.Tensor, A_ptrs: torch.Tensor,
                       seg_start: torch.Tensor, seg_adapter: torch.Tensor, r: int,
                       workspace_buf: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """V[p] (fp32, segment order) = X[rows[p]] . A_k, with X in token order."""
    M, d_in = X.shape
    if V.shape != (M, r):
        raise ValueError("V must be M x r")
    need = sgmv_workspace_bytes(seg_adapter.numel(), M, d_in, d_in, r, X.dtype)
    ws, ws_bytes = _workspace_args(workspace_buf, need, X, stream)
    st = lib.sgmv_shrink_gather(_dev(V, "V", torch.float32, 2), _dev(X, "X", dim=2), _rows_arg(rows, M),
                                _dev(A_ptrs, "A_ptrs", torch.int64, 1), A_ptrs.numel(),
                                _dev(seg_start, "seg_start", torch.int32, 1),
                                _dev(seg_adapter, "seg_adapter", torch.int32, 1), seg_adapter.numel(),
                                M, d_in, r, _dtype_code(X), ws, ws_bytes, _stream(X, stream))
    _check("sgmv_shrink_gather", st)
    return V


def sgmv_expand_scatter(Y: torch.Tensor, V: torch.Tensor, rows: torch.Tensor, B_ptrs: torch.Tensor,
                        seg_start: torch.Tensor, seg_adapter: torch.Tensor, r: int, alpha: float,
                        stream=None) -> torch.Tensor:
    """Y[rows[p]] += (alpha / r) * V[p] . B_k, with Y in token order (in place)."""
    M, d_out = Y.shape
    if V.shape != (M, r):
        raise ValueError("V must be M x r")
    st = lib.sgmv_expand_scatter(_dev(Y, "Y", dim=2), _dev(V, "V", torch.float32, 2), _rows_arg(rows, M),
                                 _dev(B_ptrs, "B_ptrs", torch.int64, 1), B_ptrs.numel(),
                                 _dev(seg_start, "seg_start", torch.int32, 1),
                                 _dev(seg_adapter, "seg_adapter", torch.int32, 1), seg_adapter.numel(),
                                 M, d_out, r, float(alpha), _dtype_code(Y), _stream(Y, stream))
    _check("sgmv_expand_scatter", st)
    return Y


def sgmv_fused_gather(Y: torch.Tensor, X: torch.Tensor, rows: torch.Tensor, A_ptrs: torch.Tensor,
                      B_ptrs: torch.Tensor, seg_start: torch.Tensor, seg_adapter: torch.Tensor, r: int,
                      alpha: float, workspace_buf: Optional[torch.Tensor] = None,
                      stream=None) -> torch.Tensor:
    """Y[rows[p]] += (alpha / r) * X[rows[p]] . A_k . B_k in one launch, with X
    and Y in token order (in place)."""
    M, d_in = X.shape
    M2, d_out = Y.shape
    if M2 != M:
        raise ValueError("X and Y must have the same number of rows")
    if A_ptrs.numel() != B_ptrs.numel():
        raise ValueError("A_ptrs and B_ptrs must have one entry per adapter")
    need = sgmv_workspace_bytes(seg_adapter.numel(), M, d_in, d_out, r, X.dtype)
    ws, ws_bytes = _workspace_args(workspace_buf, need, X, stream)
    st = lib.sgmv_fused_gather(_dev(Y, "Y", dim=2), _dev(X, "X", dim=2), _rows_arg(rows, M),
                               _dev(A_ptrs, "A_ptrs", torch.int64, 1), _dev(B_ptrs, "B_ptrs", torch.int64, 1),
                               A_ptrs.numel(), _dev(seg_start, "seg_start", torch.int32, 1),
                               _dev(seg_adapter, "seg_adapter", torch.int32, 1), seg_adapter.numel(),
                               M, d_in, d_out, r, float(alpha), _dtype_code(X), ws, ws_bytes,
                               _stream(X, stream))
    _check("sgmv_fused_gather", st)
    return Y


SGMV_MAX_PROJECTIONS = 8


class SgmvProjection(ctypes.Structure):
    """``sgmv_projection`` of include/sgmv.h: one projection of a layer call."""
    _fields_ = [("Y", ctypes.c_void_p), ("X", ctypes.c_void_p), ("A_ptrs", ctypes.c_void_p),
                ("B_ptrs", ctypes.c_void_p), ("num_adapters", ctypes.c_int32), ("d_in", ctypes.c_int32),
                ("d_out", ctypes.c_int32)]


def _projection_array(projections, check=True):
    """(Y, X, A_ptrs, B_ptrs) tuples -> a ctypes array of SgmvProjection."""
    arr = (SgmvProjection * max(1, len(projections)))()
    for q, (Y, X, A_ptrs, B_ptrs) in enumerate(projections):
        if check:
            if X.shape[0] != Y.shape[0]:
                raise ValueError(f"projection {q}: X and Y must have the same number of rows")
            if A_ptrs.numel() != B_ptrs.numel():
                raise ValueError(f"projection {q}: A_ptrs and B_ptrs must have one entry per adapter")
        arr[q] = SgmvProjection(_dev(Y, "Y", dim=2), _dev(X, "X", dim=2),
                                _dev(A_ptrs, "A_ptrs", torch.int64, 1), _dev(B_ptrs, "B_ptrs", torch.int64, 1),
                                A_ptrs.numel(), X.shape[1], Y.shape[1])
    return arr


def sgmv_layer_workspace_bytes(projections, num_segments: int, M: int, r: int, dtype: torch.dtype) -> int:
    arr = _projection_array(projections)
    return int(lib.sgmv_layer_workspace_bytes(arr, len(projections), num_segments, M, r, _DTYPES[dtype]))


def sgmv_fused_layer(projections, seg_start: torch.Tensor, seg_adapter: torch.Tensor, r: int, alpha: float,
                     rows: Optional[torch.Tensor] = None, workspace_buf: Optional[torch.Tensor] = None,
                     stream=None):
    """Every projection (Y, X, A_ptrs, B_ptrs) of one batch in one launch:
    Y += (alpha / r) * X . A_k . B_k per projection (in place). ``rows``: None
    for a batch in segment order, else the token-order index."""
    if not projections:
        return
    Y0, X0 = projections[0][0], projections[0][1]
    M = X0.shape[0]
    for Y, X, _, _ in projections:
        if X.shape[0] != M or Y.shape[0] != M:
            raise ValueError("every projection must have the batch's M rows")
        if X.dtype != X0.dtype or Y.dtype != X0.dtype:
            raise TypeError("every projection must share one dtype")
    arr = _projection_array(projections)
    need = int(lib.sgmv_layer_workspace_bytes(arr, len(projections), seg_adapter.numel(), M, r,
                                              _dtype_code(X0)))
    ws, ws_bytes = _workspace_args(workspace_buf, need, X0, stream)
    rows_p = None if rows is None else _rows_arg(rows, M)
    st = lib.sgmv_fused_layer(arr, len(projections), rows_p, _dev(seg_start, "seg_start", torch.int32, 1),
                              _dev(seg_adapter, "seg_adapter", torch.int32, 1), seg_adapter.numel(), M, r,
                              float(alpha), _dtype_code(X0), ws, ws_bytes, _stream(X0, stream))
    _check("sgmv_fused_layer", st)


def sgmv_build_segments(token_adapter) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Host: group tokens by adapter. Returns (perm, seg_start, seg_adapter)."""
    ids = np.ascontiguousarray(np.asarray(token_adapter, dtype=np.int32))
    M = int(ids.shape[0])
    perm = np.empty(M, np.int32)
    seg_start = np.empty(M + 1, np.int32)
    seg_adapter = np.empty(max(M, 1), np.int32)
    n = ctypes.c_int32(0)
    st = lib.sgmv_build_segments(ids.ctypes.data, M, perm.ctypes.data, seg_start.ctypes.data,
                                 seg_adapter.ctypes.data, ctypes.byref(n))
    _check("sgmv_build_segments", st)
    return perm, seg_start[: n.value + 1].copy(), seg_adapter[: n.value].copy()


def sgmv_pool_pointers(pool: torch.Tensor) -> torch.Tensor:
    """Device table (int64) of slot addresses of a packed pool tensor P x r x d.

    The table holds a reference to ``pool``, so the memory it points into
    cannot be freed while the table is alive."""
    if pool.dim() != 3 or not pool.is_contiguous():
        raise ValueError("pool must be a contiguous P x r x d tensor")
    P = pool.shape[0]
    table = np.empty(max(P, 1), np.uint64)
    slot_bytes = pool.shape[1] * pool.shape[2] * pool.element_size()
    st = lib.sgmv_pool_pointers(table.ctypes.data, ctypes.c_void_p(pool.data_ptr()), P, slot_bytes)
    _check("sgmv_pool_pointers", st)
    out = torch.from_numpy(table[:P].view(np.int64).copy()).to(pool.device)
    out._sgmv_pool = pool
    return out


def sgmv_admit_adapter(A_slot: torch.Tensor, B_slot: torch.Tensor, A_host: torch.Tensor, B_host: torch.Tensor,
                       A_ptrs: torch.Tensor, B_ptrs: torch.Tensor, slot: int, stream=None) -> None:
    """Copy an adapter from host memory into device slots A_slot (r x d_in)
    and B_slot (r x d_out), then point table entry `slot` at them, all in
    stream order. A_host / B_host: CPU tensors of the slots' shape and dtype
    (pinned for an asynchronous copy); keep them alive and unchanged until the
    stream reaches the copy."""
    for name, dev_t, host_t in (("A", A_slot, A_host), ("B", B_slot, B_host)):
        if host_t.device.type != "cpu" or not host_t.is_contiguous():
            raise ValueError(f"{name}_host must be a contiguous CPU tensor")
        if host_t.shape != dev_t.shape or host_t.dtype != dev_t.dtype:
            raise ValueError(f"{name}_host must match {name}_slot in shape and dtype")
    if A_ptrs.numel() != B_ptrs.numel():
        raise ValueError("A_ptrs and B_ptrs must have one entry per adapter")
    st = lib.sgmv_admit_adapter(_dev(A_slot, "A_slot"), _dev(B_slot, "B_slot"), A_host.data_ptr(),
                                B_host.data_ptr(), A_host.numel() * A_host.element_size(),
                                B_host.numel() * B_host.element_size(), _dev(A_ptrs, "A_ptrs", torch.int64, 1),
                                _dev(B_ptrs, "B_ptrs", torch.int64, 1), int(slot), A_ptrs.numel(),
                                _stream(A_slot, stream))
    _check("sgmv_admit_adapter", st)


def sgmv_check_segments(seg_start, seg_adapter, M: int, num_adapters: int) -> None:
    """Host check of segment metadata (numpy or CPU tensors): raises SGMVError
    unless the offsets start at 0, end at M and never decrease, and every
    adapter id lies in the pool."""
    ss = np.ascontiguousarray(np.asarray(seg_start, dtype=np.int32))
    sa = np.ascontiguousarray(np.asarray(seg_adapter, dtype=np.int32))
    if ss.ndim != 1 or sa.ndim != 1 or ss.shape[0] != sa.shape[0] + 1:
        raise ValueError("seg_start must hold one more entry than seg_adapter")
    _check("sgmv_check_segments",
           lib.sgmv_check_segments(ss.ctypes.data, sa.ctypes.data if sa.size else None, sa.shape[0], M,
                                   num_adapters))


class AdapterPool:
    """One projection's adapter pool in HBM: P slots of A (r x d_in) and B
    (r x d_out), packed back to back, with their device pointer tables.

    ``A_ptrs`` / ``B_ptrs`` are what the SGMV calls take. ``admit`` copies an
    adapter from host memory into a slot and points the slot's table entries
    at it, in stream order (sgmv_admit_adapter); the slot's memory is this
    pool's own."""

    def __init__(self, num_adapters: int, d_in: int, d_out: int, r: int, dtype=torch.bfloat16,
                 device="cuda"):
        self.num_adapters, self.d_in, self.d_out, self.r, self.dtype = num_adapters, d_in, d_out, r, dtype
        self.A = torch.zeros((num_adapters, r, d_in), dtype=dtype, device=device)
        self.B = torch.zeros((num_adapters, r, d_out), dtype=dtype, device=device)
        self.A_ptrs = sgmv_pool_pointers(self.A)
        self.B_ptrs = sgmv_pool_pointers(self.B)

    def admit(self, slot: int, A_host: torch.Tensor, B_host: torch.Tensor, stream=None) -> None:
        """Adapter `slot` := (A_host, B_host), CPU tensors of shape r x d_in and
        r x d_out (pinned for an asynchronous copy; keep them alive and
        unchanged until the stream reaches the copy)."""
        if not 0 <= slot < self.num_adapters:
            raise IndexError(f"slot {slot} outside the pool of {self.num_adapters}")
        sgmv_admit_adapter(self.A[slot], self.B[slot], A_host, B_host, self.A_ptrs, self.B_ptrs, slot, stream)


def sgmv_stream_probe(src: torch.Tensor, sink: torch.Tensor, nbytes: Optional[int] = None, stream=None) -> None:
    """Measurement helper: stream-read `nbytes` (default: all) of the device
    tensor `src` with sink.numel() workgroups; sink (int32) receives each
    workgroup's XOR of the words it read."""
    n = src.numel() * src.element_size() if nbytes is None else int(nbytes)
    if n > src.numel() * src.element_size():
        raise ValueError("nbytes exceeds the source tensor")
    st = lib.sgmv_stream_probe(_dev(src, "src"), n, _dev(sink, "sink", torch.int32, 1), sink.numel(),
                               _stream(src, stream))
    _check("sgmv_stream_probe", st)


def sgmv_version() -> int:
    return int(lib.sgmv_version())


__all__ = ["sgmv_shrink", "sgmv_expand", "sgmv_fused", "sgmv_shrink_gather", "sgmv_expand_scatter",
           "sgmv_fused_gather", "sgmv_fused_layer", "sgmv_layer_workspace_bytes", "SgmvProjection",
           "SGMV_MAX_PROJECTIONS", "sgmv_admit_adapter", "sgmv_check_segments", "AdapterPool", "sgmv_stream_probe",
           "sgmv_workspace_bytes", "sgmv_build_segments",
           "sgmv_pool_pointers", "sgmv_version", "workspace", "SGMVError", "lib", "EXPORTS",
           "LIBRARY", "SGMV_F32", "SGMV_BF16", "sgmv_workspace_status", "sgmv_set_wait_limit",
           "SGMV_WS_WAIT_TIMEOUT", "SGMV_WS_BAD_OFFSETS", "sgmv_fused_noalloc", "SGMV_NOALLOC_SCRATCH_BYTES"]
