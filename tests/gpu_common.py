"""Helpers for the GPU tests: move a workload to the device, run the library
through its C ABI, and compare against the oracle."""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

import segmented_gather_gemm_sgmv_amd as sg

from . import workloads as wl

# |gpu - oracle| <= TOL * (1 + |oracle|) per element (bf16 or fp32 storage,
# fp32 accumulation).
TOL = 1e-2


@dataclasses.dataclass
class DeviceCase:
    w: wl.Workload
    X: torch.Tensor
    Y0: torch.Tensor
    A_pool: torch.Tensor
    B_pool: torch.Tensor
    A_ptrs: torch.Tensor
    B_ptrs: torch.Tensor
    seg_start: torch.Tensor
    seg_adapter: torch.Tensor


def to_device(w: wl.Workload, dev, A_pool=None, B_pool=None) -> DeviceCase:
    A = A_pool if A_pool is not None else w.A_pool.to(dev)
    B = B_pool if B_pool is not None else w.B_pool.to(dev)
    return DeviceCase(
        w=w, X=w.X.to(dev).contiguous(), Y0=w.Y.to(dev).contiguous(), A_pool=A, B_pool=B,
        A_ptrs=sg.sgmv_pool_pointers(A), B_ptrs=sg.sgmv_pool_pointers(B),
        seg_start=torch.from_numpy(np.ascontiguousarray(w.seg_start, np.int32)).to(dev),
        seg_adapter=torch.from_numpy(np.ascontiguousarray(w.seg_adapter, np.int32)).to(dev))


def run_split(c: DeviceCase, Y=None, workspace=None):
    V = torch.zeros((c.w.M, c.w.r), dtype=torch.float32, device=c.X.device)
    Y = c.Y0.clone() if Y is None else Y
    sg.sgmv_shrink(V, c.X, c.A_ptrs, c.seg_start, c.seg_adapter, c.w.r, workspace_buf=workspace)
    sg.sgmv_expand(Y, V, c.B_ptrs, c.seg_start, c.seg_adapter, c.w.r, c.w.alpha)
    torch.cuda.synchronize()
    return V, Y


def run_fused(c: DeviceCase, Y=None, workspace=None):
    Y = c.Y0.clone() if Y is None else Y
    sg.sgmv_fused(Y, c.X, c.A_ptrs, c.B_ptrs, c.seg_start, c.seg_adapter, c.w.r, c.w.alpha,
                  workspace_buf=workspace)
    torch.cuda.synchronize()
    return Y


def oracle_run(orc, w: wl.Workload):
    V = orc.shrink(wl.storage(w.X), wl.storage(w.A_pool), w.seg_start, w.seg_adapter)
    Y = orc.expand(wl.storage(w.Y), V, wl.storage(w.B_pool), w.seg_start, w.seg_adapter, w.alpha)
    return V, Y


def compact_rows(w: wl.Workload, c: DeviceCase) -> wl.Workload:
    """w with its pools cut down to the slots its segments name, copied back
    from the device (each segment then names its own slot): the oracle's
    input for pools too large to hold on the host. Every row is kept."""
    ids = np.asarray(w.seg_adapter, np.int64)
    idx = torch.from_numpy(ids).to(c.A_pool.device)
    return wl.Workload(w.name, w.M, w.d_in, w.d_out, w.r, w.alpha, w.dtype, len(ids), w.seg_start,
                       np.arange(len(ids), dtype=np.int32), X=w.X, Y=w.Y,
                       A_pool=c.A_pool[idx].cpu(), B_pool=c.B_pool[idx].cpu())


def max_rel_err(gpu: torch.Tensor, ref: np.ndarray) -> float:
    g = gpu.detach().cpu().to(torch.float64).numpy()
    err = np.abs(g - ref) / (1.0 + np.abs(ref))
    return float(err.max(initial=0.0))


def assert_close(gpu: torch.Tensor, ref: np.ndarray, tol: float = TOL, what: str = ""):
    e = max_rel_err(gpu, ref)
    assert np.isfinite(e) and e <= tol, f"{what}: max rel err {e:.3e} > {tol:.1e}"
    return e


def bits(t: torch.Tensor) -> np.ndarray:
    return wl.storage(t.detach().cpu())


def oracle_bits(orc, y: np.ndarray, dtype: torch.dtype) -> np.ndarray:
    return orc.round_bf16(y) if dtype == torch.bfloat16 else orc.round_f32(y)


# -- the batch in token order (gathered calls) --------------------------------
def rows_tensor(rows, dev) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(rows, np.int32)).to(dev)


def run_split_gather(c: DeviceCase, rows: torch.Tensor, Y=None, workspace=None):
    V = torch.zeros((c.w.M, c.w.r), dtype=torch.float32, device=c.X.device)
    Y = c.Y0.clone() if Y is None else Y
    sg.sgmv_shrink_gather(V, c.X, rows, c.A_ptrs, c.seg_start, c.seg_adapter, c.w.r,
                          workspace_buf=workspace)
    sg.sgmv_expand_scatter(Y, V, rows, c.B_ptrs, c.seg_start, c.seg_adapter, c.w.r, c.w.alpha)
    torch.cuda.synchronize()
    return V, Y


def run_fused_gather(c: DeviceCase, rows: torch.Tensor, Y=None, workspace=None):
    Y = c.Y0.clone() if Y is None else Y
    sg.sgmv_fused_gather(Y, c.X, rows, c.A_ptrs, c.B_ptrs, c.seg_start, c.seg_adapter, c.w.r, c.w.alpha,
                         workspace_buf=workspace)
    torch.cuda.synchronize()
    return Y


def oracle_run_gather(orc, w: wl.Workload, rows):
    """The oracle on a batch whose X and Y are in token order: segment row p
    is token rows[p]. Returns V (segment order) and Y (token order)."""
    V = orc.shrink_gather(wl.storage(w.X), wl.storage(w.A_pool), w.seg_start, w.seg_adapter, rows)
    Y = orc.expand_scatter(wl.storage(w.Y), V, wl.storage(w.B_pool), w.seg_start, w.seg_adapter, rows,
                           w.alpha)
    return V, Y
