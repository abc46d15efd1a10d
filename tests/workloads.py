"""Seeded synthetic SGMV workloads, shared by the tests, the smoke check and
the benchmark.

This module only draws inputs. It holds none of the method's arithmetic: no
product, no sum over adapters and no output. Both the HIP path and the oracle
receive exactly the arrays built here.

Recipe (all values seeded; numpy PCG64 unless noted):

* X ~ N(0, 1), A ~ N(0, 1/d_in), B ~ N(0, 1/r) (the second parameter is the
  variance), drawn in fp32 and rounded to bf16 (nearest-even, by torch's
  conversion) when the workload is bf16. Y starts at zero.
* A pool slot holds A_k as r rows of d_in elements and B_k as r rows of d_out
  elements; a pool is a P x r x d array, one slot per adapter.
* Segment structure per workload follows the five shapes of the Punica
  evaluation stand-ins: tiny (4 segments), decode with distinct adapters (one
  row per segment), decode with Zipf(1.5)-skewed adapters sorted into
  segments, prefill (8 segments of 128..1024 rows) and a 70B-layer slice
  (7 projections, 512 rows, 512 distinct adapters out of 2000).

The Zipf draw is the truncated law P(k) proportional to k^-1.5 over
k = 1..P, mapped to adapter id k-1.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np
import torch

SEED_BASE = 1000


@dataclasses.dataclass
class Workload:
    name: str
    M: int
    d_in: int
    d_out: int
    r: int
    alpha: float
    dtype: torch.dtype               # torch.float32 or torch.bfloat16
    num_adapters: int
    seg_start: np.ndarray            # int32 [N+1]
    seg_adapter: np.ndarray          # int32 [N]
    X: Optional[torch.Tensor] = None        # CPU [M, d_in]
    Y: Optional[torch.Tensor] = None        # CPU [M, d_out] (initial value)
    A_pool: Optional[torch.Tensor] = None   # CPU [P, r, d_in]
    B_pool: Optional[torch.Tensor] = None   # CPU [P, r, d_out]
    token_adapter: Optional[np.ndarray] = None  # unsorted per-token ids, when the batch was sorted
    seed: int = 0

    @property
    def num_segments(self) -> int:
        return int(self.seg_adapter.shape[0])

    def algorithmic_bytes(self) -> int:
        """Bytes the method must move: X once, each segment's adapter once,
        Y read and written once."""
        e = 4 if self.dtype == torch.float32 else 2
        per_adapter = self.d_in * self.r + self.r * self.d_out
        return e * (self.M * self.d_in + self.num_segments * per_adapter + 2 * self.M * self.d_out)

    def flops(self) -> int:
        return 2 * self.M * self.r * (self.d_in + self.d_out)


def _normal(rng: np.random.Generator, shape, std: float, dtype: torch.dtype) -> torch.Tensor:
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    t = torch.from_numpy(a)
    return t if dtype == torch.float32 else t.to(dtype)


def segments_from_lengths(lengths) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(np.asarray(lengths, dtype=np.int64))]).astype(np.int32)


def zipf_ids(rng: np.random.Generator, n: int, num_adapters: int, s: float = 1.5) -> np.ndarray:
    k = np.arange(1, num_adapters + 1, dtype=np.float64)
    p = k ** (-s)
    p /= p.sum()
    return rng.choice(num_adapters, size=n, p=p).astype(np.int32)


def fill_tensors(w: Workload, rng: np.random.Generator, pool: bool = True) -> Workload:
    w.X = _normal(rng, (w.M, w.d_in), 1.0, w.dtype)
    w.Y = torch.zeros((w.M, w.d_out), dtype=w.dtype)
    if pool:
        w.A_pool = _normal(rng, (w.num_adapters, w.r, w.d_in), w.d_in ** -0.5, w.dtype)
        w.B_pool = _normal(rng, (w.num_adapters, w.r, w.d_out), w.r ** -0.5, w.dtype)
    return w


def tiny(seed: int = SEED_BASE + 1) -> Workload:
    """d_in = d_out = 256, r = 8, alpha = 16, fp32, 8 tokens in 4 segments of
    lengths [1, 2, 1, 4] with adapters [2, 0, 3, 1] from a pool of 4."""
    rng = np.random.Generator(np.random.PCG64(seed))
    w = Workload("tiny", 8, 256, 256, 8, 16.0, torch.float32, 4,
                 segments_from_lengths([1, 2, 1, 4]), np.array([2, 0, 3, 1], np.int32), seed=seed)
    return fill_tensors(w, rng)


def decode_distinct(seed: int = SEED_BASE + 2, M: int = 64, d: int = 4096, r: int = 16,
                    num_adapters: int = 256, pool: bool = True) -> Workload:
    """4096 -> 4096, r = 16, alpha = 32, 64 tokens each in its own length-1
    segment, adapters drawn without replacement from a pool of 256, bf16."""
    rng = np.random.Generator(np.random.PCG64(seed))
    ids = rng.choice(num_adapters, size=M, replace=False).astype(np.int32)
    w = Workload("decode_distinct", M, d, d, r, 2.0 * r, torch.bfloat16, num_adapters,
                 segments_from_lengths([1] * M), ids, seed=seed)
    return fill_tensors(w, rng, pool)


def decode_skewed(builder, seed: int = SEED_BASE + 3, M: int = 256, d_in: int = 4096,
                  d_out: int = 11008, r: int = 16, num_adapters: int = 64) -> Workload:
    """256 tokens, adapters ~ Zipf(1.5) over a pool of 64, sorted into
    contiguous segments; 4096 -> 11008, r = 16, alpha = 32, bf16.

    ``builder(token_adapter) -> (perm, seg_start, seg_adapter)`` does the
    grouping (the library's metadata builder, or the oracle's). X is drawn
    for the rows in segment order, the order the kernels see."""
    rng = np.random.Generator(np.random.PCG64(seed))
    ids = zipf_ids(rng, M, num_adapters)
    _, starts, sids = builder(ids)
    w = Workload("decode_skewed", M, d_in, d_out, r, 2.0 * r, torch.bfloat16, num_adapters,
                 np.asarray(starts, np.int32), np.asarray(sids, np.int32), token_adapter=ids,
                 seed=seed)
    return fill_tensors(w, rng)


def prefill(seed: int = SEED_BASE + 4, num_requests: int = 8, lo: int = 128, hi: int = 1024,
            d: int = 4096, r: int = 64, num_adapters: int = 32) -> Workload:
    """8 requests with lengths ~ U{128..1024}, each its own distinct adapter
    from a pool of 32; 4096 -> 4096, r = 64, alpha = 128, bf16."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lengths = rng.integers(lo, hi, size=num_requests, endpoint=True)
    ids = rng.choice(num_adapters, size=num_requests, replace=False).astype(np.int32)
    starts = segments_from_lengths(lengths)
    w = Workload("prefill", int(starts[-1]), d, d, r, 2.0 * r, torch.bfloat16, num_adapters,
                 starts, ids, seed=seed)
    return fill_tensors(w, rng)


# The seven projections of one 70B decoder layer: (name, d_in, d_out).
LLAMA70B_PROJECTIONS = [
    ("q", 8192, 8192), ("k", 8192, 1024), ("v", 8192, 1024), ("o", 8192, 8192),
    ("gate", 8192, 28672), ("up", 8192, 28672), ("down", 28672, 8192),
]


def slice70b(seed: int = SEED_BASE + 5, M: int = 512, num_adapters: int = 2000, r: int = 16,
             projections=None) -> List[Workload]:
    """512 decode tokens, each a distinct adapter from a pool of 2000, run
    through the 7 projections of a 70B layer; r = 16, alpha = 32, bf16.

    The adapter ids are shared by all projections; each projection has its
    own X and pool. Pools are NOT filled here (10.35 GB in total): use
    :func:`device_pool` on the GPU, and copy the touched slots back for the
    oracle."""
    rng = np.random.Generator(np.random.PCG64(seed))
    ids = rng.choice(num_adapters, size=M, replace=False).astype(np.int32)
    out = []
    for pi, (name, d_in, d_out) in enumerate(projections or LLAMA70B_PROJECTIONS):
        w = Workload(f"slice70b_{name}", M, d_in, d_out, r, 2.0 * r, torch.bfloat16, num_adapters,
                     segments_from_lengths([1] * M), ids.copy(), seed=seed * 100 + pi)
        prng = np.random.Generator(np.random.PCG64(w.seed))
        out.append(fill_tensors(w, prng, pool=False))
    return out


# The seven projections of one 7B decoder layer: (name, d_in, d_out).
LLAMA7B_PROJECTIONS = [
    ("q", 4096, 4096), ("k", 4096, 4096), ("v", 4096, 4096), ("o", 4096, 4096),
    ("gate", 4096, 11008), ("up", 4096, 11008), ("down", 11008, 4096),
]


def layer7b(seed: int = SEED_BASE + 6, M: int = 64, num_adapters: int = 256, r: int = 16) -> List[Workload]:
    """A whole 7B decoder layer at decode: 64 tokens, each a distinct adapter
    from a pool of 256, through the layer's 7 projections; r = 16, alpha = 32,
    bf16. Built like slice70b (pools not filled here)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    ids = rng.choice(num_adapters, size=M, replace=False).astype(np.int32)
    out = []
    for pi, (name, d_in, d_out) in enumerate(LLAMA7B_PROJECTIONS):
        w = Workload(f"layer7b_{name}", M, d_in, d_out, r, 2.0 * r, torch.bfloat16, num_adapters,
                     segments_from_lengths([1] * M), ids.copy(), seed=seed * 100 + pi)
        prng = np.random.Generator(np.random.PCG64(w.seed))
        out.append(fill_tensors(w, prng, pool=False))
    return out


def device_int_pool(num_adapters: int, r: int, d: int, lo: int, hi: int, seed: int, device) -> torch.Tensor:
    """A P x r x d bf16 pool of integers in lo..hi drawn on the device with a
    seeded torch generator (integer_case's values for pools too large to
    draw on the host)."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    pool = torch.empty((num_adapters, r, d), dtype=torch.bfloat16, device=device)
    chunk = max(1, (1 << 28) // (r * d))
    for k0 in range(0, num_adapters, chunk):
        k1 = min(num_adapters, k0 + chunk)
        pool[k0:k1].copy_(torch.randint(lo, hi + 1, (k1 - k0, r, d), generator=g, device=device))
    return pool


def device_pool(num_adapters: int, r: int, d: int, std: float, seed: int, device) -> torch.Tensor:
    """A P x r x d bf16 pool drawn on the device with a seeded torch generator
    (for pools too large to draw on the host)."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    pool = torch.empty((num_adapters, r, d), dtype=torch.bfloat16, device=device)
    chunk = max(1, (1 << 28) // (r * d))
    for k0 in range(0, num_adapters, chunk):
        k1 = min(num_adapters, k0 + chunk)
        t = torch.randn((k1 - k0, r, d), generator=g, device=device, dtype=torch.float32)
        pool[k0:k1].copy_(t.mul_(std))
        del t
    return pool


def random_case(rng: np.random.Generator, dtype=torch.float32, max_M: int = 16, max_seg: int = 6,
                max_pool: int = 5, ranks=(8, 16), max_d: int = 64, allow_empty: bool = True) -> Workload:
    """A small random SGMV problem: ragged segments (empty ones allowed),
    random adapter ids with repeats, non-square shapes, nonzero Y."""
    r = int(rng.choice(ranks))
    d_in = 8 * int(rng.integers(1, max_d // 8 + 1))
    d_out = 8 * int(rng.integers(1, max_d // 8 + 1))
    P = int(rng.integers(1, max_pool + 1))
    N = int(rng.integers(1, max_seg + 1))
    lengths = rng.integers(0 if allow_empty else 1, max(2, max_M // N + 1), size=N)
    ids = rng.integers(0, P, size=N).astype(np.int32)
    w = Workload("random", int(lengths.sum()), d_in, d_out, r, float(rng.choice([8.0, 16.0, 32.0, 3.0])),
                 dtype, P, segments_from_lengths(lengths), ids)
    fill_tensors(w, rng)
    w.Y = _normal(rng, (w.M, w.d_out), 1.0, dtype)
    return w


def integer_case(rng: np.random.Generator, w: Workload) -> Workload:
    """Replace w's values by small integers, so every partial sum is an exact
    integer below 2^24: X in {-2..2}, A and B in {-1, 0, 1}, Y in {-8..8},
    alpha = 2r (scale 2)."""
    def ints(shape, lo, hi):
        return torch.from_numpy(rng.integers(lo, hi + 1, size=shape).astype(np.float32)).to(w.dtype)
    w.X = ints((w.M, w.d_in), -2, 2)
    w.A_pool = ints((w.num_adapters, w.r, w.d_in), -1, 1)
    w.B_pool = ints((w.num_adapters, w.r, w.d_out), -1, 1)
    w.Y = ints((w.M, w.d_out), -8, 8)
    w.alpha = 2.0 * w.r
    return w


def storage(t: torch.Tensor) -> np.ndarray:
    """A CPU tensor's elements as the oracle takes them: fp32 as float32,
    bf16 as its raw bit patterns (uint16)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.float32:
        return t.numpy()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    raise TypeError(t.dtype)


def to_float64(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().to(torch.float64).numpy()


ALL_CONFIGS: Dict[str, str] = {
    "tiny": "d_in=d_out=256, r=8, alpha=16, 8 tokens in 4 segments [1,2,1,4], adapters [2,0,3,1], pool 4, fp32",
    "decode_distinct": "d_in=d_out=4096, r=16, alpha=32, 64 tokens in 64 length-1 segments, distinct adapters from 256, bf16",
    "decode_skewed": "d_in=4096, d_out=11008, r=16, alpha=32, 256 tokens, Zipf(1.5) over 64 adapters, sorted, bf16",
    "prefill": "d_in=d_out=4096, r=64, alpha=128, 8 segments of U{128..1024} rows, distinct adapters from 32, bf16",
    "slice70b": "7 projections of a 70B layer, 512 tokens, distinct adapters from 2000, r=16, alpha=32, bf16",
    "layer7b": "7 projections of a 7B layer (q/k/v/o 4096->4096, gate/up 4096->11008, down 11008->4096), "
               "64 decode tokens, distinct adapters from 256, r=16, alpha=32, bf16",
}
