"""bench.py's host logic on the CPU: the algorithmic bytes it prices each
kernel at, the committed-profile traffic lookup (gated by the kernel
sources' hash), and the token-order index of the gathered paths."""
import json
import re
from pathlib import Path

import numpy as np
import pytest

import bench
import oracle as oracle_pkg

from . import workloads as wl


def test_kernel_bytes_match_the_algorithmic_bytes():
    w = wl.decode_skewed(oracle_pkg.build_segments)
    total = w.algorithmic_bytes()
    v = 4 * w.M * w.r
    for path in ("fused", "fused_gather", "fused_permute", "fused_layer"):
        assert sum(bench.kernel_bytes(w, path).values()) == total
    for path in ("split", "split_gather"):
        kb = bench.kernel_bytes(w, path)
        assert sum(kb.values()) == total + 2 * v   # V written by the shrink, read by the expand
        assert list(kb) == bench.KERNELS[path]
    assert bench.kernel_bytes(w, "per_segment")["fused"] == pytest.approx(total / w.num_segments)
    # the headline workload: 18,350,080 bytes (X, 64 adapters' A and B, Y read and written)
    assert wl.decode_distinct(pool=False).algorithmic_bytes() == 18_350_080


def test_profiled_traffic_is_gated_by_the_sources_hash(monkeypatch):
    f = Path(bench.ROOT) / "profiles" / "fused_decode_distinct.md"
    rec = json.loads(re.search(r"<!-- bench-traffic (\{.*\}) -->", f.read_text()).group(1))
    monkeypatch.setattr(bench, "sources_sha256", lambda: rec["sources_sha256"])
    got = bench.profiled_traffic("decode_distinct", "fused", "fused")
    assert got == rec["kernels"]["fused"]["traffic_bytes"]
    k = rec["kernels"]["fused"]
    scaled = (k["fetch_kib_raw"] * rec["fetch_scale"] + k["write_kib_raw"] * rec["write_scale"]) * 1024
    assert got == pytest.approx(scaled)
    monkeypatch.setattr(bench, "sources_sha256", lambda: "0" * 64)
    assert bench.profiled_traffic("decode_distinct", "fused", "fused") is None
    assert bench.profiled_traffic("decode_distinct", "fused_permute", "fused") is None


def test_token_rows():
    w = wl.decode_skewed(oracle_pkg.build_segments)
    perm, _, _ = oracle_pkg.build_segments(w.token_adapter)
    assert np.array_equal(bench.token_rows(w), perm)
    w2 = wl.tiny()
    rows = bench.token_rows(w2)
    assert sorted(rows.tolist()) == list(range(w2.M))
