"""SGMV benchmark on one MI355X: the fused shrink+expand kernel per call (or,
with --path split, the shrink and expand kernels back to back), through the C
ABI, on seeded synthetic batches resident in HBM.

Default workload: decode with distinct adapters (d_in = d_out = 4096,
r = 16, alpha = 32, 64 tokens in 64 length-1 segments, adapters drawn without
replacement from a pool of 256, bf16). One step is one call of the hot path
over one batch. To keep the 256 MB Infinity Cache from serving the weights,
the steps rotate over R replicas of the pools and activations (each its own
HBM region), so a replica's bytes are cold when it comes round again.

Paths: fused (one launch) and split (shrink, then expand) take the batch in
segment order; fused_gather and split_gather take it in token order with a
row index (for decode_skewed the grouping's own permutation, for the other
workloads a seeded shuffle); fused_permute is the comparison for those: torch
row gathers of X and Y into segment order around the contiguous fused call,
and a torch scatter of Y back. fused_layer runs all projections of a step
(the 70B slice's seven) in one launch. per_segment is the schedule SGMV
replaces: one fused launch per segment (each on its own rows and adapter),
so a step costs one launch per segment instead of one in all.

Prints ONE JSON line: value = algorithmic HBM GB/s (X read once, each
segment's adapter read once, Y read and written once) over the timed steps,
plus a roofline object for the dominant kernel and the CPU oracle's rate on
a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "SGMV shrink+expand µs/call and HBM GB/s (% peak), 4096-d r=16, 64 adapters"
HBM_PEAK_GBS = 8000.0   # MI355X published HBM3E bandwidth


def sources_sha256():
    """sha256 over the kernel sources, in name order (name, then bytes)."""
    import hashlib
    from pathlib import Path
    h = hashlib.sha256()
    for f in sorted((Path(ROOT) / "segmented_gather_gemm_sgmv_amd" / "csrc").glob("*")):
        h.update(f.name.encode())
        h.update(f.read_bytes())
    return h.hexdigest()


def profiled_traffic(workload, path, kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary for this workload and path (FETCH_SIZE + WRITE_SIZE, each scaled
    by what it reads for a plain 256 MiB device copy), or None when there is
    no summary or the kernel sources have changed since it was taken."""
    import re
    from pathlib import Path
    prefix = {"fused": "fused", "split": "shrink_expand", "fused_gather": "fused_gather",
              "split_gather": "shrink_expand_gather", "fused_layer": "fused_layer"}.get(path)
    if prefix is None:
        return None
    name = f"{prefix}_{workload}.md"
    f = Path(ROOT) / "profiles" / name
    if not f.exists():
        return None
    m = re.search(r"<!-- bench-traffic (\{.*\}) -->", f.read_text())
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("sources_sha256") != sources_sha256():
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if k is None else k["traffic_bytes"]


def profiled_mfma(workload):
    """Per-kernel MfmaUtil (percent) from the committed rocprofv3 counter
    summary for this workload (profiles/mfma_<workload>.md), or None when
    there is none or the kernel sources have changed since it was taken."""
    import re
    from pathlib import Path
    f = Path(ROOT) / "profiles" / f"mfma_{workload}.md"
    if not f.exists():
        return None
    m = re.search(r"<!-- bench-mfma (\{.*\}) -->", f.read_text())
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("sources_sha256") != sources_sha256():
        return None
    return rec.get("kernels")


def cpu_model():
    """The host CPU's model name (/proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=2000)
    p.add_argument("--warmup", type=int, default=200)
    p.add_argument("--workload", default="decode_distinct",
                   choices=["tiny", "decode_distinct", "decode_skewed", "prefill", "slice70b", "layer7b"])
    p.add_argument("--path", default="fused",
                   choices=["split", "fused", "split_gather", "fused_gather", "fused_permute", "fused_layer",
                            "per_segment"])
    p.add_argument("--replicas", type=int, default=0, help="0 = enough to exceed 1 GiB of touched bytes")
    p.add_argument("--cpu-seconds", type=float, default=8.0, help="per CPU-baseline leg (1 core, all cores)")
    p.add_argument("--no-all-configs", action="store_true",
                   help="skip the other workloads' summary (all_configs) in the default run")
    p.add_argument("--config-steps", type=int, default=400, help="timed steps per path in all_configs")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cold-calls", type=int, default=50,
                   help="calls timed one by one after writing 1 GiB, which evicts L2 and the Infinity Cache (0: skip)")
    p.add_argument("--no-hbm-probe", action="store_true",
                   help="skip the streaming-read probe of what a plain kernel reaches")
    p.add_argument("--admission", action="store_true",
                   help="also time adapter admission from pinned host memory (7B and 70B adapters)")
    p.add_argument("--copy-probe-mib", type=int, default=0,
                   help="also run one plain device copy of this size (for counter scaling)")
    return p.parse_args()


class Replica:
    """One HBM-resident copy of a workload's inputs (device tensors)."""

    def __init__(self, w, dev, A_pool, B_pool, X, Y):
        import torch
        import segmented_gather_gemm_sgmv_amd as sg
        self.w = w
        self.X, self.Y = X, Y
        # the pools must outlive the device tables that point into them
        self.A_pool, self.B_pool = A_pool, B_pool
        self.A_ptrs = sg.sgmv_pool_pointers(A_pool)
        self.B_ptrs = sg.sgmv_pool_pointers(B_pool)
        self.seg_start = torch.from_numpy(np.ascontiguousarray(w.seg_start, np.int32)).to(dev)
        self.seg_adapter = torch.from_numpy(np.ascontiguousarray(w.seg_adapter, np.int32)).to(dev)
        self.V = torch.zeros((w.M, w.r), dtype=torch.float32, device=dev)
        rows = token_rows(w)
        self.rows = torch.from_numpy(rows).to(dev)                    # int32, for the gathered calls
        self.rows64 = torch.from_numpy(rows.astype(np.int64)).to(dev)  # for torch's row permutes
        self.Xs = torch.empty_like(X)   # segment-order copies (fused_permute)
        self.Ys = torch.empty_like(Y)
        self._segments = None

    @property
    def segments(self):
        """per_segment: each segment as a batch of its own (rows a..b-1,
        offsets [0, b - a], its adapter), built on first use."""
        import torch
        if self._segments is None:
            w = self.w
            self._segments = []
            for s in range(w.num_segments):
                a, b = int(w.seg_start[s]), int(w.seg_start[s + 1])
                if b > a:
                    meta = torch.tensor([0, b - a, int(w.seg_adapter[s])], dtype=torch.int32, device=self.X.device)
                    self._segments.append((a, b, meta[:2], meta[2:]))
        return self._segments


def token_rows(w):
    """Token row of each segment row: decode_skewed keeps its draw's arrival
    order (the grouping's permutation); other workloads get a seeded
    shuffle."""
    if w.token_adapter is not None:
        order = np.argsort(np.asarray(w.token_adapter, np.int64), kind="stable")
        return order.astype(np.int32)
    return np.random.Generator(np.random.PCG64(90)).permutation(w.M).astype(np.int32)


def make_workloads(name):
    from tests import workloads as wl
    import segmented_gather_gemm_sgmv_amd as sg
    if name == "tiny":
        return [wl.tiny()]
    if name == "decode_distinct":
        return [wl.decode_distinct(pool=False)]
    if name == "decode_skewed":
        return [wl.decode_skewed(sg.sgmv_build_segments)]
    if name == "prefill":
        return [wl.prefill()]
    if name == "layer7b":
        return wl.layer7b()
    return wl.slice70b()


def build_replicas(ws, dev, R):
    """R replicas of every projection's inputs. Pools are drawn on the device
    (seeded); X is the workload's own seeded draw."""
    import torch
    from tests import workloads as wl
    reps = []
    for q in range(R):
        group = []
        for w in ws:
            A = wl.device_pool(w.num_adapters, w.r, w.d_in, w.d_in ** -0.5, w.seed * 7 + 2 * q + 1, dev)
            B = wl.device_pool(w.num_adapters, w.r, w.d_out, w.r ** -0.5, w.seed * 7 + 2 * q + 2, dev)
            if w.dtype == torch.float32:
                A, B = A.float(), B.float()
            X = w.X.to(dev)
            Y = w.Y.to(dev)
            group.append(Replica(w, dev, A, B, X, Y))
        reps.append(group)
    return reps


def layer_call(group, ws=None):
    import segmented_gather_gemm_sgmv_amd as sg
    rp0 = group[0]
    sg.sgmv_fused_layer([(rp.Y, rp.X, rp.A_ptrs, rp.B_ptrs) for rp in group], rp0.seg_start, rp0.seg_adapter,
                        rp0.w.r, rp0.w.alpha, workspace_buf=ws)


def step(group, path, ws=None):
    import torch
    import segmented_gather_gemm_sgmv_amd as sg
    if path == "fused_layer":
        layer_call(group, ws)
        return
    if path == "per_segment":
        for rp in group:
            for a, b, ss, sa in rp.segments:
                sg.sgmv_fused(rp.Y[a:b], rp.X[a:b], rp.A_ptrs, rp.B_ptrs, ss, sa, rp.w.r, rp.w.alpha,
                              workspace_buf=ws)
        return
    for rp in group:
        w = rp.w
        if path == "fused":
            sg.sgmv_fused(rp.Y, rp.X, rp.A_ptrs, rp.B_ptrs, rp.seg_start, rp.seg_adapter, w.r, w.alpha,
                          workspace_buf=ws)
        elif path == "split":
            sg.sgmv_shrink(rp.V, rp.X, rp.A_ptrs, rp.seg_start, rp.seg_adapter, w.r, workspace_buf=ws)
            sg.sgmv_expand(rp.Y, rp.V, rp.B_ptrs, rp.seg_start, rp.seg_adapter, w.r, w.alpha)
        elif path == "fused_gather":
            sg.sgmv_fused_gather(rp.Y, rp.X, rp.rows, rp.A_ptrs, rp.B_ptrs, rp.seg_start, rp.seg_adapter,
                                 w.r, w.alpha, workspace_buf=ws)
        elif path == "split_gather":
            sg.sgmv_shrink_gather(rp.V, rp.X, rp.rows, rp.A_ptrs, rp.seg_start, rp.seg_adapter, w.r,
                                  workspace_buf=ws)
            sg.sgmv_expand_scatter(rp.Y, rp.V, rp.rows, rp.B_ptrs, rp.seg_start, rp.seg_adapter, w.r,
                                   w.alpha)
        else:  # fused_permute: the caller moves rows into segment order and back
            torch.index_select(rp.X, 0, rp.rows64, out=rp.Xs)
            torch.index_select(rp.Y, 0, rp.rows64, out=rp.Ys)
            sg.sgmv_fused(rp.Ys, rp.Xs, rp.A_ptrs, rp.B_ptrs, rp.seg_start, rp.seg_adapter, w.r, w.alpha,
                          workspace_buf=ws)
            rp.Y.index_copy_(0, rp.rows64, rp.Ys)


def capture(reps, path, first, count, ws):
    """A HIP graph of `count` consecutive steps starting at replica `first`:
    replaying it launches the kernels back to back with no host work."""
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(count):
            step(reps[(first + i) % len(reps)], path, ws)
    return g


KERNELS = {"fused": ["fused"], "split": ["shrink", "expand"], "fused_gather": ["fused_gather"],
           "split_gather": ["shrink_gather", "expand_scatter"], "fused_permute": ["fused"],
           "fused_layer": ["fused_layer"], "per_segment": ["fused"]}


def kernel_bytes(w, path):
    """Algorithmic bytes per launch of each kernel of the path (the row
    index, like the segment metadata, is a few KB and not counted)."""
    e = 4 if str(w.dtype).endswith("float32") else 2
    N = w.num_segments
    x = e * w.M * w.d_in
    a = e * N * w.r * w.d_in
    b = e * N * w.r * w.d_out
    y = 2 * e * w.M * w.d_out
    v = 4 * w.M * w.r
    if path == "per_segment":  # one launch per segment: the average launch's bytes
        return {"fused": (x + a + b + y) / max(1, N)}
    if path in ("fused", "fused_gather", "fused_permute", "fused_layer"):
        return {KERNELS[path][0]: x + a + b + y}
    names = KERNELS[path]
    return {names[0]: x + a + v, names[1]: b + y + v}


def launch_kernel(rp, name, ws=None):
    import segmented_gather_gemm_sgmv_amd as sg
    w = rp.w
    if name == "fused":
        sg.sgmv_fused(rp.Y, rp.X, rp.A_ptrs, rp.B_ptrs, rp.seg_start, rp.seg_adapter, w.r, w.alpha,
                      workspace_buf=ws)
    elif name == "shrink":
        sg.sgmv_shrink(rp.V, rp.X, rp.A_ptrs, rp.seg_start, rp.seg_adapter, w.r, workspace_buf=ws)
    elif name == "expand":
        sg.sgmv_expand(rp.Y, rp.V, rp.B_ptrs, rp.seg_start, rp.seg_adapter, w.r, w.alpha)
    elif name == "fused_gather":
        sg.sgmv_fused_gather(rp.Y, rp.X, rp.rows, rp.A_ptrs, rp.B_ptrs, rp.seg_start, rp.seg_adapter,
                             w.r, w.alpha, workspace_buf=ws)
    elif name == "shrink_gather":
        sg.sgmv_shrink_gather(rp.V, rp.X, rp.rows, rp.A_ptrs, rp.seg_start, rp.seg_adapter, w.r,
                              workspace_buf=ws)
    else:
        sg.sgmv_expand_scatter(rp.Y, rp.V, rp.rows, rp.B_ptrs, rp.seg_start, rp.seg_adapter, w.r, w.alpha)


def time_kernels(reps, path, steps, wsbuf):
    """Average duration of each kernel of the path: a HIP graph holding only
    that kernel, launched once per replica (and projection) in turn, replayed
    until `steps` launches were timed, bracketed by HIP events recorded on the
    replay stream."""
    import torch
    names = KERNELS[path]
    R = len(reps)
    out = {}
    for name in names:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for group in reps:
                if name == "fused_layer":
                    layer_call(group, wsbuf)
                    continue
                if path == "per_segment":
                    step(group, path, wsbuf)
                    continue
                for rp in group:
                    launch_kernel(rp, name, wsbuf)
        g.replay()
        torch.cuda.synchronize()
        n_replays = max(1, steps // R)
        stream = torch.cuda.current_stream()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(n_replays):
            g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        if name == "fused_layer":
            launches = n_replays * len(reps)
        elif path == "per_segment":
            launches = n_replays * sum(len(rp.segments) for gr in reps for rp in gr)
        else:
            launches = n_replays * sum(len(gr) for gr in reps)
        out[name] = a.elapsed_time(b) * 1e3 / launches   # microseconds per launch
        del g
    return out


def cold_calls(reps, path, wsbuf, n):
    """Each step timed on its own, right after a 1 GiB write that evicts the
    L2s and the 256 MB Infinity Cache: HIP events bracket the step alone, on
    the stream it runs on (the host enqueues the step while the write runs,
    so the events see no launch gap). Median, p10 and p90 in microseconds."""
    import torch
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=reps[0][0].X.device)
    stream = torch.cuda.current_stream()
    pairs = []
    for i in range(n):
        flush.fill_(i & 0xff)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        step(reps[i % len(reps)], path, wsbuf)
        b.record(stream)
        pairs.append((a, b))
    torch.cuda.synchronize()
    us = np.array([a.elapsed_time(b) * 1e3 for a, b in pairs])
    return {"calls": n, "median_us": float(np.median(us)), "p10_us": float(np.percentile(us, 10)),
            "p90_us": float(np.percentile(us, 90))}


def hbm_probe(dev, workload_bytes, full=True):
    """What a plain streaming-read kernel (the library's stream probe) reaches
    on this GPU: over 4 GiB, and over the workload's own byte count (windows
    rotated over 1 GiB, so the Infinity Cache cannot serve them), best of a
    few grid sizes, each from a replayed HIP graph timed with events."""
    import torch
    import segmented_gather_gemm_sgmv_amd as sg
    stream = torch.cuda.current_stream()

    def timed(launches, reps):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for src, n, sink in launches:
                sg.sgmv_stream_probe(src, sink, n)
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / (reps * len(launches))   # us per launch

    out = {}
    if full:
        big = torch.empty(4 << 30, dtype=torch.uint8, device=dev)
        best = None
        for blocks in (256, 512, 1024, 2048, 4096):
            sink = torch.empty(blocks, dtype=torch.int32, device=dev)
            us = timed([(big, big.numel(), sink)], 5)
            best = us if best is None or us < best else best
        out["GB_per_s_4GiB"] = big.numel() / (best * 1e-6) / 1e9
        del big
    n = (workload_bytes + 15) // 16 * 16
    windows = max(1, (1 << 30) // n)
    buf = torch.empty(windows * n, dtype=torch.uint8, device=dev)
    best, best_blocks = None, None
    for blocks in (256, 512, 1024, 2048):
        sink = torch.empty(blocks, dtype=torch.int32, device=dev)
        us = timed([(buf[i * n:(i + 1) * n], n, sink) for i in range(windows)], 20)
        if best is None or us < best:
            best, best_blocks = us, blocks
    out.update({"bytes_at_workload_size": n, "us_at_workload_size": best, "blocks": best_blocks,
                "GB_per_s_at_workload_size": n / (best * 1e-6) / 1e9})
    del buf
    return out


def admission_times(dev, reps=40):
    """sgmv_admit_adapter from pinned host memory: one adapter of each shape
    (every projection of a 7B and of a 70B layer, r = 16, bf16), copied into
    a spare device slot and pointed at by a table entry; `reps` admissions per
    shape, bracketed by HIP events on the stream they are enqueued on."""
    import torch
    import segmented_gather_gemm_sgmv_amd as sg
    from tests import workloads as wl
    out = {}
    for layer, projs in (("7b", wl.LLAMA7B_PROJECTIONS), ("70b", wl.LLAMA70B_PROJECTIONS)):
        r = 16
        slots, hosts, tables = [], [], []
        nbytes = 0
        for _, d_in, d_out in projs:
            A = torch.empty((r, d_in), dtype=torch.bfloat16, device=dev)
            B = torch.empty((r, d_out), dtype=torch.bfloat16, device=dev)
            Ah = torch.empty((r, d_in), dtype=torch.bfloat16, pin_memory=True).normal_()
            Bh = torch.empty((r, d_out), dtype=torch.bfloat16, pin_memory=True).normal_()
            slots.append((A, B))
            hosts.append((Ah, Bh))
            tables.append((torch.zeros(4, dtype=torch.int64, device=dev), torch.zeros(4, dtype=torch.int64, device=dev)))
            nbytes += 2 * r * (d_in + d_out)
        def admit_all():
            for (A, B), (Ah, Bh), (ta, tb) in zip(slots, hosts, tables):
                sg.sgmv_admit_adapter(A, B, Ah, Bh, ta, tb, 1)
        admit_all()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            admit_all()
        b.record(stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / reps
        out[f"layer{layer}_adapter"] = {"projections": len(projs), "bytes": nbytes, "ms": ms,
                                        "GB_per_s": nbytes / (ms * 1e-3) / 1e9}
        del slots, hosts, tables
    # a whole 7B adapter (32 layers x 7 projections, r = 16) held as one slab
    # pair (all A matrices, all B matrices), admitted with one call
    r, layers = 16, 32
    a_elems = layers * r * sum(d_in for _, d_in, _ in wl.LLAMA7B_PROJECTIONS)
    b_elems = layers * r * sum(d_out for _, _, d_out in wl.LLAMA7B_PROJECTIONS)
    A = torch.empty(a_elems, dtype=torch.bfloat16, device=dev)
    B = torch.empty(b_elems, dtype=torch.bfloat16, device=dev)
    Ah = torch.empty(a_elems, dtype=torch.bfloat16, pin_memory=True).normal_()
    Bh = torch.empty(b_elems, dtype=torch.bfloat16, pin_memory=True).normal_()
    ta, tb = torch.zeros(4, dtype=torch.int64, device=dev), torch.zeros(4, dtype=torch.int64, device=dev)
    sg.sgmv_admit_adapter(A, B, Ah, Bh, ta, tb, 1)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = 10
    a.record(stream)
    for _ in range(n):
        sg.sgmv_admit_adapter(A, B, Ah, Bh, ta, tb, 1)
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / n
    nbytes = 2 * (a_elems + b_elems)
    out["whole7b_adapter_one_slab"] = {"layers": layers, "bytes": nbytes, "ms": ms,
                                       "GB_per_s": nbytes / (ms * 1e-3) / 1e9}
    return out


def cpu_baseline(ws, seconds):
    """The oracle (C, fp64 arithmetic), as it stands, on a bounded sample of
    the same workload: whole batches of the first projection, repeated for
    about `seconds`, once on one core (this thread pinned to one CPU, one
    OpenMP thread) and once on all cores (the OpenMP default). Affinity and
    thread count are restored afterwards."""
    import oracle
    from tests import workloads as wl
    orc = oracle.get()
    w = ws[0]
    rng = np.random.Generator(np.random.PCG64(99))
    if w.A_pool is None:
        # only the touched slots matter to the oracle: draw those, remap ids
        N = w.num_segments
        A = wl._normal(rng, (N, w.r, w.d_in), w.d_in ** -0.5, w.dtype)
        B = wl._normal(rng, (N, w.r, w.d_out), w.r ** -0.5, w.dtype)
        seg_adapter = np.arange(N, dtype=np.int32)
    else:
        A, B, seg_adapter = w.A_pool, w.B_pool, w.seg_adapter
    args = (wl.storage(w.Y), wl.storage(w.X), wl.storage(A), wl.storage(B), w.seg_start, seg_adapter, w.alpha)
    nbytes = w.algorithmic_bytes()

    def leg():
        orc.sgmv(*args)  # warm
        reps = 0
        t0 = time.perf_counter()
        while True:
            orc.sgmv(*args)
            reps += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
        per_call = el / reps
        return {"value": nbytes / per_call / 1e9, "unit": "GB/s", "cores": oracle.threads_used(),
                "us_per_call": per_call * 1e6, "calls": reps, "seconds": el}

    all_cores = leg()
    mask = os.sched_getaffinity(0)
    old_threads = oracle.set_threads(1)
    try:
        os.sched_setaffinity(0, {min(mask)})
        one_core = leg()
    finally:
        os.sched_setaffinity(0, mask)
        oracle.set_threads(old_threads)
    return {"value": all_cores["value"], "unit": "GB/s", "cores": all_cores["cores"], "kind": "oracle",
            "precision": "fp64 (C loops, inputs widened exactly)", "cpu_model": cpu_model(),
            "us_per_call": all_cores["us_per_call"],
            "sample": f"whole {w.name} batches ({w.M} rows, {w.num_segments} segments, {nbytes} algorithmic "
                      f"bytes each): {all_cores['calls']} calls in {all_cores['seconds']:.1f} s on "
                      f"{all_cores['cores']} threads, {one_core['calls']} calls in {one_core['seconds']:.1f} s "
                      f"on one core",
            "all_cores": all_cores, "one_core": one_core}


def workspace_for(ws, group, path, dev):
    """One zero-filled workspace that serves every call of the path (calls
    run in order on one stream and each leaves it zero)."""
    import torch
    import segmented_gather_gemm_sgmv_amd as sg
    need = max(sg.sgmv_workspace_bytes(w.num_segments, w.M, w.d_in, w.d_out, w.r, w.dtype) for w in ws)
    if path == "fused_layer":
        need = sg.sgmv_layer_workspace_bytes([(rp.Y, rp.X, rp.A_ptrs, rp.B_ptrs) for rp in group],
                                             ws[0].num_segments, ws[0].M, ws[0].r, ws[0].dtype)
    return torch.zeros(max(need, 256), dtype=torch.uint8, device=dev)


def timed_steps(reps, path, steps, warmup, wsbuf):
    """Milliseconds per step: `warmup` untimed steps, then exactly `steps`
    steps replayed from HIP graphs (one graph over all replicas, plus one for
    the remainder), bracketed by events on the replay stream."""
    import torch
    R = len(reps)
    for i in range(warmup):
        step(reps[i % R], path, wsbuf)
    torch.cuda.synchronize()
    full = capture(reps, path, 0, R, wsbuf) if steps >= R else None
    rem = steps % R if steps >= R else steps
    tail = capture(reps, path, 0, rem, wsbuf) if rem else None
    if full is not None:
        full.replay()  # untimed replay: page in the graph
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps // R if full is not None else 0):
        full.replay()
    if tail is not None:
        tail.replay()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def launch_bytes(ws, path):
    """Algorithmic bytes per launch of each kernel of the path, averaged over
    the projections as the kernel timings average launches."""
    if path == "fused_layer":  # one launch covers every projection
        return {"fused_layer": sum(w.algorithmic_bytes() for w in ws)}
    per_kernel = kernel_bytes(ws[0], path)
    if len(ws) > 1:
        for w in ws[1:]:
            for n, b in kernel_bytes(w, path).items():
                per_kernel[n] += b
        per_kernel = {n: b / len(ws) for n, b in per_kernel.items()}
    return per_kernel


def config_summary(name, dev, steps, cold_n):
    """One workload in brief, for the all_configs object: per path, the step
    time, the rate and its fraction of the 8 TB/s peak, each kernel's
    average duration and fraction, the HBM traffic over algorithmic bytes
    from the committed counter summaries (None when stale), and the cold
    median; then the rate over what a plain streaming read reaches at the
    same byte count. Prefill adds its matrix-core figures."""
    import torch
    ws = make_workloads(name)
    nbytes = sum(w.algorithmic_bytes() for w in ws)
    R = max(1, min(256, -(-(1 << 30) // nbytes)))
    reps = build_replicas(ws, dev, R)
    out = {"algorithmic_bytes_per_step": nbytes, "projections": len(ws), "replicas": R,
           "tokens": ws[0].M, "segments": ws[0].num_segments, "r": ws[0].r}
    paths = ["fused", "split"] + (["fused_layer"] if len(ws) > 1 else [])
    for path in paths:
        wsbuf = workspace_for(ws, reps[0], path, dev)
        ms = timed_steps(reps, path, steps, max(10, steps // 10), wsbuf)
        kus = time_kernels(reps, path, steps, wsbuf)
        kb = launch_bytes(ws, path)
        rate = nbytes / (ms * 1e-3) / 1e9
        rec = {"us_per_step": ms * 1e3, "GB_per_s": rate, "frac_of_peak": rate / HBM_PEAK_GBS,
               "kernels_us": kus,
               "kernel_frac_of_peak": {k: kb[k] / (kus[k] * 1e-6) / 1e9 / HBM_PEAK_GBS for k in kus},
               "traffic_over_algorithmic": {}}
        for k in kus:
            t = profiled_traffic(name, path, k)
            rec["traffic_over_algorithmic"][k] = None if t is None else t / kb[k]
        if cold_n > 0:
            rec["cold_median_us"] = cold_calls(reps, path, wsbuf, cold_n)["median_us"]
        out[path] = rec
        del wsbuf
    probe = hbm_probe(dev, nbytes, full=False)
    out["probe_GB_per_s_at_workload_size"] = probe["GB_per_s_at_workload_size"]
    out["value_over_probe"] = out["fused"]["GB_per_s"] / probe["GB_per_s_at_workload_size"]
    if name == "prefill":
        flops = sum(w.flops() for w in ws)
        us = out["fused"]["kernels_us"]["fused"]
        out["mfma"] = {"algorithmic_TFLOP_per_s": flops / (us * 1e-6) / 1e12,
                       "frac_of_2500_TFLOP_per_s": flops / (us * 1e-6) / 1e12 / 2500.0,
                       "MfmaUtil_pct_profiled": profiled_mfma(name)}
    del reps
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1 "
                                   "(the multi-GPU split is described, not built)"}))
        sys.exit(2)
    import torch
    import segmented_gather_gemm_sgmv_amd as sg
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    ws = make_workloads(args.workload)
    touched = sum(w.algorithmic_bytes() for w in ws)
    R = args.replicas or max(1, min(256, -(-(1 << 30) // touched)))
    reps = build_replicas(ws, dev, R)
    if args.path == "per_segment":  # per-segment metadata is copied to the GPU before any capture
        for group in reps:
            for rp in group:
                rp.segments
    torch.cuda.synchronize()

    wsbuf = workspace_for(ws, reps[0], args.path, dev)
    ms = timed_steps(reps, args.path, args.steps, args.warmup, wsbuf)

    # per-kernel durations, for the roofline
    kus = time_kernels(reps, args.path, args.steps, wsbuf)
    per_kernel = launch_bytes(ws, args.path)
    dom = max(kus, key=kus.get)   # the kernel that takes the most time per step
    achieved = per_kernel[dom] / (kus[dom] * 1e-6) / 1e9

    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    nbytes = sum(w.algorithmic_bytes() for w in ws)
    flops = sum(w.flops() for w in ws)
    w0 = ws[0]
    value = nbytes / (ms * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "us_per_call": ms * 1e3,
        "tokens_per_s": w0.M / (ms * 1e-3),
        "hbm_frac": value / HBM_PEAK_GBS,
        "tflops": flops / (ms * 1e-3) / 1e12,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w0.dtype == torch.bfloat16 else "f32",
        "data": "synthetic",
        "config": {"workload": args.workload,
                   "path": {"split": "shrink+expand", "split_gather": "shrink_gather+expand_scatter"}.get(
                       args.path, args.path),
                   "d_in": w0.d_in, "d_out": w0.d_out, "r": w0.r, "alpha": w0.alpha, "tokens": w0.M,
                   "segments": w0.num_segments, "pool": w0.num_adapters, "projections": len(ws),
                   "replicas": R, "algorithmic_bytes_per_step": nbytes},
        "kernels_us": kus,
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": profiled_traffic(args.workload, args.path, dom),
                     "bytes_per_launch": per_kernel[dom], "us_per_launch": kus[dom]},
    }
    if args.cold_calls > 0:
        out["cold"] = cold_calls(reps, args.path, wsbuf, args.cold_calls)
    if not args.no_hbm_probe:
        probe = hbm_probe(dev, nbytes)
        probe["value_over_probe_at_workload_size"] = value / probe["GB_per_s_at_workload_size"]
        out["hbm_probe"] = probe
    if args.admission:
        out["admission"] = admission_times(dev)
    if args.workload == "decode_distinct" and args.path == "fused" and not args.no_all_configs:
        del reps, wsbuf
        torch.cuda.empty_cache()
        out["all_configs"] = {name: config_summary(name, dev, args.config_steps, 20 if args.cold_calls else 0)
                              for name in ("tiny", "decode_skewed", "prefill", "slice70b")}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(ws, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
