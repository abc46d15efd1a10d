"""Build libsgmv.so (the C-ABI library) in-tree with hipcc for gfx950.

Usage: ``python segmented_gather_gemm_sgmv_amd/build.py``.

The kernel file is compiled once per rank (-DSGMV_RANK=8, 16, 32, 64) and
once more for the rank dispatch and helper kernels; these objects and the
C ABI's compile in parallel, then link into one shared library.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
INCLUDE = ROOT / "include"
LIBRARY = PKG / "libsgmv.so"

KERNELS = CSRC / "sgmv_kernels.hip"
API = CSRC / "sgmv_api.cpp"
HOST = CSRC / "sgmv_host.cpp"  # host-only entry points (no HIP): also built alone with the sanitizers
SOURCES = [KERNELS, API, HOST]
RANKS = (8, 16, 32, 64)
ARCH = "gfx950"

# Packed fp32 instructions are disabled: hipcc would otherwise form them from
# ordinary float code. The host pass does not know the feature and says so.
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function"]
NOISE = "-packed-fp32-ops' is not a recognized feature"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and Path(cand).exists():
            return cand
    raise FileNotFoundError("hipcc not found (ROCm is required to build libsgmv.so)")


def _messages(res) -> list:
    return [ln for ln in (res.stdout + res.stderr).splitlines() if NOISE not in ln]


def build(output: Path = LIBRARY, extra_flags=(), verbose: bool = False, jobs: int = 0) -> Path:
    """Compile every HIP/C++ source into one shared library (always rebuilds)."""
    cc = hipcc()
    inc = [f"-I{INCLUDE}", f"-I{CSRC}"]
    jobs = jobs or min(8, os.cpu_count() or 1)
    with tempfile.TemporaryDirectory(prefix="sgmv_build_") as tmp:
        units = [(KERNELS, [f"-DSGMV_RANK={r}"], Path(tmp) / f"kernels_r{r}.o") for r in RANKS]
        units += [(KERNELS, [], Path(tmp) / "kernels_dispatch.o"), (API, [], Path(tmp) / "api.o"),
                  (HOST, [], Path(tmp) / "host.o")]
        pending = list(units)
        running = []
        failed = []
        while pending or running:
            while pending and len(running) < jobs:
                src, defs, obj = pending.pop(0)
                cmd = [cc, *FLAGS, *extra_flags, *defs, *inc, "-c", str(src), "-o", str(obj)]
                if verbose:
                    print(" ".join(cmd), flush=True)
                running.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE,
                                                      text=True)))
            cmd, proc = running.pop(0)
            out, err = proc.communicate()
            res = subprocess.CompletedProcess(cmd, proc.returncode, out, err)
            msgs = _messages(res)
            if proc.returncode != 0:
                failed.append(" ".join(cmd) + "\n" + "\n".join(msgs))
            elif verbose and msgs:
                print("\n".join(msgs))
        if failed:
            raise RuntimeError("hipcc failed:\n" + "\n\n".join(failed))
        tmp_out = output.with_suffix(".so.tmp")
        cmd = [cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *extra_flags,
               *[str(u[2]) for u in units], "-o", str(tmp_out)]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError("hipcc link failed:\n" + "\n".join(_messages(res)))
    os.replace(tmp_out, output)
    return output


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
