"""Build libsgmv.so (the C-ABI library) in-tree with hipcc for gfx950.

Usage: ``python -m segmented_gather_gemm_sgmv_amd.build``.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
INCLUDE = ROOT / "include"
LIBRARY = PKG / "libsgmv.so"

SOURCES = [CSRC / "sgmv_kernels.hip", CSRC / "sgmv_api.cpp"]
ARCH = "gfx950"

# Packed fp32 instructions are disabled: hipcc would otherwise form them from
# ordinary float code. The host pass does not know the feature and says so.
FLAGS = ["-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and Path(cand).exists():
            return cand
    raise FileNotFoundError("hipcc not found (ROCm is required to build libsgmv.so)")


def build(output: Path = LIBRARY, extra_flags=(), verbose: bool = False) -> Path:
    """Compile every HIP/C++ source into one shared library (always rebuilds)."""
    tmp = output.with_suffix(".so.tmp")
    cmd = [hipcc(), *FLAGS, *extra_flags, f"-I{INCLUDE}", f"-I{CSRC}",
           *map(str, SOURCES), "-o", str(tmp)]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "-packed-fp32-ops' is not a recognized feature"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, output)
    return output


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
