"""Host code under the sanitizers (CPU only).

* The oracle (oracle/sgmv_oracle.c) and the library's host-only entry points
  (segmented_gather_gemm_sgmv_amd/csrc/sgmv_host.cpp: size queries, segment
  building and checking, pool tables) are built with AddressSanitizer and
  UndefinedBehaviorSanitizer into tests/host_sanitize_driver.cpp, which runs
  them on exactly sized buffers with valid, invalid and extreme inputs and
  checks their results; any sanitizer report fails the run.
* The oracle built with UndefinedBehaviorSanitizer (which, unlike
  AddressSanitizer, can be loaded into a running interpreter) serves the
  oracle pin and mutant suites in a child pytest process.
"""
import os
import shutil
import subprocess
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent
CSRC = ROOT / "segmented_gather_gemm_sgmv_amd" / "csrc"
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _need(tool):
    if shutil.which(tool) is None:
        pytest.skip(f"{tool} not found")


def test_oracle_and_host_helpers_under_asan_ubsan(tmp_path):
    _need("g++")
    _need("gcc")
    oracle_o = tmp_path / "oracle.o"
    subprocess.run(["gcc", "-std=c11", "-O1", "-g", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", *SAN,
                    "-c", str(ROOT / "oracle" / "sgmv_oracle.c"), "-o", str(oracle_o)], check=True)
    exe = tmp_path / "host_driver"
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fopenmp", *SAN, f"-I{ROOT / 'include'}", f"-I{CSRC}",
                    str(ROOT / "tests" / "host_sanitize_driver.cpp"), str(CSRC / "sgmv_host.cpp"), str(oracle_o),
                    "-o", str(exe), "-lm"], check=True)
    env = dict(os.environ, OMP_NUM_THREADS="1",
               ASAN_OPTIONS="halt_on_error=1:detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=600)
    assert res.returncode == 0, res.stdout[-4000:] + res.stderr[-4000:]
    assert "all checks passed" in res.stdout
    assert "runtime error" not in res.stderr and "Sanitizer" not in res.stderr, res.stderr[-4000:]


def test_oracle_pins_under_ubsan(tmp_path):
    _need("gcc")
    lib = tmp_path / "liboracle_ubsan.so"
    subprocess.run(["gcc", "-std=c11", "-O1", "-g", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
                    "-fsanitize=undefined", "-fno-sanitize-recover=all", "-fPIC", "-shared",
                    str(ROOT / "oracle" / "sgmv_oracle.c"), "-o", str(lib), "-lm"], check=True)
    env = dict(os.environ, SGMV_ORACLE_LIBRARY=str(lib), UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                          str(ROOT / "tests" / "test_oracle_pins.py"), str(ROOT / "tests" / "test_oracle_mutants.py"),
                          "-m", "not gpu"], capture_output=True, text=True, env=env, cwd=ROOT, timeout=900)
    assert res.returncode == 0, res.stdout[-4000:] + res.stderr[-4000:]
    assert "runtime error" not in res.stdout + res.stderr
