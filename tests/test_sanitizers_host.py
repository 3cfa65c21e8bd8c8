"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

- the coefficient backward's work partition (mhc_partition.hpp) through its checker,
  partition_check.cpp, over the same grid of shapes as test_partition_host.py;
- every function of the fp64 oracle (oracle/mhc_oracle.c) through oracle_sanitize.c,
  for n = 1, 2, 4, 8, with the optional outputs present and absent, on exactly-sized
  heap arrays.

Built with the host compiler (g++/gcc; no device code is involved), run with leak
detection on; any report aborts the program and fails the test."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "manifold_constrained_residuals_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="2")


def _run(cmd, exe):
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=ENV, timeout=600)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    return r.stdout


def test_partition_under_sanitizers(tmp_path):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("no g++")
    exe = tmp_path / "partition_check_san"
    out = _run([cxx, "-std=c++17", "-O1", *SAN, "-I", CSRC,
                os.path.join(HERE, "partition_check.cpp"), "-o", str(exe)], exe)
    assert "0 failures" in out


def test_oracle_under_sanitizers(tmp_path):
    cc = shutil.which("gcc")
    if cc is None:
        pytest.skip("no gcc")
    exe = tmp_path / "oracle_san"
    out = _run([cc, "-std=c99", "-O1", "-fopenmp", "-ffp-contract=off", *SAN,
                os.path.join(ROOT, "oracle", "mhc_oracle.c"), os.path.join(HERE, "oracle_sanitize.c"),
                "-o", str(exe), "-lm"], exe)
    assert "oracle sanitize run done" in out
