"""Host code under the compilers' sanitizers (CPU only).

Two seeded random drivers are built with AddressSanitizer and
UndefinedBehaviorSanitizer (and the oracle once more with ThreadSanitizer)
and must exit cleanly:

- tests/sanitize/plan_driver.cpp links the library's host-side planner and
  entry points (the same source file the library is built from) against stub
  kernel launchers, and drives it over valid and invalid descriptors, packed
  sequences with empty members, every context-parallel mode, aliasing,
  misalignment and short workspaces;
- tests/sanitize/oracle_driver.c drives the fp64 oracle over small dense and
  packed problems with exactly-sized buffers, checks that outputs are finite,
  that the thread count changes no bit, and that bad arguments are refused.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gated_deltanet_chunked_chunk_amd", "csrc")
SAN = ["-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1:verify_asan_link_order=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", TSAN_OPTIONS="halt_on_error=1")


def _build(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, "build failed:\n" + r.stderr[-4000:]


def _run(exe, *args):
    r = subprocess.run([exe, *args], capture_output=True, text=True, env=ENV, timeout=300)
    print(r.stdout)
    assert r.returncode == 0, f"{os.path.basename(exe)} exited {r.returncode}:\n{r.stdout[-2000:]}\n{r.stderr[-6000:]}"
    assert "0 failed checks" in r.stdout


@pytest.mark.skipif(shutil.which("g++") is None, reason="no host C++ compiler")
def test_planner_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "plan_driver")
    _build(["g++", "-std=c++17", *SAN, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
            os.path.join(CSRC, "gdn_plan.cpp"), os.path.join(ROOT, "tests", "sanitize", "plan_driver.cpp"),
            "-o", exe])
    _run(exe, "3000")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no host C compiler")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _build(["gcc", "-std=c11", *SAN, os.path.join(ROOT, "oracle", "gdn_oracle.c"),
            os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"), "-lm", "-lpthread", "-o", exe])
    _run(exe, "300")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no host C compiler")
def test_oracle_threads_under_tsan(tmp_path):
    exe = str(tmp_path / "oracle_driver_tsan")
    _build(["gcc", "-std=c11", "-g", "-O1", "-fsanitize=thread", os.path.join(ROOT, "oracle", "gdn_oracle.c"),
            os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"), "-lm", "-lpthread", "-o", exe])
    _run(exe, "100")
