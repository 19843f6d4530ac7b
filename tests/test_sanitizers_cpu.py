"""The oracle and the library's host code under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

- The C oracle is built with gcc and driven by tests/sanitize/oracle_drive.c:
  every function on seeded small inputs, guard bytes around every output,
  round trips and refusals.
- The library's host sources (argument checks, run-table validation and
  plan layout, the fetch planner, page lists, the streamed schedule and
  driver) are built with g++ against a mock of the HIP runtime API in which
  device memory is host memory (tests/sanitize/mock_hip), and driven by
  tests/sanitize/host_drive.cpp: valid and corrupted tables, injected
  runtime failures (event creation and recording, uploads), and a check that
  no event is leaked or destroyed twice.

Any sanitizer report aborts the program (-fno-sanitize-recover=all), so the
test is a plain exit-status check."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-Wall"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:allocator_may_return_null=1", UBSAN_OPTIONS="print_stacktrace=1")

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None,
                                reason="needs gcc and g++")


def _build_and_run(cmd, exe, what):
    r = subprocess.run(cmd, capture_output=True, text=True, cwd=ROOT)
    assert r.returncode == 0, f"building {what} failed:\n{r.stderr[-4000:]}"
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=240)
    assert r.returncode == 0, f"{what} under sanitizers failed (status {r.returncode}):\n{r.stdout[-2000:]}\n{r.stderr[-6000:]}"
    return r.stdout


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_drive")
    cmd = ["gcc", "-std=c11", *SAN, "-fno-fast-math", "-ffp-contract=off", "-I", "oracle", "oracle/oracle.c",
           "tests/sanitize/oracle_drive.c", "-o", exe]
    assert "all checks passed" in _build_and_run(cmd, exe, "the oracle")


def test_library_host_code_under_sanitizers(tmp_path):
    exe = str(tmp_path / "host_drive")
    csrc = "bf16_wire_all_amd/csrc"
    cmd = ["g++", "-std=c++17", *SAN, "-I", "tests/sanitize/mock_hip", "-I", "include", "-I", csrc, "-I",
           "tests/sanitize", f"{csrc}/api.cpp", f"{csrc}/groups.cpp", f"{csrc}/pages.cpp",
           f"{csrc}/stream_pipeline.cpp", "tests/sanitize/mock_hip.cpp", "tests/sanitize/host_drive.cpp", "-o", exe]
    assert "all checks passed" in _build_and_run(cmd, exe, "the library's host code")
