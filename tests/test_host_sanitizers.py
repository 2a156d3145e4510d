"""The library's host code (planner, validators, block allocator) and the C oracle built
with AddressSanitizer and UndefinedBehaviorSanitizer (g++ / gcc, host only, no GPU) and
driven by the programs in tests/sanitize/: random batches, random allocator walks checked
against a model of the reference counts (the allocator's HIP event calls replaced by a
fake device whose work completes when the program says so), and the oracle on small
random batches.  Any sanitizer report aborts the program."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_attention_04_amd", "csrc")
SAN = ["-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _run(cmd, exe):
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    out = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert out.returncode == 0, out.stdout + out.stderr
    assert "ERROR: AddressSanitizer" not in out.stderr and "runtime error" not in out.stderr, out.stderr
    return out.stdout


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_planner_validators_allocator_under_sanitizers(tmp_path):
    exe = str(tmp_path / "host_checks")
    cmd = ["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-I", "/opt/rocm/include", "-o", exe, os.path.join(ROOT, "tests", "sanitize", "host_checks.cpp"),
           os.path.join(CSRC, "pa_host.cpp"), os.path.join(CSRC, "pa_alloc.cpp")]
    assert "host checks ok" in _run(cmd, exe)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_checks")
    cmd = ["gcc", "-std=c11", *SAN, "-o", exe, os.path.join(ROOT, "tests", "sanitize", "oracle_checks.c"),
           os.path.join(ROOT, "oracle", "pa_oracle.c"), "-lm"]
    assert "oracle checks ok" in _run(cmd, exe)
