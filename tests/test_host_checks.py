"""Host-side argument checks of every entry point, built on their own with
the address and undefined-behaviour sanitizers (no GPU, no HIP runtime).

tests/host_checks.cpp holds the table of cases (null, misaligned and
out-of-range arguments, the largest accepted sizes, out-of-range enum values
as a C caller may pass them); this test compiles it with
kv_cache_reuse_hs2_amd/csrc/validate.cpp, the same checks that libhs2 runs
before its first enqueue, and requires every case to return its expected
status with no sanitizer report.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "kv_cache_reuse_hs2_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_checks_under_sanitizers(tmp_path):
    exe = str(tmp_path / "host_checks")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-Wall", "-Wextra",
           "-Werror", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
           os.path.join(CSRC, "validate.cpp"), os.path.join(ROOT, "tests", "host_checks.cpp"),
           "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    out = run.stdout + run.stderr
    assert run.returncode == 0, out
    assert "runtime error" not in out and "AddressSanitizer" not in out, out
    assert " 0 mismatches" in run.stdout, out
