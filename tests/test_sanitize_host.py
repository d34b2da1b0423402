"""The library's host C++ (codebook tables, encoders, entropy coder) built
with AddressSanitizer and UndefinedBehaviorSanitizer together with a small
driver (tests/sanitize/host_check.cpp) that runs every CPU entry point on
small layers, their error paths included; any sanitizer report fails."""
import os
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "dequant_e8_codebook_amd", "csrc")
SOURCES = [os.path.join(CSRC, f) for f in ("glq_codebook.cpp", "glq_encode.cpp", "glq_ep.cpp")]
DRIVER = os.path.join(ROOT, "tests", "sanitize", "host_check.cpp")


def test_host_code_under_asan_and_ubsan():
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "host_check")
        cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-pthread",
               "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
               "-I" + os.path.join(ROOT, "include"), "-I" + CSRC, DRIVER] + SOURCES + ["-o", exe]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0 and "sanitizer" in (r.stderr or "").lower() and "cannot find" in r.stderr:
            pytest.skip("sanitizer runtime not installed")
        assert r.returncode == 0, r.stderr[-4000:]
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
        run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
        assert run.returncode == 0 and "host_check ok" in run.stdout, (run.stdout + run.stderr)[-4000:]
        assert "runtime error" not in run.stderr and "AddressSanitizer" not in run.stderr, run.stderr[-4000:]
