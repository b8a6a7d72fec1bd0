"""Host planning/validation code under g++ with AddressSanitizer and UBSan (CPU only)."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_attention_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_host_logic_under_asan():
    with tempfile.TemporaryDirectory() as td:
        exe = os.path.join(td, "host_test")
        cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
               "-I", CSRC, "-I", os.path.join(ROOT, "include"),
               os.path.join(ROOT, "tests", "host", "test_host_logic.cpp"), os.path.join(CSRC, "host_logic.cpp"),
               "-o", exe]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="halt_on_error=1")
        r = subprocess.run([exe], capture_output=True, text=True, env=env)
        assert r.returncode == 0, r.stdout + r.stderr
        assert "all checks passed" in r.stdout
