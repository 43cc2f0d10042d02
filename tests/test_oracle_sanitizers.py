"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer:
oracle/sanitize_driver.cpp (every exported oracle function on small shapes,
both storage modes, both lock policies and samplers, overrides, a sampled
step) is built with g++ together with oracle.cpp and must run clean."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_oracle_clean_under_asan_ubsan():
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, "oracle_sanitized")
        cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fopenmp",
               "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
               "-I", os.path.join(ROOT, "oracle"),
               os.path.join(ROOT, "oracle", "sanitize_driver.cpp"), "-o", exe]
        b = subprocess.run(cmd, capture_output=True, text=True)
        assert b.returncode == 0, b.stderr[-4000:]
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="2")
        r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
        assert r.returncode == 0 and "sanitized run ok" in r.stdout, \
            (r.returncode, r.stdout[-2000:], r.stderr[-6000:])
