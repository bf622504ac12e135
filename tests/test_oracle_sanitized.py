"""The oracle's C code under AddressSanitizer and UndefinedBehaviorSanitizer.

oracle.c is rebuilt with gcc -fsanitize=address,undefined (host code only)
and the oracle's pins (tests/test_oracle_pins.py, test_oracle_profiling.py)
run against that build in a child process, with the sanitizer runtimes
preloaded and every report fatal.  An out-of-bounds access, use after free,
signed overflow or misaligned load anywhere in the oracle's paths fails the
test.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_pins_under_address_and_ub_sanitizers(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("sanitizer runtimes not installed")
    lib = str(tmp_path / "liboracle_sanitized.so")
    subprocess.check_call(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                           "-fno-sanitize-recover=undefined", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                           "-o", lib, os.path.join(ROOT, "oracle", "oracle.c"), "-lm"])
    env = dict(os.environ, LD_PRELOAD=f"{asan} {ubsan}", SAF_ORACLE_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="4")
    # the child really loads the sanitized build
    probe = subprocess.run([sys.executable, "-c", "import oracle; oracle.lib(); "
                            "print(sum('liboracle_sanitized' in l for l in open('/proc/self/maps')))"],
                           env=env, cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert probe.returncode == 0 and int(probe.stdout.split()[-1]) > 0, probe.stdout + probe.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "tests/test_oracle_pins.py", "tests/test_oracle_profiling.py"],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, (r.stdout[-4000:], r.stderr[-4000:])
    assert "passed" in r.stdout
