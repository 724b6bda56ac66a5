"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer: the C
oracle is rebuilt with -fsanitize=address,undefined and the oracle's pin
tests run against that build in a child process (the sanitizer runtime
preloaded, leak checks off: the Python interpreter itself is not
instrumented).  Any out-of-bounds access, use after free or undefined
operation in the oracle aborts the child and fails this test."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PIN_TESTS = ["tests/test_oracle.py", "tests/test_oracle_norm.py", "tests/test_oracle_mx4.py",
             "tests/test_oracle_backward.py"]


def runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(runtime("libasan.so") is None or runtime("libubsan.so") is None,
                    reason="gcc sanitizer runtimes not installed")
def test_oracle_pins_under_address_and_undefined_sanitizers(tmp_path):
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
                    "-fopenmp", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-shared", "-fPIC",
                    os.path.join(ROOT, "oracle", "moe_oracle.c"), "-o", lib, "-lm"], check=True)
    env = dict(os.environ, MOE_ORACLE_LIB=lib,
               LD_PRELOAD=f"{runtime('libasan.so')}:{runtime('libubsan.so')}",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, "-m", "pytest", *PIN_TESTS, "-x", "-q",
                        "-p", "no:cacheprovider", "-m", "not gpu"], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=900)
    report = r.stdout[-3000:] + r.stderr[-3000:]
    assert r.returncode == 0, report
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, report
    assert " passed" in r.stdout, report
