"""The oracle's pin suites against a build of oracle.c with AddressSanitizer
and UndefinedBehaviorSanitizer (host code only; CPU).  Any out-of-bounds
access, use after free or undefined operation in the oracle aborts the run.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SUITES = ["tests/test_oracle_pins.py", "tests/test_oracle_backward.py", "tests/test_oracle_capacity.py"]


def _asan_runtime():
    gcc = shutil.which("gcc")
    if not gcc:
        return None
    p = subprocess.run([gcc, "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return p if p and os.path.isabs(p) and os.path.exists(p) else None


def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    runtime = _asan_runtime()
    if runtime is None:
        pytest.skip("gcc with libasan not available")
    lib = str(tmp_path / "liboracle355_asan.so")
    build = ["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
             "-fno-fast-math", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
             "-fno-omit-frame-pointer", os.path.join(ROOT, "oracle", "oracle.c"), "-o", lib, "-lm"]
    subprocess.run(build, check=True, cwd=ROOT)
    env = dict(os.environ, MOE_ORACLE_LIB=lib, LD_PRELOAD=runtime,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-s", "-p", "no:cacheprovider", "-m", "not gpu",
                        *SUITES], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout, tail
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail
