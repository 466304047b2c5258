"""The CPU oracle and the CPU input generator under AddressSanitizer and
UndefinedBehaviorSanitizer: their pins and tests run again in a child
process that loads the instrumented gcc builds (ORACLE_SANITIZE=1) with the
ASan runtime preloaded.  Any out-of-bounds access, use after free or
undefined behaviour in the C code aborts the child, and the test fails."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    r = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.timeout(600)
def test_oracle_and_generator_under_sanitizers():
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc's ASan runtime is not installed")
    env = dict(os.environ, ORACLE_SANITIZE="1", LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    env.pop("ORACLE_LIB", None)
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
           os.path.join(ROOT, "tests", "test_oracle_pins.py"), os.path.join(ROOT, "tests", "test_synth.py")]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=580)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout, tail
