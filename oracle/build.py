"""Builds the CPU oracle (test infrastructure) into oracle/liboracle.so with gcc.

With ORACLE_SANITIZE=1 in the environment (or sanitize=True) it builds
oracle/liboracle_san.so instead, instrumented with AddressSanitizer and
UndefinedBehaviorSanitizer, and the oracle package loads that one.  The
process must then preload the ASan runtime (the launcher test in
tests/test_sanitizers.py shows how)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")
LIB_SAN = os.path.join(HERE, "liboracle_san.so")
# host-only instrumentation of the gcc build (no GPU code is built here)
SANITIZE_FLAGS = ["-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


def sanitize_requested() -> bool:
    return os.environ.get("ORACLE_SANITIZE") == "1"


def build(verbose: bool = False, sanitize=None) -> str:
    san = sanitize_requested() if sanitize is None else sanitize
    out = LIB_SAN if san else LIB
    cmd = ["gcc", "-O1" if san else "-O2", "-std=c99", "-Wall", "-Wextra", "-ffp-contract=off", "-fPIC", "-shared",
           *(SANITIZE_FLAGS if san else []), os.path.join(HERE, "oracle.c"), "-o", out + ".tmp", "-lm", "-lpthread"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
