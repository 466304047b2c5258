"""Builds the CPU oracle (test infrastructure) into oracle/liboracle.so with gcc."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c99", "-Wall", "-Wextra", "-ffp-contract=off", "-fPIC", "-shared",
           os.path.join(HERE, "oracle.c"), "-o", LIB + ".tmp", "-lm", "-lpthread"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
