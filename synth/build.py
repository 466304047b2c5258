"""Builds the seeded input generators: libsynth.so (gcc, CPU) and
libsynth_gpu.so (hipcc, gfx950)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_CPU = os.path.join(HERE, "libsynth.so")
LIB_GPU = os.path.join(HERE, "libsynth_gpu.so")
LIB_CPU_SAN = os.path.join(HERE, "libsynth_san.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# host-only instrumentation of the gcc build (ORACLE_SANITIZE=1): the CPU
# generator next to the sanitized oracle; the GPU generator is never built so
SANITIZE_FLAGS = ["-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


def sanitize_requested():
    return os.environ.get("ORACLE_SANITIZE") == "1"


def build_cpu(verbose=False, sanitize=None):
    san = sanitize_requested() if sanitize is None else sanitize
    out = LIB_CPU_SAN if san else LIB_CPU
    cmd = ["gcc", "-O1" if san else "-O2", "-std=c99", "-Wall", "-Wextra", "-fPIC", "-shared",
           *(SANITIZE_FLAGS if san else []), os.path.join(HERE, "synth.c"), "-o", out + ".tmp", "-lm", "-lpthread"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def build_gpu(verbose=False):
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-fPIC", "-shared", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           os.path.join(HERE, "synth_gpu.hip"), "-o", LIB_GPU + ".tmp"]
    if verbose:
        print(" ".join(cmd))
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + r.stderr)
    os.replace(LIB_GPU + ".tmp", LIB_GPU)
    return LIB_GPU


def build(verbose=False):
    return build_cpu(verbose), build_gpu(verbose)


if __name__ == "__main__":
    print(build(verbose=True))
