"""Build the CPU oracle (test infrastructure only) with gcc.

Produces ``oracle/libbdoracle.so``.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg load it.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libbdoracle.so")


def build(force=True):
    if not force and os.path.exists(LIB):
        return LIB
    src = os.path.join(HERE, "bdoracle.c")
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def build_sanitized(out_dir, sanitizers=("address", "undefined")):
    """The oracle under the given sanitizers, built with the ROCm clang so
    that it shares one sanitizer runtime with the sanitized libbdattn (CPU
    sanitizer job; OpenMP off, so the runtime sees plain threads)."""
    os.makedirs(out_dir, exist_ok=True)
    clang = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm", "bin", "clang")
    out = os.path.join(out_dir, "libbdoracle.so")
    cmd = [clang, "-O1", "-g", "-std=c99", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-fsanitize=" + ",".join(sanitizers), "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           "-shared-libsan", "-o", out, os.path.join(HERE, "bdoracle.c"), "-lm"]
    subprocess.run(cmd, check=True)
    return out


if __name__ == "__main__":
    print(build())
