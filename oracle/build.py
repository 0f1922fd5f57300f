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


if __name__ == "__main__":
    print(build())
