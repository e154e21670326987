"""Compile the fp64 CPU oracle (test infrastructure only) with gcc.

The oracle is the checker of the HIP library: only tests, the smoke check and
the benchmark's CPU-baseline leg load it.  Building it is part of the build
step so a fresh checkout can run the CPU tests.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "conv2d_oracle.c")
LIB = os.path.join(HERE, "liboracle_conv2d.so")


def build(force=False):
    """Compile conv2d_oracle.c into liboracle_conv2d.so next to it."""
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-std=c11",
           "-Wall", "-Wextra", "-fPIC", "-shared", SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(force=True))
