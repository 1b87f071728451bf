"""Build the fp64 CPU oracle (test infrastructure only) with gcc.

The oracle is plain C99; it is compiled -O2 without fast-math so that every
floating-point operation is the IEEE one written in the source.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "moe_oracle.c")
LIB = os.path.join(HERE, "libmoe_oracle.so")


def build(force: bool = True) -> str:
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-std=c99", "-O2", "-fopenmp", "-fPIC", "-shared",
           "-D_DEFAULT_SOURCE", "-Wall", "-Wextra", "-o", tmp, SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
