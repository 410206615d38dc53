"""Build step for the CPU oracle library (test infrastructure only).

Compiles ``pkv_oracle.c`` with gcc into ``liboracle.so`` beside it.  Plain
``-O2`` for the baseline x86-64 target (no ``-march=native``: the library is
built in one container and may run on another host), OpenMP for spreading
independent units over threads, and no fast-math so the fp64 arithmetic is
the plain IEEE one.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "pkv_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(force: bool = True) -> str:
    if not force and os.path.exists(LIB):
        return LIB
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
           "-shared", "-fPIC", "-Wall", "-Wextra", "-o", tmp, SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
