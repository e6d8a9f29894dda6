"""Build the fp64 CPU oracle (test infrastructure) into oracle/liboracle.so.

Plain gcc, -O2, OpenMP over independent (sequence, head) recurrences, no
fast-math, so every operation is IEEE fp64 in the order the source states.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ssd_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(src: str = SRC, out: str = LIB, extra=()) -> str:
    cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
           "-fno-fast-math", "-ffp-contract=off", "-Wall", "-Werror",
           *extra, src, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


if __name__ == "__main__":
    print(build(*sys.argv[1:2]))
